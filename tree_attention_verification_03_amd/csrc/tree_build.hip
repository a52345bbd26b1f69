// EAGLE-2 draft-tree construction: top-k expansion per step, rerank to N nodes.
//
// SGLang "Speculative Decoding" page, sections "EAGLE Decoding" (num_steps,
// eagle_topk, num_draft_tokens) and "References" (tree-style extension with
// topk branches per step; unlikely branches stop; rerank keeps the top
// num_draft_tokens); lesty.tech "EAGLE-2 & Lookahead Decoding", section 4
// "Dynamic Tree Construction Mechanics" (confidence = product of conditional
// probabilities, kept as an fp64 sum of log-probs).
//
// Kernels:
//   build_step_kernel    one launch per step; block (slice, frontier slot f,
//                        sequence) takes the top-k of a slice of row f and
//                        publishes it; the last block of the sequence's step
//                        (atomic ticket) merges every row's slices in LDS; step 1
//                        seeds the pool and frontier from the root row; at step
//                        d >= 2 the k rows' children join the pool, the k*k
//                        children are ranked and the next frontier is written.
//   build_finish_kernel  one block per sequence: rank the whole pool, keep the
//                        N best, number them in pool order, emit parents /
//                        depth / ancestry words / q_row.
// Ranking keys are exact: vocabulary top-k uses the 64-bit key
// (order(logprob) << 32) | (2^32 - 1 - token); pool ranking compares fp64
// scores, ties broken by the smaller pool index.
#include <cstdlib>

#include "api_common.h"
#include "spec_common.h"

namespace spectree {
namespace {

constexpr int kMaxTopk = 8;
constexpr int kMaxDepth = 16;
constexpr int kRowThreads = 256;
constexpr int kCandPerLane = 4;
constexpr int kCand = kCandPerLane * kWave;  // candidates per draft row (n_slices * k), four per lane of the merging wave
constexpr int kMaxEpl = 16;                  // row elements per thread and load batch: 8 or 16
constexpr int kMaxBatches = 2;               // load batches per slice the block-count target may ask for
constexpr int kFinishThreads = 256;
constexpr int kTicketStride = 32;  // uint32: each sequence's ticket on its own 128-byte line

struct BuildWs {
  int32_t* tok;    // [B, P]
  int32_t* par;    // [B, P] parent pool index, -1 = root
  int32_t* depth;  // [B, P]
  int32_t* fslot;  // [B, P] frontier slot held at its own step, -1 if never frontier
  double* score;   // [B, P]
  int32_t* frontier;  // [B, max_topk] pool indices, rank order
  double* fscore;     // [B, max_topk] their scores
  uint32_t* ticket;   // [B * kTicketStride] blocks of the sequence's step that have finished (own 128-byte lines)
  uint64_t* cand;     // [B, max_topk, kCand] per-slice top-k keys, slice x at x * k
};

size_t pool_cap(int max_topk, int max_depth) {
  return size_t(max_topk) + size_t(max_depth - 1) * max_topk * max_topk;
}

// The pool, frontier and candidates, which carry a build from step to step, sit at the start of the
// workspace; the tickets, the only part that must start at zero, sit at the end of its ws_bytes. A workspace
// zero-filled once therefore serves builds of several shapes without clearing: no build's pool lands on
// another shape's tickets as long as ws_bytes covers the largest pool plus the largest tickets. With ws null
// (or ws_bytes below *total) only *total is meaningful.
BuildWs carve(void* ws, size_t ws_bytes, int B, int max_topk, int max_depth, size_t* total) {
  const size_t P = pool_cap(max_topk, max_depth);
  char* c = static_cast<char*>(ws);
  size_t off = 0;
  BuildWs w;
  auto take = [&](size_t bytes) {
    char* r = c ? c + off : nullptr;
    off = align_up(off + bytes, 256);
    return r;
  };
  w.score = reinterpret_cast<double*>(take(sizeof(double) * B * P));
  w.tok = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * B * P));
  w.par = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * B * P));
  w.depth = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * B * P));
  w.fslot = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * B * P));
  w.frontier = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * B * max_topk));
  w.fscore = reinterpret_cast<double*>(take(sizeof(double) * B * max_topk));
  w.cand = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * B * max_topk * kCand));
  const size_t tickets = align_up(sizeof(uint32_t) * B * kTicketStride, 256);
  *total = off + tickets;
  w.ticket = c && ws_bytes >= *total ? reinterpret_cast<uint32_t*>(c + ((ws_bytes - tickets) & ~size_t(255))) : nullptr;
  return w;
}

__device__ __forceinline__ int clamp_i(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// canonical log-prob -> 64-bit ranking key (value desc, token asc)
__device__ __forceinline__ uint64_t lp_key(float x, int token) {
  if (x != x) x = -INFINITY;  // NaN ranks as -inf
  if (x >= 0.f) x = 0.f;      // log-probs are <= 0; also maps -0 to +0
  return (uint64_t(f32_order_key(x)) << 32) | uint64_t(0xffffffffu - uint32_t(token));
}

__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t o = uint32_t(key >> 32);
  const uint32_t bits = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(bits);
}

__device__ __forceinline__ int key_token(uint64_t key) { return int(0xffffffffu - uint32_t(key)); }

// A draft-row index as a token: through the token map of a truncated draft vocabulary (entry i of a
// row stands for token map[i]), or the index itself without a map.
__device__ __forceinline__ int map_token(const int32_t* map, int idx) { return (map && idx >= 0) ? map[idx] : idx; }

// Element j of a thread in the batch that starts at `base`: VEC -> base + 4 * tid + 4 * kRowThreads *
// (j / 4) + j % 4, scalar -> base + tid + kRowThreads * j (both visit a thread's tokens in increasing
// order).
template <bool VEC>
__device__ __forceinline__ int batch_token(int base, int j) {
  return VEC ? base + 4 * int(threadIdx.x) + 4 * kRowThreads * (j >> 2) + (j & 3)
             : base + int(threadIdx.x) + kRowThreads * j;
}

// Loads one batch of EPL elements per thread without branches: addresses past `hi` are clamped into
// the slice (those elements are masked out later), so every load of the batch is in flight at once.
template <bool VEC, int EPL>
__device__ __forceinline__ void load_batch(const float* row, int base, int hi, float* xs) {
  if (VEC) {
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i) {
      const int v = min(batch_token<VEC>(base, 4 * i), hi - 4);
      const float4 q = *reinterpret_cast<const float4*>(row + v);
      xs[4 * i] = q.x;
      xs[4 * i + 1] = q.y;
      xs[4 * i + 2] = q.z;
      xs[4 * i + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) xs[j] = row[min(batch_token<VEC>(base, j), hi - 1)];
  }
}

// Top-2 lists (t0 > t1, 0 = none) merged: the larger head, then the larger of the winner's second
// and the loser's head.
__device__ __forceinline__ void top2_merge(uint64_t a0, uint64_t a1, uint64_t b0, uint64_t b1, uint64_t& t0,
                                           uint64_t& t1) {
  const bool c = a0 > b0;
  const uint64_t x = c ? a1 : b1, y = c ? b0 : a0;
  t0 = c ? a0 : b0;
  t1 = x > y ? x : y;
}

// Two largest keys of this thread's elements of one batch (those below `below` if BOUNDED), folded
// into the sorted cache c[0..2): groups of 8 elements reduce by a balanced tree of merges (independent
// compare chains) and fold into the cache one group at a time, which bounds the live registers.
template <bool VEC, int EPL, bool BOUNDED>
__device__ __forceinline__ void lane_top2(const float* xs, int base, int hi, uint64_t below, uint64_t* c) {
  constexpr int G = 8;
  const bool full = base + EPL * kRowThreads <= hi;
#pragma unroll
  for (int g0 = 0; g0 < EPL; g0 += G) {
    uint64_t t0[G / 2], t1[G / 2];
#pragma unroll
    for (int i = 0; i < G / 2; ++i) {
      uint64_t k2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = g0 + 2 * i + h, v = batch_token<VEC>(base, j);
        uint64_t key = (full || v < hi) ? lp_key(xs[j], v) : 0ull;
        if (BOUNDED) key = key < below ? key : 0ull;
        k2[h] = key;
      }
      const bool g = k2[0] > k2[1];
      t0[i] = g ? k2[0] : k2[1];
      t1[i] = g ? k2[1] : k2[0];
    }
#pragma unroll
    for (int w = 1; w < G / 2; w *= 2) {
#pragma unroll
      for (int i = 0; i + w < G / 2; i += 2 * w) top2_merge(t0[i], t1[i], t0[i + w], t1[i + w], t0[i], t1[i]);
    }
    top2_merge(c[0], c[1], t0[0], t1[0], c[0], c[1]);
  }
}

// Compare-exchange of two keys: a holds the larger afterwards.
__device__ __forceinline__ void cas_key(uint64_t& a, uint64_t& b) {
  const bool sw = b > a;
  const uint64_t hi = sw ? b : a;
  b = sw ? a : b;
  a = hi;
}

// The four largest of two descending 4-lists, descending, into a: max(a[i], b[3 - i]) are the four
// largest of the union and form a bitonic sequence, which two rounds of compare-exchange sort.
__device__ __forceinline__ void top4_merge(uint64_t* a, const uint64_t* b) {
  uint64_t m[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) m[i] = a[i] > b[3 - i] ? a[i] : b[3 - i];
  cas_key(m[0], m[2]);
  cas_key(m[1], m[3]);
  cas_key(m[0], m[1]);
  cas_key(m[2], m[3]);
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = m[i];
}

// Two descending pairs merged into one descending 4-list (odd-even merge: heads, tails, then the
// middle two).
__device__ __forceinline__ void pair_merge(uint64_t a0, uint64_t a1, uint64_t b0, uint64_t b1, uint64_t* out) {
  cas_key(a0, b0);
  cas_key(a1, b1);
  cas_key(b0, a1);
  out[0] = a0;
  out[1] = b0;
  out[2] = a1;
  out[3] = b1;
}

// Four largest keys of this thread's elements of one batch (those below `below` if BOUNDED), folded
// into the descending cache c[0..4) (0 = none): each group of 8 elements is sorted down to its top
// four by a fixed network (pairs, two pair merges, one 4-list merge; independent compare chains) and
// merged into the cache one group at a time, which bounds the live registers.
template <bool VEC, int EPL, bool BOUNDED>
__device__ __forceinline__ void lane_top4(const float* xs, int base, int hi, uint64_t below, uint64_t* c) {
  constexpr int G = 8;
  const bool full = base + EPL * kRowThreads <= hi;
#pragma unroll
  for (int g0 = 0; g0 < EPL; g0 += G) {
    uint64_t k[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int v = batch_token<VEC>(base, g0 + j);
      uint64_t key = (full || v < hi) ? lp_key(xs[g0 + j], v) : 0ull;
      if (BOUNDED) key = key < below ? key : 0ull;
      k[j] = key;
    }
#pragma unroll
    for (int j = 0; j < G; j += 2) cas_key(k[j], k[j + 1]);
    uint64_t q0[4], q1[4];
    pair_merge(k[0], k[1], k[2], k[3], q0);
    pair_merge(k[4], k[5], k[6], k[7], q1);
    top4_merge(q0, q1);
    top4_merge(c, q0);
  }
}

// The NC (2 or 4) largest keys of this thread's elements of one batch into the descending cache c.
template <int NC, bool VEC, int EPL, bool BOUNDED>
__device__ __forceinline__ void lane_top(const float* xs, int base, int hi, uint64_t below, uint64_t* c) {
  if constexpr (NC == 4)
    lane_top4<VEC, EPL, BOUNDED>(xs, base, hi, below, c);
  else
    lane_top2<VEC, EPL, BOUNDED>(xs, base, hi, below, c);
}

// ------------------------------------------------------------------ wave-wide selection
// Wave maximum of a u32, uniform: DPP steps within each 16-lane row (fused into the max), the row
// broadcasts carry rows 0-1 into 1 and 2-3 into 3, then 0-1 into 2-3, so lane 63 holds the maximum.
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_max_rows(uint32_t v) {
  return max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROWS, 0xf, false)));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_rows<dpp::kXor1, 0xf>(v);
  v = dpp_max_rows<dpp::kXor2, 0xf>(v);
  v = dpp_max_rows<dpp::kHalfMirror, 0xf>(v);
  v = dpp_max_rows<dpp::kMirror, 0xf>(v);
  v = dpp_max_rows<kRowBcast15, 0xa>(v);
  v = dpp_max_rows<kRowBcast31, 0xc>(v);
  return __builtin_amdgcn_readlane(v, 63);
}

struct Popped {
  uint64_t key;  // the wave's largest head key (0 = none left)
  int lane;      // the lowest lane holding it
};

// Takes the largest of the lanes' heads c[0] (every lane of the wave active; caches sorted, 0 =
// none): the high words are reduced first, the low words only if several lanes share the largest
// high word; the lowest lane holding the maximum gives it up (shifts its cache), so equal keys
// leave in lane order.
template <int N>
__device__ __forceinline__ Popped wave_pop(uint64_t* c) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t hi = uint32_t(c[0] >> 32), lo = uint32_t(c[0]);
  const uint32_t mh = wave_max_u32(hi);
  const uint64_t tied = __ballot(hi == mh);
  uint32_t ml;
  if (__popcll(tied) == 1)
    ml = __builtin_amdgcn_readlane(lo, __ffsll(static_cast<unsigned long long>(tied)) - 1);
  else
    ml = wave_max_u32(hi == mh ? lo : 0u);
  Popped p;
  p.key = (uint64_t(mh) << 32) | ml;
  p.lane = __ffsll(static_cast<unsigned long long>(__ballot(c[0] == p.key))) - 1;
  if (lane == p.lane && p.key != 0) {
#pragma unroll
    for (int i = 0; i + 1 < N; ++i) c[i] = c[i + 1];
    c[N - 1] = 0;
  }
  return p;
}

// Block-wide top-k (k <= 8) of row[lo, hi) in rank order (0 = none) in out_key[0..k); with per_wave
// each wave's own top k are returned instead (lane r holds the wave's r-th key) and out_key is unused.
// xs holds the first batch (load_batch(row, lo, hi, xs)). Every lane keeps the NC largest keys of
// its own elements; each wave pops its k largest (a lane that gives up all NC refills them with its
// largest keys below the last one taken, so the pops are exact), and wave 0 pops the k best of the
// waves' lists. NC is 4 with 16 elements per thread and batch: a lane holds two of a wave's first seven
// picks about once in four waves (a birthday collision over 64 lanes), four of them about once in ten
// thousand, and every refill re-reads the slice batch after batch. With 8 elements per thread (short
// rows, one batch) the cheaper two-key lane pass wins. xs is consumed (free after the lane pass).
template <bool VEC, int EPL>
__device__ __forceinline__ uint64_t block_slice_topk(const float* row, int lo, int hi, int k, bool per_wave,
                                                     float* xs, uint64_t* out_key) {
  constexpr int NWV = kRowThreads / kWave;
  constexpr int kBatch = EPL * kRowThreads;
  __shared__ uint64_t wk[NWV * kMaxTopk];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  constexpr int NC = EPL >= 16 ? 4 : 2;
  uint64_t c[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) c[i] = 0;
  for (int base = lo; base < hi; base += kBatch) {
    float nxt[EPL];  // the next batch's loads are in flight while this one is reduced
    const bool more = base + kBatch < hi;
    if (more) load_batch<VEC, EPL>(row, base + kBatch, hi, nxt);
    lane_top<NC, VEC, EPL, false>(xs, base, hi, 0, c);
    if (more) {
#pragma unroll
      for (int j = 0; j < EPL; ++j) xs[j] = nxt[j];
    }
  }
  uint64_t mine = 0;
  for (int r = 0; r < k; ++r) {
    const Popped p = wave_pop<NC>(c);
    if (lane == r) mine = p.key;
    if (lane == p.lane && p.key != 0 && c[0] == 0 && r + 1 < k) {
      // this lane gave all its cached keys: refill with its NC largest below the one just taken
      // (re-read from memory, so the batch's registers are free during the pops)
      for (int base = lo; base < hi; base += kBatch) {
        float ys[EPL];
        load_batch<VEC, EPL>(row, base, hi, ys);
        lane_top<NC, VEC, EPL, true>(ys, base, hi, p.key, c);
      }
    }
  }
  if (per_wave) return mine;  // every wave publishes its own list (lane r: its r-th key)
  if (lane < k) wk[wave * k + lane] = mine;
  __syncthreads();
  if (wave == 0) {
    uint64_t v = lane < NWV * k ? wk[lane] : 0ull, best = 0;
    for (int r = 0; r < k; ++r) {
      const Popped p = wave_pop<1>(&v);
      if (lane == r) best = p.key;
    }
    if (lane < k) out_key[lane] = best;
  }
  __syncthreads();
  return 0;
}

// Finish, selection (wave 0): the N best pool entries by (score desc, pool index asc). Entry e sits
// in lane e % 64, slot e / 64 (PL slots per lane). A bitwise search on ballot counts finds the N-th
// largest score key t (high words, then low words where the high word ties); the kept entries are
// those above t and, in pool order, the first N - #(above t) equal to t. pool_of[1..N] receives them
// in pool order, node_of[e] their node numbers.
template <int PL>
__device__ __forceinline__ void finish_select(const double* sc, int pool, int N, int* pool_of, int* node_of) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t below = (1ull << lane) - 1;
  uint64_t key[PL];
  uint32_t hi[PL];
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const int e = lane + kWave * j;
    key[j] = e < pool ? f64_order_key(sc[e] + 0.0) : 0ull;  // scores: no NaN; +0.0 folds -0 into +0
    hi[j] = uint32_t(key[j] >> 32);
  }
  auto count = [&](auto pred) {
    int n = 0;
#pragma unroll
    for (int j = 0; j < PL; ++j) n += __popcll(__ballot(pred(j)));
    return n;
  };
  uint32_t th = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = th | (1u << bit);
    if (count([&](int j) { return hi[j] >= cand; }) >= N) th = cand;
  }
  uint64_t t = uint64_t(th) << 32;
  const int g_hi = count([&](int j) { return hi[j] > th; });
  const int e_hi = count([&](int j) { return hi[j] == th; });
  if (g_hi + e_hi > N) {  // the boundary falls inside one high word: search its low words
    uint32_t tl = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tl | (1u << bit);
      if (count([&](int j) { return hi[j] == th && uint32_t(key[j]) >= cand; }) >= N - g_hi) tl = cand;
    }
    t |= tl;
  }
  const int need = N - count([&](int j) { return key[j] > t; });
  int base = 0, eq_seen = 0;
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const bool eq = key[j] == t && key[j] != 0;
    const uint64_t me = __ballot(eq);
    const bool kept = key[j] > t || (eq && eq_seen + __popcll(me & below) < need);
    const uint64_t mk = __ballot(kept);
    if (kept) {
      const int n = 1 + base + __popcll(mk & below), e = lane + kWave * j;
      pool_of[n] = e;
      node_of[e] = n;
    }
    base += __popcll(mk);
    eq_seen += __popcll(me);
  }
}

// Outputs of the finish (the caller's arrays, [B, max_T]).
struct FinishArgs {
  const int32_t* root_tokens;
  const int32_t* num_draft;
  int max_T;
  int32_t* tokens;
  int32_t* parents;
  int32_t* depth_out;
  uint64_t* anc_mask;
  int32_t* q_row;
};

// Finish of sequence b by one block of kFinishThreads: keep the N best pool entries, number them
// 1..N in pool order and emit parents (node numbers), depth, ancestry words and q_row. Wave 0 does
// everything after the loads: the kept set is closed under parents (scores never increase down a path
// and a parent has the smaller pool index), and node n's ancestry is found by pointer doubling over
// lanes (node n in lane n - 1; depth <= 16, so four rounds). COHERENT loads read the pool at device
// scope (entries this kernel wrote).
template <bool COHERENT>
__device__ __forceinline__ void finish_sequence(const BuildWs& w, int P, int b, int k, int D, int max_topk,
                                                const FinishArgs& fa) {
  constexpr int kPool = kMaxTopk + (kMaxDepth - 1) * kMaxTopk * kMaxTopk;
  static_assert(kPool <= 16 * kWave, "pool fits 16 slots per lane");
  __shared__ double sc[kPool];
  __shared__ int par_e[kPool], dep_e[kPool], fs_e[kPool], tok_e[kPool], node_of[kPool];
  __shared__ int pool_of[kWave + 1];
  const int tid = threadIdx.x;
  const int max_T = fa.max_T;
  const int pool = k + (D - 1) * k * k;
  const int N = clamp_i(fa.num_draft[b], 1, min(pool, max_T - 1));
  const int T = N + 1;
  const size_t row = size_t(b) * P;
  auto ld = [](const auto* q) { return COHERENT ? ld_agent(q) : *q; };
  // one round trip: every field of the pool
  for (int e = tid; e < pool; e += kFinishThreads) {
    sc[e] = ld(w.score + row + e);
    par_e[e] = ld(w.par + row + e);
    dep_e[e] = ld(w.depth + row + e);
    fs_e[e] = ld(w.fslot + row + e);
    tok_e[e] = ld(w.tok + row + e);
  }
  __syncthreads();
  if (tid >= kWave) return;
  const int lane = tid;
  if (pool <= kWave) finish_select<1>(sc, pool, N, pool_of, node_of);
  else if (pool <= 2 * kWave) finish_select<2>(sc, pool, N, pool_of, node_of);
  else if (pool <= 4 * kWave) finish_select<4>(sc, pool, N, pool_of, node_of);
  else if (pool <= 8 * kWave) finish_select<8>(sc, pool, N, pool_of, node_of);
  else finish_select<16>(sc, pool, N, pool_of, node_of);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // node n = lane + 1 (n <= N): its entry, parent node (0 = root) and ancestry by pointer doubling
  const int n = lane + 1;
  const bool real = n <= N;
  const int e = real ? pool_of[n] : 0;
  int par_node = 0;
  if (real) {
    const int pe = par_e[e];
    par_node = pe >= 0 ? node_of[pe] : 0;
  }
  uint64_t anc = real ? (1ull << lane) : 0ull;
  int jump = par_node;  // 0 = reached the root
  while (__ballot(jump != 0)) {
    const int src = jump > 0 ? jump - 1 : lane;
    const uint64_t pa = (uint64_t(uint32_t(__shfl(int(anc >> 32), src))) << 32) | uint32_t(__shfl(int(anc), src));
    const int pj = __shfl(jump, src);
    if (jump != 0) {
      anc |= pa;
      jump = pj;
    }
  }
  const size_t o = size_t(b) * max_T;
  if (lane == 0) {  // the root
    fa.tokens[o] = fa.root_tokens[b];
    fa.parents[o] = -1;
    fa.depth_out[o] = 0;
    fa.anc_mask[o] = 0;
    fa.q_row[o] = 0;
  }
  if (n < max_T) {  // output row n: node n if n <= N, else padding
    const int d = real ? dep_e[e] : 0;
    const int fs = real ? fs_e[e] : -1;
    fa.tokens[o + n] = real ? tok_e[e] : -1;
    fa.parents[o + n] = real ? par_node : -1;
    fa.depth_out[o + n] = d;
    fa.anc_mask[o + n] = anc;
    fa.q_row[o + n] = (real && fs >= 0 && d < D) ? 1 + (d - 1) * max_topk + fs : -1;
  }
}

// Step >= 2, wave 0 of the merging block (one child per lane): row r's c-th best token becomes pool
// entry base + r * k + c; the next frontier is the k best by score (ties -> smaller pool index): k
// pops of their scores' order keys, where the lowest lane wins ties.
__device__ __forceinline__ void step_children(const BuildWs& w, int P, int b, int step, int k, int base,
                                              int max_topk, const uint64_t* top, const double* fsc_s,
                                              const int* cpar, const int32_t* token_map, int32_t* frontier_tokens) {
  const int lane = threadIdx.x & (kWave - 1);
  {
    const int n = k * k;
    const int r = lane / k, c = lane - r * k;
    double sc = 0.0;
    uint64_t key = 0, sk = 0;
    int tok = -1;
    if (lane < n) {
      key = top[r * kMaxTopk + c];
      tok = map_token(token_map, key_token(key));
      sc = fsc_s[r] + double(key_value(key));
      sk = f64_order_key(sc + 0.0);  // no NaN; +0.0 folds -0 into +0
      const size_t e = size_t(b) * P + base + lane;
      w.tok[e] = tok;
      w.par[e] = cpar[r];
      w.depth[e] = step;
      w.score[e] = sc;
    }
    int rank = -1;
    for (int q = 0; q < k; ++q) {
      const Popped p = wave_pop<1>(&sk);
      if (lane == p.lane) rank = q;
    }
    if (lane < n) {
      w.fslot[size_t(b) * P + base + lane] = rank;
      if (rank >= 0) {
        w.frontier[b * max_topk + rank] = base + lane;
        w.fscore[b * max_topk + rank] = sc;
        frontier_tokens[b * max_topk + rank] = tok;
      }
    }
  }
  if (lane >= k && lane < max_topk) frontier_tokens[b * max_topk + lane] = -1;
}

// One kernel for every step. Block (slice x, frontier slot f, sequence b) reduces a slice of
// step-`step` draft row f to its top-k keys and publishes them; the last block of the sequence's
// step to finish (ticket) merges the slices of every row: at step 1 the root row fills the pool and
// the frontier; at step >= 2 the k rows' k children join the pool (score = parent score + log-prob,
// an fp64 left fold), the k*k children are ranked and the best k form the next frontier.
// Every block reads its row slice before it knows k_b and D_b (rows f < gridDim.y must exist), and
// the frontier with its scores, so that those latencies overlap.
template <bool VEC, int EPL>
__global__ void __launch_bounds__(kRowThreads, 5) build_step_kernel(BuildWs w, int P, int step, const float* draft,
                                                                  int64_t seq_stride, const int32_t* topk,
                                                                  const int32_t* depth, int max_topk, int max_depth,
                                                                  int V, int slice, int per_wave, int early_k,
                                                                  int32_t* frontier_tokens, const int32_t* token_map,
                                                                  FinishArgs fa) {
  constexpr int NWV = kRowThreads / kWave;
  __shared__ uint64_t keys[kMaxTopk];
  __shared__ uint64_t top[kMaxTopk * kMaxTopk];  // [row][rank]
  __shared__ double fsc_s[kMaxTopk];
  __shared__ int cpar[kMaxTopk];
  __shared__ int last;
  const int x = blockIdx.x, f = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int n_slices = gridDim.x;
  const float* row = draft + b * seq_stride + int64_t(f) * V;
  const int lo = x * slice, hi = min(V, lo + slice);
  const int k_in = topk[b], d_in = depth[b];
  // launches with many rows (early_k) learn k and the depth before any row load, so the rows a sequence
  // does not expand are never read; small launches issue the first batch first (one round trip less)
  if (early_k && (step > clamp_i(d_in, 1, max_depth) || f >= (step == 1 ? 1 : clamp_i(k_in, 1, max_topk)))) return;
  float xs[EPL];
  load_batch<VEC, EPL>(row, lo, hi, xs);
  int fpar = 0;
  double fsc = 0.0;
  if (step >= 2 && tid < max_topk) {
    fpar = w.frontier[b * max_topk + tid];
    fsc = w.fscore[b * max_topk + tid];
  }
  const int k = clamp_i(k_in, 1, max_topk);
  const int D = clamp_i(d_in, 1, max_depth);
  const int rows = step == 1 ? 1 : k;
  // a row the sequence does not expand (slot past its k, or a step past its depth) stops here (without
  // early_k its first load batch was issued before k and the depth were known; the rest is never read)
  if (step > D || f >= rows) return;
  const uint64_t wave_key = block_slice_topk<VEC, EPL>(row, lo, hi, k, per_wave, xs, keys);
  uint64_t* cand = w.cand + (size_t(b) * max_topk + f) * kCand;
  if (per_wave) {  // the wave lists of slice x are lists x NWV .. x NWV + NWV - 1 of the row
    if (lane < k) st_agent(cand + (x * NWV + wave) * k + lane, wave_key);
  } else if (tid < k) {
    st_agent(cand + x * k + tid, keys[tid]);
  }
  wait_global_stores();
  __syncthreads();
  if (tid == 0) last = (ticket_add(w.ticket + size_t(b) * kTicketStride) == uint32_t(n_slices * rows - 1));
  __syncthreads();
  if (!last) return;
  if (tid == 0) ticket_reset(w.ticket + size_t(b) * kTicketStride);  // leave the workspace ready for the next step

  // every row's n_slices * k <= kCand candidates (0 = empty); wave w merges rows w and w + NWV,
  // each lane holding up to four candidates of a row
  const int nc = n_slices * (per_wave ? NWV : 1) * k;
  uint64_t cv[2][kCandPerLane];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
#pragma unroll
    for (int h = 0; h < kCandPerLane; ++h) {
      const int r = wave + it * NWV, j = lane + h * kWave;
      cv[it][h] = (r < rows && j < nc) ? ld_agent(w.cand + (size_t(b) * max_topk + r) * kCand + j) : 0ull;
    }
  }
  if (tid < k) {
    cpar[tid] = fpar;
    fsc_s[tid] = fsc;
  }
  const int base = k + (step - 2) * k * k;  // pool index of this step's first child (step >= 2)
  // row r's k best in rank order: k pops (a lane holds all of its candidates); a wave with two rows
  // runs both in the same rounds, so the two chains overlap
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    uint64_t* q = cv[it];
    auto cs = [](uint64_t& x, uint64_t& y) {
      const bool g = y > x;
      const uint64_t t = g ? y : x;
      y = g ? x : y;
      x = t;
    };
    cs(q[0], q[1]);
    cs(q[2], q[3]);
    cs(q[0], q[2]);
    cs(q[1], q[3]);
    cs(q[1], q[2]);
  }
  if (wave < rows) {
    const bool two = wave + NWV < rows;
    uint64_t r0 = 0, r1 = 0;
    for (int r = 0; r < k; ++r) {
      const Popped p0 = wave_pop<kCandPerLane>(cv[0]);
      if (lane == r) r0 = p0.key;
      if (two) {
        const Popped p1 = wave_pop<kCandPerLane>(cv[1]);
        if (lane == r) r1 = p1.key;
      }
    }
    if (lane < k) {
      top[wave * kMaxTopk + lane] = r0;
      if (two) top[(wave + NWV) * kMaxTopk + lane] = r1;
    }
  }
  __syncthreads();

  if (step == 1) {
    if (tid < max_topk) {
      const int c = tid;
      int tok = -1;
      if (c < k) {
        const size_t e = size_t(b) * P + c;
        const double sc = 0.0 + double(key_value(top[c]));
        tok = map_token(token_map, key_token(top[c]));
        w.tok[e] = tok;
        w.par[e] = -1;
        w.depth[e] = 1;
        w.fslot[e] = c;
        w.score[e] = sc;
        w.frontier[b * max_topk + c] = c;
        w.fscore[b * max_topk + c] = sc;
      }
      frontier_tokens[b * max_topk + c] = tok;
    }
  } else if (wave == 0) {
    step_children(w, P, b, step, k, base, max_topk, top, fsc_s, cpar, token_map, frontier_tokens);
  }
  if (fa.tokens && step == D) {  // the sequence's last step: rerank now (its pool is complete)
    wait_global_stores();
    __syncthreads();
    finish_sequence<true>(w, P, b, k, D, max_topk, fa);
  }
}


__global__ void __launch_bounds__(kFinishThreads) build_finish_kernel(BuildWs w, int P, const int32_t* topk,
                                                                       const int32_t* depth, int max_topk,
                                                                       int max_depth, FinishArgs fa) {
  const int b = blockIdx.x;
  finish_sequence<false>(w, P, b, clamp_i(topk[b], 1, max_topk), clamp_i(depth[b], 1, max_depth), max_topk, fa);
}

int32_t check_build(const char* who, int32_t B, int32_t max_topk, int32_t max_depth) {
  if (B < 1) return fail(SPEC_E_INVAL, "%s: B=%d", who, B);
  if (max_topk < 1 || max_topk > kMaxTopk) return fail(SPEC_E_UNSUPPORTED, "%s: max_topk=%d not in [1, %d]", who, max_topk, kMaxTopk);
  if (max_depth < 1 || max_depth > kMaxDepth)
    return fail(SPEC_E_UNSUPPORTED, "%s: max_depth=%d not in [1, %d]", who, max_depth, kMaxDepth);
  return SPEC_OK;
}

}  // namespace
}  // namespace spectree

using namespace spectree;

extern "C" size_t spec_tree_build_workspace_size(int32_t B, int32_t max_topk, int32_t max_depth) {
  if (check_build("spec_tree_build_workspace_size", B, max_topk, max_depth) != SPEC_OK) return 0;
  size_t total = 0;
  carve(nullptr, 0, B, max_topk, max_depth, &total);
  return total;
}

namespace spectree {
namespace {

int32_t launch_step(const char* who, void* ws, size_t ws_bytes, int32_t step, const float* draft_logprobs,
                    const int32_t* token_map, int64_t seq_stride, const int32_t* topk, const int32_t* depth, int32_t B, int32_t max_topk,
                    int32_t max_depth, int32_t V, int32_t* frontier_tokens, const FinishArgs& fa, void* stream) {
  int32_t rc = check_build(who, B, max_topk, max_depth);
  if (rc != SPEC_OK) return rc;
  if (step < 1 || step > max_depth) return fail(SPEC_E_INVAL, "%s: step=%d not in [1, %d]", who, step, max_depth);
  if (V < max_topk || V >= (1 << 30)) return fail(SPEC_E_INVAL, "%s: V=%d must be in [max_topk, 2^30)", who, V);
  if (!draft_logprobs || !topk || !depth || !frontier_tokens) return fail(SPEC_E_INVAL, "%s: null pointer", who);
  const int64_t min_stride = (step == 1 ? 1 : max_topk) * int64_t(V);
  if (B > 1 && seq_stride < min_stride)
    return fail(SPEC_E_INVAL, "%s: seq_stride=%lld < %lld", who, (long long)seq_stride, (long long)min_stride);
  size_t need = 0;
  BuildWs w = carve(ws, ws_bytes, B, max_topk, max_depth, &need);
  if (!ws || ws_bytes < need) return fail(SPEC_E_WORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 15) return fail(SPEC_E_INVAL, "%s: ws must be 16-byte aligned", who);
  const int P = int(pool_cap(max_topk, max_depth));
  hipStream_t st = static_cast<hipStream_t>(stream);
  // about 256 blocks per launch, within: slices of at least 8 elements per thread and of at most
  // kMaxBatches load batches of 16 per thread, and at most kCand / max_topk slices per row (a row's
  // candidates fit the merging wave). EPL is the smaller of 8, 16 that covers a slice in one batch,
  // else 16 with several batches (each prefetched while the previous one is reduced). Registers stay
  // within 5 waves per SIMD.
  const int rows_grid = step == 1 ? 1 : max_topk;
  const int max_sl = std::max(1, kCand / max_topk);
  static const int target = [] {
    const char* e = std::getenv("SPEC_TREE_BUILD_BLOCKS");  // blocks per launch (tuning override)
    const int v = e ? std::atoi(e) : 0;
    return v > 0 ? v : 256;
  }();
  static const int max_batches = [] {
    const char* e = std::getenv("SPEC_TREE_BUILD_BATCHES");  // load batches per slice (tuning override)
    const int v = e ? std::atoi(e) : 0;
    return v > 0 ? std::min(v, kMaxBatches) : kMaxBatches;
  }();
  const int want = std::max(1, (target + B * rows_grid - 1) / (B * rows_grid));
  int n_slices = std::min(want, (V + 8 * kRowThreads - 1) / (8 * kRowThreads));
  n_slices = std::max(n_slices, (V + max_batches * kMaxEpl * kRowThreads - 1) / (max_batches * kMaxEpl * kRowThreads));
  n_slices = std::max(1, std::min(n_slices, max_sl));
  const int per = (V + n_slices - 1) / n_slices;
  int epl = 8;
  while (epl < kMaxEpl && epl * kRowThreads < per) epl *= 2;
  const int batch = epl * kRowThreads;
  const int slice = (per + batch - 1) / batch * batch;
  n_slices = (V + slice - 1) / slice;
  const dim3 grid(n_slices, rows_grid, B);
  // each wave publishes its own list when every row's wave lists fit the merging wave (saves the
  // block's cross-wave selection: a barrier and k pops)
  const int per_wave = n_slices * (kRowThreads / kWave) * max_topk <= kCand ? 1 : 0;
  // 64 or more rows per launch: skip the rows a sequence does not expand before loading them (mixed batch
  // of 32 sequences with k in 4..8 and depth 4..6: about half the rows of a step)
  const int early_k = B * rows_grid >= 64 ? 1 : 0;
  const bool vec = (V % 4 == 0) && (seq_stride % 4 == 0) && ((reinterpret_cast<uintptr_t>(draft_logprobs) & 15) == 0);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kRowThreads), 0, st, w, P, step, draft_logprobs, seq_stride, topk, depth,
                       max_topk, max_depth, V, slice, per_wave, early_k, frontier_tokens, token_map, fa);
  };
  if (vec) {
    if (epl == 8) go(build_step_kernel<true, 8>);
    else go(build_step_kernel<true, 16>);
  } else {
    if (epl == 8) go(build_step_kernel<false, 8>);
    else go(build_step_kernel<false, 16>);
  }
  return check_launch(who);
}

}  // namespace
}  // namespace spectree



extern "C" int32_t spec_tree_build_step(void* ws, size_t ws_bytes, int32_t step, const float* draft_logprobs,
                                        int64_t seq_stride, const int32_t* topk, const int32_t* depth, int32_t B,
                                        int32_t max_topk, int32_t max_depth, int32_t V, int32_t* frontier_tokens,
                                        void* stream) {
  const FinishArgs none{};
  return launch_step("spec_tree_build_step", ws, ws_bytes, step, draft_logprobs, nullptr, seq_stride, topk, depth, B,
                     max_topk, max_depth, V, frontier_tokens, none, stream);
}

extern "C" int32_t spec_tree_build_step_map(void* ws, size_t ws_bytes, int32_t step, const float* draft_logprobs,
                                            const int32_t* token_map, int64_t seq_stride, const int32_t* topk,
                                            const int32_t* depth, int32_t B, int32_t max_topk, int32_t max_depth,
                                            int32_t V, int32_t* frontier_tokens, void* stream) {
  const FinishArgs none{};
  return launch_step("spec_tree_build_step_map", ws, ws_bytes, step, draft_logprobs, token_map, seq_stride, topk,
                     depth, B, max_topk, max_depth, V, frontier_tokens, none, stream);
}

static int32_t step_finish(const char* who, void* ws, size_t ws_bytes, int32_t step, const float* draft_logprobs,
                           const int32_t* token_map, int64_t seq_stride, const int32_t* topk, const int32_t* depth,
                           int32_t B, int32_t max_topk, int32_t max_depth, int32_t V, int32_t* frontier_tokens,
                           const int32_t* root_tokens, const int32_t* num_draft, int32_t max_T, int32_t* tokens,
                           int32_t* parents, int32_t* depth_out, uint64_t* anc_mask, int32_t* q_row, void* stream) {
  if (max_T < 2 || max_T > 65) return fail(SPEC_E_UNSUPPORTED, "%s: max_T=%d not in [2, 65]", who, max_T);
  if (!root_tokens || !num_draft || !tokens || !parents || !depth_out || !anc_mask || !q_row)
    return fail(SPEC_E_INVAL, "%s: null pointer", who);
  const FinishArgs fa{root_tokens, num_draft, max_T, tokens, parents, depth_out, anc_mask, q_row};
  return launch_step(who, ws, ws_bytes, step, draft_logprobs, token_map, seq_stride, topk, depth, B, max_topk,
                     max_depth, V, frontier_tokens, fa, stream);
}

extern "C" int32_t spec_tree_build_step_finish(void* ws, size_t ws_bytes, int32_t step, const float* draft_logprobs,
                                               int64_t seq_stride, const int32_t* topk, const int32_t* depth,
                                               int32_t B, int32_t max_topk, int32_t max_depth, int32_t V,
                                               int32_t* frontier_tokens, const int32_t* root_tokens,
                                               const int32_t* num_draft, int32_t max_T, int32_t* tokens,
                                               int32_t* parents, int32_t* depth_out, uint64_t* anc_mask,
                                               int32_t* q_row, void* stream) {
  return step_finish("spec_tree_build_step_finish", ws, ws_bytes, step, draft_logprobs, nullptr, seq_stride, topk,
                     depth, B, max_topk, max_depth, V, frontier_tokens, root_tokens, num_draft, max_T, tokens, parents,
                     depth_out, anc_mask, q_row, stream);
}

extern "C" int32_t spec_tree_build_step_finish_map(void* ws, size_t ws_bytes, int32_t step,
                                                   const float* draft_logprobs, const int32_t* token_map,
                                                   int64_t seq_stride, const int32_t* topk, const int32_t* depth,
                                                   int32_t B, int32_t max_topk, int32_t max_depth, int32_t V,
                                                   int32_t* frontier_tokens, const int32_t* root_tokens,
                                                   const int32_t* num_draft, int32_t max_T, int32_t* tokens,
                                                   int32_t* parents, int32_t* depth_out, uint64_t* anc_mask,
                                                   int32_t* q_row, void* stream) {
  return step_finish("spec_tree_build_step_finish_map", ws, ws_bytes, step, draft_logprobs, token_map, seq_stride,
                     topk, depth, B, max_topk, max_depth, V, frontier_tokens, root_tokens, num_draft, max_T, tokens,
                     parents, depth_out, anc_mask, q_row, stream);
}

extern "C" int32_t spec_tree_build_finish(void* ws, size_t ws_bytes, const int32_t* root_tokens, const int32_t* topk,
                                          const int32_t* depth, const int32_t* num_draft, int32_t B, int32_t max_topk,
                                          int32_t max_depth, int32_t max_T, int32_t* tokens, int32_t* parents,
                                          int32_t* depth_out, uint64_t* anc_mask, int32_t* q_row, void* stream) {
  int32_t rc = check_build("spec_tree_build_finish", B, max_topk, max_depth);
  if (rc != SPEC_OK) return rc;
  if (max_T < 2 || max_T > 65) return fail(SPEC_E_UNSUPPORTED, "spec_tree_build_finish: max_T=%d not in [2, 65]", max_T);
  if (!root_tokens || !topk || !depth || !num_draft || !tokens || !parents || !depth_out || !anc_mask || !q_row)
    return fail(SPEC_E_INVAL, "spec_tree_build_finish: null pointer");
  size_t need = 0;
  BuildWs w = carve(ws, ws_bytes, B, max_topk, max_depth, &need);
  if (!ws || ws_bytes < need) return fail(SPEC_E_WORKSPACE, "spec_tree_build_finish: workspace %zu < %zu bytes", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 15) return fail(SPEC_E_INVAL, "spec_tree_build_finish: ws must be 16-byte aligned");
  const int P = int(pool_cap(max_topk, max_depth));
  const FinishArgs fa{root_tokens, num_draft, max_T, tokens, parents, depth_out, anc_mask, q_row};
  hipLaunchKernelGGL(build_finish_kernel, dim3(B), dim3(kFinishThreads), 0, static_cast<hipStream_t>(stream), w, P,
                     topk, depth, max_topk, max_depth, fa);
  return check_launch("spec_tree_build_finish");
}
