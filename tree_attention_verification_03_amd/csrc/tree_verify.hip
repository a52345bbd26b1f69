// Tree verification: greedy argmax, or rejection sampling with residual resampling.
//
// n1n.ai "Speculative Decoding in Production: EAGLE-3 Dynamic Trees", section
// "Mathematical Proof of Lossless Speedup" (alpha = min(1, p/q); accept iff
// r <= alpha; on rejection draw from norm(max(0, p - q))) and section "From
// Linear Sequences to Dynamic Draft Trees" (a rejected sibling does not end
// the tree: B1 rejected, B2 accepted); tanhdev "Tech Radar: SGLang EAGLE-2",
// section 5 "Speculative Rejection Sampling: Mathematical Invariance";
// lesty.tech "EAGLE-2 & Lookahead Decoding", "Tree Attention Masking and
// Target Verification" (all paths are checked at once; the longest valid path
// wins and one more token is emitted).
//
// Every node's outcome depends only on its own rows, its children's tokens and
// the node's uniforms, so all nodes are evaluated in parallel, in two launches
// of 256-thread blocks:
//   rows kernel    greedy slice blocks reduce a slice of a greedy row to a
//                  packed 64-bit key (order(value) << 32 | ~index) merged with
//                  a 64-bit atomicMax - order-free, bit-exact; the last slice
//                  block of a greedy sequence (ticket) walks its tree. Sampling
//                  slice blocks take every (node, slice) of the sampling
//                  sequences by a fixed stride and publish the slice's exact
//                  integer sums of fx(p) and fx(q) and its ratio-bin window
//                  record (below).
//   decide kernel  one block per sampling node: it tests the node's children in
//                  index order against the residual, each rejection's residual
//                  mass from the window records, or (outside the window) from
//                  a pass of its own over the row, then resamples if no child
//                  is accepted; the block finishing a sequence's last node
//                  (ticket) walks its tree.
// Nothing waits on another block: hand-offs are the kernel boundary and
// last-arriver tickets. The walk emits the longest valid path (greedy) or the
// chain of ACCEPT links (sampling), the tokens, bonus and status, and
// re-zeroes the workspace's tickets and keys.
#include <stdlib.h>

#include "api_common.h"
#include "spec_common.h"

namespace spectree {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kSampleSlice = 8192;  // row elements per sampling slice block
constexpr int kGreedySlice = 8192;  // row elements per greedy block (one round trip of loads) ...
constexpr int kGreedySliceMax = 3 * kGreedySlice;  // ... up to three times that when the rows need many blocks
constexpr int kGreedyBlocksTarget = 448;           // greedy blocks one launch keeps resident (2 per CU, less room)
constexpr int kMaxSampleBlocks = 2048;  // sampling slice blocks of one rows launch (items by a fixed stride)
constexpr int kMaxKids = 64;  // children of one node (T <= 65)
// every ticket (kQ uint32 apart) and greedy argmax key (kKS uint64) sits on its own 128-byte line
constexpr int kQ = 32;
constexpr int kKS = 16;
constexpr int kMaxSampleMap = 2048;  // sampling sequences a block lists in LDS
constexpr int kRs = 8;               // u64 words of a node's published resampling state
constexpr int kKidsSeqs = 256;       // sampling sequences whose child masks a slice block keeps in LDS

// Residual mass from a window of ratio bins. Over a node's row, the mass after j rejections,
// W(G) = sum_v max(0, P[v] S_Q - G Q[v]) with G = gamma_j, only counts elements whose ratio P/Q exceeds
// theta = G / S_Q. Each slice block sorts its elements with P > 0 by n = floor(8 P / Q): for 1/2 <= P/Q < 8
// into bins 0..59 (bin n - 4, keeping the bin's sums of P and Q and the elements themselves, grouped by
// bin), P/Q >= 8 or Q = 0 into the high set (sums only), smaller ratios nowhere. For 1/2 <= theta < 8 every
// element of a bin above floor(8 theta) counts in full (P S_Q - G Q >= 0) and every element below it not at
// all, so W(G) is the high set's and those bins' sums plus an exact per-element sum over the one bin that
// holds theta: no pass over the row. theta_1 = S_P / S_Q (1 for normalised rows) and each rejection adds at
// most theta_1, so a node with up to 8 children stays inside the window; outside it, or when a slice holds
// more window elements than it keeps, the deciding block takes a pass over the row instead.
constexpr int kWinBins = 60;     // window bins (ratios 1/2 .. 8 in steps of 1/8)
constexpr int kWinHi = 60;       // record slot of the high set
constexpr int kWinSlots = 64;    // record slots per slice (bins, high set, padding)
constexpr int kWinCap = 2048;    // window elements a slice keeps (a quarter of its elements)
constexpr int kFastMaxSl = 16;   // slices per row the decision keeps in LDS (V <= 131072)
constexpr uint64_t kWinOverflow = 4;  // slice flag: the window was not (fully) recorded

struct VerifyWs {
  uint64_t* keys;      // [B*max_T] greedy argmax keys (0 = empty)
  uint32_t* rowflag;   // [B*max_T] NaN seen in the greedy row
  int32_t* acc_child;  // [B*max_T] sampling: accepted child node or -1
  uint64_t* rstate;    // [B*max_T][kRs] sampling: a node without an accepted child: W (u128), gamma, S_Q, K,
                       // plain | mass source << 8 (its per-slice masses: ssum or smass)
  uint32_t* nflag;     // [B*max_T] sampling node flags
  uint32_t* tickets;   // [B] greedy: rows done; sampling: nodes done
  uint32_t* rtick;     // [B*max_T] greedy: slice blocks of the row done
  uint64_t* ssum;      // [B*max_T][nsl] slice sums of fx(p)
  uint64_t* psum;      // [B*max_T][nsl][2] slice sum of fx(q), NaN / window bits
  uint64_t* smass;     // [B*max_T][nsl][2] a decision's own row pass: per-slice residual masses (u128)
  // window records (null when a row has more than kFastMaxSl slices)
  uint32_t* wcnt;      // [B*max_T*nsl][kWinSlots] elements per window bin; slot kWinHi: all window elements
  uint64_t* wsum;      // [B*max_T*nsl][kWinSlots][2] sums of P and Q per bin; slot kWinHi: the high set
  uint64_t* wel;       // [B*max_T*nsl][kWinCap] window elements (P << 32 | Q), grouped by bin
};

int sample_slices(int V) { return (V + kSampleSlice - 1) / kSampleSlice; }

// the parts that need not start at zero, laid out from c (null: sizes only); returns their size
size_t carve_data(char* c, size_t n, size_t nsl, VerifyWs& w) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = c ? c + off : nullptr;
    off = align_up(off + bytes, 256);
    return r;
  };
  w.acc_child = reinterpret_cast<int32_t*>(take(4 * n));
  w.rstate = reinterpret_cast<uint64_t*>(take(8 * n * kRs));
  w.nflag = reinterpret_cast<uint32_t*>(take(4 * n));
  w.ssum = reinterpret_cast<uint64_t*>(take(8 * n * nsl));
  w.psum = reinterpret_cast<uint64_t*>(take(16 * n * nsl));
  w.smass = reinterpret_cast<uint64_t*>(take(16 * n * nsl));
  w.wcnt = nullptr;
  w.wsum = nullptr;
  w.wel = nullptr;
  if (nsl <= size_t(kFastMaxSl)) {
    w.wcnt = reinterpret_cast<uint32_t*>(take(4 * n * nsl * kWinSlots));
    w.wsum = reinterpret_cast<uint64_t*>(take(16 * n * nsl * kWinSlots));
    w.wel = reinterpret_cast<uint64_t*>(take(8 * n * nsl * kWinCap));
  }
  return off;
}

// The parts that must start at zero (keys, row flags, tickets) sit at the start of the workspace, at offsets
// set by B and max_T alone; the rest sits at the end of its ws_bytes. A workspace zero-filled once therefore
// serves calls of several shapes without clearing: no call's data lands on another shape's zero parts as
// long as ws_bytes covers the largest zero parts plus every call's data. With ws null (or ws_bytes below
// *total) only *total is meaningful.
VerifyWs carve(void* ws, size_t ws_bytes, int B, int max_T, int V, size_t* total) {
  const size_t n = size_t(B) * max_T;
  const size_t nsl = size_t(sample_slices(V));
  char* c = static_cast<char*>(ws);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = c ? c + off : nullptr;
    off = align_up(off + bytes, 256);
    return r;
  };
  VerifyWs w;
  w.keys = reinterpret_cast<uint64_t*>(take(8 * n * kKS));
  w.rowflag = reinterpret_cast<uint32_t*>(take(4 * n));
  w.tickets = reinterpret_cast<uint32_t*>(take(4 * size_t(B) * kQ));
  w.rtick = reinterpret_cast<uint32_t*>(take(4 * n * kQ));
  const size_t data = carve_data(nullptr, n, nsl, w);
  *total = off + data;
  if (c && ws_bytes >= *total) carve_data(c + ((ws_bytes - data) & ~size_t(255)), n, nsl, w);
  return w;
}

struct VerifyArgs {
  const float* target;
  const float2* sm_part;     // logits given: every sampling row's slice partials (max, sum of exp), else null
  const float* temperature;  // logits given: per-sequence temperatures (null: 1)
  int sm_nsl;                // logits given: partials per row
  const float* draft;
  const int32_t* q_row;
  const int32_t* tokens;
  const int32_t* parents;
  const int32_t* T_b;
  const int8_t* mode;
  uint64_t key0, key1, offset;
  int B, max_T, R, V, n_slices, slice, nsl, n_greedy_blocks, n_sample_blocks;
  int sample_first;  // sampling slice blocks take the grid's first ids (else the greedy blocks do)
  int row_tickets;  // greedy: count slice blocks per row first (sequences with many slice blocks)
  int fast;         // sampling: residual masses from the window records when they allow it
  int32_t* accept_len;
  int32_t* accept_nodes;
  int32_t* out_tokens;
  uint32_t* status;
};

__device__ __forceinline__ int seq_T(const int32_t* T_b, int b, int max_T) {
  int T = T_b ? T_b[b] : max_T;
  return T < 1 ? 1 : (T > max_T ? max_T : T);
}

// e^t for t <= 0 (a softmax term against its row's maximum): the hardware base-2 exponential of t log2(e).
// Rounding t log2(e) costs at most half an ulp of t in the exponent, the same order as the rounding of
// t itself; results below 2^-126 flush toward zero, far below the 2^-32 resolution of the sampling rule.
__device__ __forceinline__ float exp_nonpos(float t) { return __builtin_amdgcn_exp2f(t * 1.4426950408889634f); }

// a sequence's sampling temperature, 0 when it is not a finite positive number
__device__ __forceinline__ float sm_temperature(const float* temperature, int b) {
  const float T = temperature ? temperature[b] : 1.f;
  return (T > 0.f && isfinite(T)) ? T : 0.f;
}

// A node's target probabilities for the sampling rule: the row as the caller supplies it (LG false), or
// formed from the target's logits (LG true) as p[v] = exp(x - M) * (1 / S) with x = l[v] * (1 / T_b), where
// M and S are the row's maximum and sum of exponentials merged from its slice partials in a fixed order.
// Every block merges them the same way, so p[v] is the same number in every pass that reads it. A
// non-finite x gives NaN, and so does every element of a row whose temperature is not a finite positive
// number (NaN probabilities count as zero and raise SPEC_STATUS_NAN_INPUT).
template <bool LG>
struct ProbRow {
  float inv = 1.f, M = 0.f, rS = 1.f;  // rS = 1 / S
  __device__ __forceinline__ float operator()(float l) const {
    if constexpr (!LG) {
      return l;
    } else {
      const float x = l * inv;
      return isfinite(x) ? exp_nonpos(x - M) * rS : NAN;
    }
  }
};

// the row's partials are merged across each wave's lanes (lane j takes partials j, j + 64, ...) with xor
// butterflies, the same fixed order in every wave, block and pass (fp32 max and add are commutative, so every
// lane ends with the same M and S)
template <bool LG>
__device__ __forceinline__ ProbRow<LG> prob_row(const VerifyArgs& a, size_t node) {
  ProbRow<LG> r;
  if constexpr (LG) {
    const float T = sm_temperature(a.temperature, int(node / size_t(a.max_T)));
    if (T == 0.f) {
      r.inv = NAN;
      return r;
    }
    r.inv = 1.f / T;
    const float2* pr = a.sm_part + node * size_t(a.sm_nsl);
    const int lane = threadIdx.x & (kWave - 1), n = a.sm_nsl;
    const float2 q0 = lane < n ? pr[lane] : make_float2(-INFINITY, 0.f);
    float M = q0.x;
    for (int j = lane + kWave; j < n; j += kWave) M = fmaxf(M, pr[j].x);
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, kWave));
    float S = q0.x != -INFINITY ? q0.y * exp_nonpos(q0.x - M) : 0.f;
    for (int j = lane + kWave; j < n; j += kWave) {
      const float2 q = pr[j];
      if (q.x != -INFINITY) S += q.y * exp_nonpos(q.x - M);
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) S += __shfl_xor(S, o, kWave);
    r.M = M;
    r.rS = 1.f / S;
  }
  return r;
}

__device__ __forceinline__ const float* sample_row(const VerifyArgs& a, size_t node) {
  return a.target + node * size_t(a.V);
}

__device__ __forceinline__ uint64_t argmax_key(float x, int v) {
  if (x != x) x = -INFINITY;  // NaN counts as -inf
  if (x == 0.f) x = 0.f;      // -0 == +0
  return (uint64_t(f32_order_key(x)) << 32) | uint64_t(0xffffffffu - uint32_t(v));
}

// ------------------------------------------------------------------ greedy
template <bool VEC, int NV>
__device__ __forceinline__ void greedy_slice(const VerifyWs& w, const VerifyArgs& a, int row, int lo) {
  __shared__ uint64_t red[kWaves];
  __shared__ uint32_t nanred[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = min(a.V, lo + a.slice);
  const float* r = a.target + size_t(row) * a.V;
  uint64_t best = 0;
  bool nan = false;
  if (VEC) {  // a slice is at most 4 * kThreads * NV elements: all of a thread's loads in one round trip
    float4 xs[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = lo + 4 * tid + 4 * kThreads * i;
      xs[i] = v < hi ? *reinterpret_cast<const float4*>(r + v) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = lo + 4 * tid + 4 * kThreads * i;
      if (v >= hi) continue;
      const float4 x = xs[i];
      nan |= (x.x != x.x) | (x.y != x.y) | (x.z != x.z) | (x.w != x.w);
      uint64_t k0 = argmax_key(x.x, v), k1 = argmax_key(x.y, v + 1), k2 = argmax_key(x.z, v + 2), k3 = argmax_key(x.w, v + 3);
      k0 = k0 > k1 ? k0 : k1;
      k2 = k2 > k3 ? k2 : k3;
      k0 = k0 > k2 ? k0 : k2;
      best = k0 > best ? k0 : best;
    }
  } else {
    for (int v = lo + tid; v < hi; v += kThreads) {
      const float x = r[v];
      nan |= (x != x);
      const uint64_t k = argmax_key(x, v);
      best = k > best ? k : best;
    }
  }
  best = wave_max_u64(best);
  const uint32_t nw = wave_or_u32(nan ? 1u : 0u);
  if (lane == 0) {
    red[wave] = best;
    nanred[wave] = nw;
  }
  __syncthreads();
  if (tid == 0) {
    uint64_t m = red[0];
    uint32_t f = nanred[0];
    for (int i = 1; i < kWaves; ++i) {
      m = red[i] > m ? red[i] : m;
      f |= nanred[i];
    }
    atomicMax(reinterpret_cast<unsigned long long*>(w.keys + size_t(row) * kKS), (unsigned long long)m);
    if (f) atomicOr(w.rowflag + row, 1u);
  }
}

// ------------------------------------------------------------------ sampling
__device__ __forceinline__ uint32_t fx(float x) {
  // 2^-32 fixed point: 0 for NaN / x <= 0, 2^32-1 for x >= 1, floor(x * 2^32) otherwise. x * 2^32 is exact (a
  // power-of-two scaling) and the hardware conversion truncates and clamps (NaN and negatives to 0, 2^32 and
  // above to 2^32 - 1): two instructions. C++ leaves an out-of-range conversion undefined, hence the
  // instruction itself
  uint32_t r;
  asm("v_cvt_u32_f32 %0, %1" : "=v"(r) : "v"(x * 4294967296.0f));
  return r;
}

__device__ __forceinline__ u128 mul64x32(uint64_t a, uint32_t b) {
  const uint64_t lo = uint64_t(uint32_t(a)) * b;
  const uint64_t hi = (a >> 32) * b;
  return (u128(hi) << 32) + lo;
}

// residual N[v] = max(0, P[v] * S_Q - gamma * Q[v]); with plain_p it is P[v] itself
__device__ __forceinline__ u128 residual(uint32_t P, uint32_t Q, uint64_t S_Q, uint64_t gamma, bool plain_p) {
  if (plain_p) return u128(P);
  const u128 a = mul64x32(S_Q, P);
  const u128 c = mul64x32(gamma, Q);
  return a > c ? a - c : u128(0);
}

// does element (P, Q) have a positive residual, P S_Q > gamma Q (always, for a plain resample from p)? P = 0
// never does; otherwise the products' fp32 estimates are within 2^-22 of the exact values, so they decide unless
// within 1e-6 of each other
__device__ __forceinline__ bool res_pos(uint32_t P, uint32_t Q, uint64_t S_Q, uint64_t gamma, bool plain_p) {
  if (P == 0u) return false;
  if (plain_p) return true;
  const float a = float(P) * float(S_Q), c = float(gamma) * float(Q);
  if (a > c * 1.000001f) return true;
  if (a < c * 0.999999f) return false;
  return mul64x32(S_Q, P) > mul64x32(gamma, Q);
}

// sum of the residuals of a set of positive-residual elements from their sums of P and Q (exact:
// sum (P S_Q - gamma Q) = S_Q sum P - gamma sum Q over elements that are each positive)
__device__ __forceinline__ u128 res_sum(uint64_t sp, uint64_t sq, uint64_t S_Q, uint64_t gamma, bool plain_p) {
  if (plain_p) return u128(sp);
  return u128(S_Q) * sp - u128(gamma) * sq;
}

// x + y after a row swap of the pair: the 32-lane swap exchanges the upper half of x with the lower half of y,
// so lanes 0-31 get x summed with its xor-32 partner and lanes 32-63 get y summed likewise (the 16-lane swap:
// even 16-lane rows x, odd rows y, over the xor-16 partners)
template <bool HALVES>
__device__ __forceinline__ uint64_t swap_add_u64(uint64_t x, uint64_t y) {
  const uint32_t xl = uint32_t(x), xh = uint32_t(x >> 32), yl = uint32_t(y), yh = uint32_t(y >> 32);
  const auto l = HALVES ? __builtin_amdgcn_permlane32_swap(xl, yl, false, false) : __builtin_amdgcn_permlane16_swap(xl, yl, false, false);
  const auto h = HALVES ? __builtin_amdgcn_permlane32_swap(xh, yh, false, false) : __builtin_amdgcn_permlane16_swap(xh, yh, false, false);
  return ((uint64_t(uint32_t(h[0])) << 32) | uint32_t(l[0])) + ((uint64_t(uint32_t(h[1])) << 32) | uint32_t(l[1]));
}

// the wave sums of 8 u64 values at once: lane l returns the sum of v[l / 8] over the wave. A transposing
// butterfly halves the values held per lane at each step (32-lane halves, 16-lane rows, 8-lane halves of a row
// by rotation: each step pairs lanes that differ in the bit that selects which value they keep), then sums the
// 8 lanes left (half-row mirror, quad): about a third of the instructions of 8 separate sums
__device__ __forceinline__ uint64_t wave_sum8_u64(const uint64_t (&v)[8]) {
  constexpr int kRor8 = 0x128;  // row_ror:8 (xor 8 inside a 16-lane row)
  const int lane = threadIdx.x & 63;
  uint64_t w[4], u[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = swap_add_u64<true>(v[j], v[j + 4]);
#pragma unroll
  for (int j = 0; j < 2; ++j) u[j] = swap_add_u64<false>(w[j], w[j + 2]);
  const bool b3 = (lane & 8) != 0;
  uint64_t x = (b3 ? u[1] : u[0]) + dpp_u64<kRor8>(b3 ? u[0] : u[1]);
  x += dpp_u64<dpp::kHalfMirror>(x);
  x += dpp_u64<dpp::kXor1>(x);
  return x + dpp_u64<dpp::kXor2>(x);
}

__device__ __forceinline__ u128 shfl_xor_u128(u128 x, int o) {
  const uint64_t lo = __shfl_xor(uint64_t(x), o, kWave);
  const uint64_t hi = __shfl_xor(uint64_t(x >> 64), o, kWave);
  return (u128(hi) << 64) | lo;
}

__device__ __forceinline__ u128 shfl_up_u128(u128 x, int o) {
  const uint64_t lo = __shfl_up(uint64_t(x), o, kWave);
  const uint64_t hi = __shfl_up(uint64_t(x >> 64), o, kWave);
  return (u128(hi) << 64) | lo;
}

template <int CTRL>
__device__ __forceinline__ u128 dpp_u128(u128 v) {
  return (u128(dpp_u64<CTRL>(uint64_t(v >> 64))) << 64) | dpp_u64<CTRL>(uint64_t(v));
}

// the two row-swap results of a u128 (every lane's partner value is in one of them)
template <bool HALVES>
__device__ __forceinline__ void swap_u128(u128 v, u128& r0, u128& r1) {
  uint32_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = uint32_t(v >> (32 * i));
    const auto r = HALVES ? __builtin_amdgcn_permlane32_swap(x, x, false, false) : __builtin_amdgcn_permlane16_swap(x, x, false, false);
    a[i] = uint32_t(r[0]);
    b[i] = uint32_t(r[1]);
  }
  r0 = (u128(a[3]) << 96) | (u128(a[2]) << 64) | (u128(a[1]) << 32) | a[0];
  r1 = (u128(b[3]) << 96) | (u128(b[2]) << 64) | (u128(b[1]) << 32) | b[0];
}

__device__ __forceinline__ u128 wave_sum_u128(u128 x) {
  x += dpp_u128<dpp::kXor1>(x);
  x += dpp_u128<dpp::kXor2>(x);
  x += dpp_u128<dpp::kHalfMirror>(x);
  x += dpp_u128<dpp::kMirror>(x);
  u128 r0, r1;
  swap_u128<false>(x, r0, r1);
  x = r0 + r1;
  swap_u128<true>(x, r0, r1);
  return r0 + r1;
}

// f(v, p, q) over the wave's segment [lo, hi) of a row pair; q may be null (then 0)
template <bool VEC, typename F>
__device__ __forceinline__ void seg_for(const float* p, const float* q, int lo, int hi, int lane, F&& f) {
  if (VEC) {
    if (q) {
#pragma unroll 2
      for (int v = lo + 4 * lane; v < hi; v += 4 * kWave) {
        const float4 x = *reinterpret_cast<const float4*>(p + v);
        const float4 y = *reinterpret_cast<const float4*>(q + v);
        f(v, x.x, y.x);
        f(v + 1, x.y, y.y);
        f(v + 2, x.z, y.z);
        f(v + 3, x.w, y.w);
      }
    } else {
#pragma unroll 2
      for (int v = lo + 4 * lane; v < hi; v += 4 * kWave) {
        const float4 x = *reinterpret_cast<const float4*>(p + v);
        f(v, x.x, 0.f);
        f(v + 1, x.y, 0.f);
        f(v + 2, x.z, 0.f);
        f(v + 3, x.w, 0.f);
      }
    }
  } else {
    for (int v = lo + lane; v < hi; v += kWave) f(v, p[v], q ? q[v] : 0.f);
  }
}

// inclusive scan over the block's threads (u128); returns this thread's exclusive prefix
__device__ __forceinline__ u128 block_exclusive_scan_u128(u128 x, u128* wtot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  u128 incl = x;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const u128 t = shfl_up_u128(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) wtot[wave] = incl;
  __syncthreads();
  u128 before = 0;
  for (int i = 0; i < wave; ++i) before += wtot[i];
  return before + incl - x;
}

// the q row named by q_row whether or not the node has children (pass 0 reads it before the children
// are known; its sums only count for a node with children)
__device__ __forceinline__ const float* node_qrow_any(const VerifyArgs& a, int b, int u) {
  const int qr = a.q_row ? a.q_row[size_t(b) * a.max_T + u] : -1;
  return (a.draft != nullptr && qr >= 0 && qr < a.R) ? a.draft + (size_t(b) * a.R + qr) * a.V : nullptr;
}

// f(v, p, q) over this thread's elements of [lo, hi) (q may be null: then 0), p taken through the
// transform that pre() returns once the elements' loads are issued; a slice is at most kSampleSlice
// elements, so the vector path loads all of a thread's elements in one round trip
template <bool VEC, typename Pre, typename F>
__device__ __forceinline__ void slice_for(const float* p, const float* q, int lo, int hi, Pre&& pre, F&& f) {
  const int tid = threadIdx.x;
  if (VEC) {
    constexpr int NV = kSampleSlice / (4 * kThreads);
    float4 x[NV], y[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = lo + 4 * tid + 4 * kThreads * i;
      x[i] = v < hi ? *reinterpret_cast<const float4*>(p + v) : make_float4(0.f, 0.f, 0.f, 0.f);
      y[i] = (q && v < hi) ? *reinterpret_cast<const float4*>(q + v) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const auto tr = pre();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = lo + 4 * tid + 4 * kThreads * i;
      if (v < hi) {
        f(v, tr(x[i].x), y[i].x);
        f(v + 1, tr(x[i].y), y[i].y);
        f(v + 2, tr(x[i].z), y[i].z);
        f(v + 3, tr(x[i].w), y[i].w);
      }
    }
  } else {
    const auto tr = pre();
    for (int v = lo + tid; v < hi; v += kThreads) f(v, tr(p[v]), q ? q[v] : 0.f);
  }
}

// the block's sums of three u64 values; valid in thread 0
__device__ __forceinline__ void block_sum3(uint64_t& x0, uint64_t& x1, uint64_t& x2, uint64_t (*red)[3]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x0 = wave_sum_u64(x0);
  x1 = wave_sum_u64(x1);
  x2 = wave_sum_u64(x2);
  if (lane == 0) {
    red[wave][0] = x0;
    red[wave][1] = x1;
    red[wave][2] = x2;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int i = 1; i < kWaves; ++i) {
      x0 += red[i][0];
      x1 += red[i][1];
      x2 += red[i][2];
    }
}

template <bool VEC, bool LG>
__device__ __forceinline__ void sample_finish(const VerifyWs& w, const VerifyArgs& a, int b, int u, int acc, uint32_t flags,
                                              bool trivial);

// window bin of an element (see kWinBins): 0..kWinBins-1 for 1/2 <= P/Q < 8 (floor(8 P / Q) - 4), kWinHi
// for P/Q >= 8 or Q = 0, -1 for P = 0 or P/Q < 1/2. e = 8 P / Q from a hardware reciprocal is within 3e-5 of
// the exact quotient wherever it matters (below 64.0001), so floor(e) is exact unless e lies within 1e-4 of
// an integer; only then do 64-bit integer products decide
__device__ __forceinline__ int win_bin(uint32_t P, uint32_t Q) {
  if (P == 0u) return -1;
  if (Q == 0u) return kWinHi;
  const float e = float(P) * 8.f * __builtin_amdgcn_rcpf(float(Q));
  if (e >= 64.0001f) return kWinHi;
  if (e < 3.9999f) return -1;
  int n = int(e);
  const float r = rintf(e);
  if (fabsf(e - r) < 1e-4f) {  // near a bin edge k: 8 P >= k Q decides
    const int k = int(r);
    n = (uint64_t(P) << 3) >= uint64_t(k) * Q ? k : k - 1;
  }
  return n >= 64 ? kWinHi : (n < 4 ? -1 : n - 4);
}

// slice s of a sampling node: sums of fx(p) and fx(q) and NaN bits, published per slice
// (the node's decision block reduces them); for a node with a q row also the slice's window record and its window
// elements grouped by bin. Window elements are first staged in LDS, each wave in its own region at a running
// ballot offset, then counted and summed per bin, then placed by per-bin cursors: the order inside a bin is
// arbitrary, and nothing depends on it.
template <bool VEC, bool LG>
__device__ __forceinline__ void sample_slice(const VerifyWs& w, const VerifyArgs& a, int b, int u, int s, bool kids) {
  __shared__ uint64_t red[kWaves][3];
  __shared__ uint32_t wc_s[kWinSlots], wcur_s[kWinSlots], wn_s[kWaves];
  __shared__ unsigned long long wp_s[kWinSlots], wq_s[kWinSlots];
  __shared__ uint64_t stage_s[kWinCap];
  __shared__ uint8_t sbin_s[kWinCap];
  const int tid = threadIdx.x, lane = tid & 63;
  const size_t node = size_t(b) * a.max_T + u;
  const size_t rec = node * a.nsl + s;
  const float* prow = sample_row(a, node);
  const float* qrow = kids ? node_qrow_any(a, b, u) : nullptr;  // a node without children never reads its q row
  const int lo = s * kSampleSlice, hi = min(a.V, lo + kSampleSlice);
  const bool win = a.fast && qrow != nullptr && w.wcnt != nullptr;
  if (win && tid < kWinSlots) {
    wc_s[tid] = 0u;
    wp_s[tid] = 0ull;
    wq_s[tid] = 0ull;
  }
  if (win) __syncthreads();
  constexpr uint32_t kCapW = kWinCap / kWaves;  // staging slots per wave
  uint64_t* const stage_w = stage_s + (tid >> 6) * kCapW;
  uint8_t* const sbin_w = sbin_s + (tid >> 6) * kCapW;
  uint32_t run = 0;  // the wave's window elements so far (wave-uniform)
  uint64_t sp = 0, sq = 0, hp = 0, hq = 0;
  uint64_t nanp = 0, nanq = 0;  // lanes that met a NaN in p / q (wave-uniform ballots)
  const auto pre = [&] { return prob_row<LG>(a, node); };
  if (qrow) {
    slice_for<VEC>(prow, qrow, lo, hi, pre, [&](int v, float x, float y) {
      nanp |= __ballot(x != x);
      nanq |= __ballot(y != y);
      const uint32_t P = fx(x), Q = fx(y);
      sp += P;
      sq += Q;
      if (win) {
        const int bin = win_bin(P, Q);
        if (bin == kWinHi) {
          hp += P;
          hq += Q;
        }
        const bool in = bin >= 0 && bin < kWinBins;
        const uint64_t m = __ballot(in);
        const uint32_t pos = run + uint32_t(__popcll(m & ((1ull << lane) - 1)));
        if (in && pos < kCapW) {
          stage_w[pos] = (uint64_t(P) << 32) | Q;
          sbin_w[pos] = uint8_t(bin);
        }
        run += uint32_t(__popcll(m));
      }
    });
  } else {  // no q row (a childless node, or none given): p's sum and NaN bit only
    slice_for<VEC>(prow, nullptr, lo, hi, pre, [&](int, float x, float) {
      nanp |= __ballot(x != x);
      sp += fx(x);
    });
  }
  if (win && lane == 0) wn_s[tid >> 6] = run;
  // NaN bits travel through the block sum as counts (lane 0 of each wave): p in bits 0-3, q in bits 4-7
  const uint32_t nw = (nanp ? 1u : 0u) | (nanq ? 2u : 0u);
  uint64_t nn = lane == 0 ? uint64_t(nw & 1u) + ((nw & 2u) ? 16u : 0u) : 0u;
  if (win) {
    hp = wave_sum_u64(hp);
    hq = wave_sum_u64(hq);
    if (lane == 0) {
      atomicAdd(&wp_s[kWinHi], (unsigned long long)hp);
      atomicAdd(&wq_s[kWinHi], (unsigned long long)hq);
    }
  }
  block_sum3(sp, sq, nn, red);  // its barrier also completes the staging
  uint64_t wflag = kWinOverflow;
  if (win) {
    uint32_t total = 0;
    bool over = false;
    for (int i = 0; i < kWaves; ++i) {
      total += wn_s[i];
      over |= wn_s[i] > kCapW;
    }
    // staged element j: wave region j / kCapW, slot j % kCapW, valid below that wave's count
    auto staged = [&](int j) { return uint32_t(j % kCapW) < min(wn_s[j / kCapW], kCapW); };
    for (int j = tid; j < kWinCap; j += kThreads) {  // per-bin counts and sums
      if (!staged(j)) continue;
      const int bin = sbin_s[j];
      const uint64_t pq = stage_s[j];
      atomicAdd(&wc_s[bin], 1u);
      atomicAdd(&wp_s[bin], (unsigned long long)(pq >> 32));
      atomicAdd(&wq_s[bin], (unsigned long long)uint32_t(pq));
    }
    __syncthreads();
    if (tid < kWave) {  // the bins' offsets
      const uint32_t c = tid < kWinBins ? wc_s[tid] : 0u;
      uint32_t incl = c;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
      }
      wcur_s[tid] = incl - c;
    }
    __syncthreads();
    if (!over) {
      wflag = 0;
      uint64_t* el = w.wel + rec * kWinCap;
      for (int j = tid; j < kWinCap; j += kThreads)
        if (staged(j)) el[atomicAdd(&wcur_s[sbin_s[j]], 1u)] = stage_s[j];
    }
    if (tid < kWinSlots) {
      w.wcnt[rec * kWinSlots + tid] = tid < kWinBins ? wc_s[tid] : (tid == kWinHi ? total : 0u);
      w.wsum[(rec * kWinSlots + tid) * 2] = uint64_t(wp_s[tid]);
      w.wsum[(rec * kWinSlots + tid) * 2 + 1] = uint64_t(wq_s[tid]);
    }
  }
  if (tid == 0) {
    uint64_t* ps = w.psum + rec * 2;
    w.ssum[rec] = sp;
    ps[0] = sq;
    ps[1] = uint64_t(((nn & 15u) ? 1u : 0u) | ((nn >> 4) ? 2u : 0u)) | wflag;
  }
}

// LDS of a decision's fast path: the node's window records, per slice and bin
struct WinLds {
  uint32_t cnt[kFastMaxSl][kWinSlots];
  uint64_t sp[kFastMaxSl][kWinSlots], sq[kFastMaxSl][kWinSlots];  // slot kWinHi: the high set; above it zero
};

// the node's window records into LDS (every thread; no barrier: the caller's next one publishes them)
__device__ __forceinline__ void win_load(const VerifyWs& w, const VerifyArgs& a, size_t node, WinLds& L) {
  for (int i = threadIdx.x; i < a.nsl * kWinSlots; i += kThreads) {
    const int sl = i / kWinSlots, n = i - sl * kWinSlots;
    const size_t r = (node * a.nsl + sl) * kWinSlots + n;
    L.cnt[sl][n] = n < kWinBins ? w.wcnt[r] : 0u;
    L.sp[sl][n] = n <= kWinHi ? w.wsum[r * 2] : 0ull;
    L.sq[sl][n] = n <= kWinHi ? w.wsum[r * 2 + 1] : 0ull;
  }
}

// the window admits gamma: 1/2 <= gamma / S_Q < 8
__device__ __forceinline__ bool win_admits(uint64_t gamma, uint64_t S_Q) {
  const u128 g8 = u128(gamma) << 3;
  return g8 >= (u128(S_Q) << 2) && g8 < (u128(S_Q) << 6);
}

// sum over each 16-lane row of a wave (DPP only)
__device__ __forceinline__ u128 row16_sum_u128(u128 x) {
  x += dpp_u128<dpp::kXor1>(x);
  x += dpp_u128<dpp::kXor2>(x);
  x += dpp_u128<dpp::kHalfMirror>(x);
  return x + dpp_u128<dpp::kMirror>(x);
}

__device__ __forceinline__ uint64_t row16_sum_u64(uint64_t x) {
  x += dpp_u64<dpp::kXor1>(x);
  x += dpp_u64<dpp::kXor2>(x);
  x += dpp_u64<dpp::kHalfMirror>(x);
  return x + dpp_u64<dpp::kMirror>(x);
}

// Residual masses under gamma (admitted by the window) of every slice of the row into ssl, their total
// returned (every thread). Slice s is served by the 16 threads of row s of the block: bins above the
// straddling one and the high set from their sums, the straddling bin element by element.
__device__ __forceinline__ u128 win_mass(const VerifyWs& w, const VerifyArgs& a, size_t node, uint64_t S_Q, uint64_t gamma,
                                         const WinLds& L, u128* ssl) {
  const int tid = threadIdx.x, sl = tid >> 4, j = tid & 15, nsl = a.nsl;
  const int nb = int(div_u128_u64(u128(gamma) << 3, S_Q)) - 4;  // straddling bin, in [0, kWinBins)
  uint32_t below = 0, cnt = 0;
  uint64_t fp = 0, fq = 0;
  if (sl < nsl) {
#pragma unroll
    for (int n = j; n < kWinSlots; n += 16) {
      const uint32_t c = L.cnt[sl][n];
      below += n < nb ? c : 0u;
      cnt += n == nb ? c : 0u;
      fp += n > nb ? L.sp[sl][n] : 0ull;
      fq += n > nb ? L.sq[sl][n] : 0ull;
    }
  }
  below = uint32_t(row16_sum_u64(below));
  cnt = uint32_t(row16_sum_u64(cnt));
  fp = row16_sum_u64(fp);
  fq = row16_sum_u64(fq);
  u128 acc = 0;
  if (sl < nsl) {
    const uint64_t* el = w.wel + (node * nsl + sl) * kWinCap + below;
    for (int e0 = j; e0 < int(cnt); e0 += 8 * 16) {  // eight independent loads per round trip
      uint64_t pq[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) pq[k] = e0 + 16 * k < int(cnt) ? el[e0 + 16 * k] : 0ull;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc += residual(uint32_t(pq[k] >> 32), uint32_t(pq[k]), S_Q, gamma, false);
    }
  }
  acc = row16_sum_u128(acc);
  if (sl < nsl && j == 0) ssl[sl] = u128(S_Q) * fp - u128(gamma) * fq + acc;
  __syncthreads();
  u128 W = 0;
  for (int i = 0; i < nsl; ++i) W += ssl[i];
  return W;
}

// Residual masses under gamma from a pass of the deciding block over the row (outside the window): slice by
// slice, each wave sums its share and one thread adds the four shares in order (one barrier per slice,
// alternating LDS buffers); per-slice masses go to ssl (the first kThreads) and to smass, the total to W_out
template <bool VEC, bool LG>
__device__ __forceinline__ void row_mass(const VerifyWs& w, const VerifyArgs& a, size_t node, const float* prow,
                                         const float* qrow, const ProbRow<LG>& pr, uint64_t S_Q, uint64_t gamma,
                                         u128* ssl, u128 (*part)[kWaves], u128* W_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nsl = a.nsl, V = a.V;
  u128 total = 0;
  for (int sl = 0; sl < nsl; ++sl) {
    const int lo = sl * kSampleSlice, hi = min(V, lo + kSampleSlice);
    uint64_t sp = 0, sq = 0;  // sums of P and Q over the elements with a positive residual (res_sum)
    slice_for<VEC>(prow, qrow, lo, hi, [&] { return pr; }, [&](int, float x, float y) {
      const uint32_t P = fx(x), Q = fx(y);
      const bool pos = res_pos(P, Q, S_Q, gamma, false);
      sp += pos ? P : 0u;
      sq += pos ? Q : 0u;
    });
    sp = wave_sum_u64(sp);
    sq = wave_sum_u64(sq);
    if (lane == 0) part[sl & 1][wave] = (u128(sq) << 64) | sp;
    __syncthreads();
    if (tid == 0) {
      uint64_t SPs = 0, SQs = 0;
      for (int i = 0; i < kWaves; ++i) {
        SPs += uint64_t(part[sl & 1][i]);
        SQs += uint64_t(part[sl & 1][i] >> 64);
      }
      const u128 m = res_sum(SPs, SQs, S_Q, gamma, false);
      if (sl < kThreads) ssl[sl] = m;
      uint64_t* sm = w.smass + (node * nsl + sl) * 2;  // read by the block that walks the tree
      st_agent(sm, uint64_t(m));
      st_agent(sm + 1, uint64_t(m >> 64));
      total += m;
    }
  }
  if (tid == 0) *W_out = total;
  __syncthreads();
}

template <bool VEC, bool LG>
__device__ __forceinline__ void decide_node(const VerifyWs& w, const VerifyArgs& a, int b, int u, int T) {
  __shared__ int kid_s[kMaxKids], nkid_s;
  __shared__ uint64_t kpq_s[kMaxKids];  // children: (fx(p[t]) << 32) | fx(q[t]), ~0 = invalid token
  __shared__ uint64_t km_s[kMaxKids];   // node c's acceptance integer m at km_s[c - 1]
  __shared__ int act_s;  // accepted child; -1: a rejection needs the next residual mass; -2: resample
  __shared__ int fast_s, fastok_s, ki_s, tested_s, test_s, src_s;
  __shared__ u128 W_s, part_s[2][kWaves];
  __shared__ uint64_t SP_s, SQ_s, gamma_s, K_s;
  __shared__ uint32_t flags_s;
  __shared__ int plain_s;
  __shared__ u128 ssl_s[kThreads];  // per-slice masses of the current W (the first kThreads slices)
  __shared__ u128 wred_s[kWaves];
  __shared__ uint64_t red_s[kWaves][2];
  __shared__ WinLds win_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, max_T = a.max_T, V = a.V;
  const size_t node = size_t(b) * max_T + u;
  const float* prow = sample_row(a, node);
  const ProbRow<LG> pr = prob_row<LG>(a, node);

  // ---- one round trip: every slice's sums, the node's children, and (a node that may test children) its
  // window records; meanwhile wave 1 draws the uniforms of every potential child and wave 2 the node's own
  // resampling uniform
  const int qr = a.q_row ? a.q_row[node] : -1;
  const bool may_win = a.fast && w.wcnt != nullptr && qr >= 0 && qr < a.R && a.draft != nullptr;
  if (may_win) win_load(w, a, node, win_s);
  uint64_t sp = 0, sq = 0, nanb = 0;
  for (int sl = tid; sl < a.nsl; sl += kThreads) {
    const size_t r = node * a.nsl + sl;
    const uint64_t v = w.ssum[r];
    const uint64_t* p2 = w.psum + r * 2;
    if (sl < kThreads) ssl_s[sl] = u128(v);
    sp += v;
    sq += p2[0];
    nanb |= p2[1];
  }
  int c_kid = 0, c_tok = -1;  // wave 0, lane l: the tree's node l + 1 if it is a child of u, its token
  if (wave == 0) {
    const int c = lane + 1;
    if (c < T) {
      int pc = a.parents[size_t(b) * max_T + c];
      if (pc < 0 || pc >= c) pc = 0;
      c_kid = pc == u;
      c_tok = a.tokens[size_t(b) * max_T + c];
    }
  } else if (wave == 1) {
    if (lane + 1 < T) {
      const U64x4 r = philox4x64_10(a.offset, uint64_t(b), uint64_t(lane + 1), 0, a.key0, a.key1);
      km_s[lane] = (r.w[0] >> 40) + 1;  // r = m / 2^24 in (0, 1]
    }
  } else if (wave == 2 && lane == 0) {
    const U64x4 r = philox4x64_10(a.offset, uint64_t(b), uint64_t(u), 0, a.key0, a.key1);
    K_s = r.w[1] >> 32;
  }
  // ---- reductions (sum, sum, max, or) and the child list in index order
  sp = wave_sum_u64(sp);
  sq = wave_sum_u64(sq);
  nanb = wave_or_u32(uint32_t(nanb));
  if (lane == 0) {
    wred_s[wave] = u128(sp);
    red_s[wave][0] = sq;
    red_s[wave][1] = nanb;
  }
  int kslot = -1;  // this lane's position in the child list
  if (wave == 0) {
    const uint64_t m = __ballot(c_kid);
    if (c_kid) {
      kslot = __popcll(m & ((1ull << lane) - 1));
      kid_s[kslot] = lane + 1;
    }
    if (lane == 0) nkid_s = __popcll(m);
  }
  __syncthreads();
  const int nkid = nkid_s;
  // the node's q row, or null if it has none (no children, no draft tensor, or q_row out of range)
  const float* qrow = (nkid > 0 && a.draft != nullptr && qr >= 0 && qr < a.R) ? a.draft + (size_t(b) * a.R + qr) * V : nullptr;
  if (wave == 0 && kslot >= 0) {  // the children's p and q at their tokens
    uint64_t pq = ~0ull;
    if (c_tok >= 0 && c_tok < V) pq = (uint64_t(fx(pr(prow[c_tok]))) << 32) | (qrow ? fx(qrow[c_tok]) : 0u);
    kpq_s[kslot] = pq;
  }
  __syncthreads();
  if (tid == 0) {
    uint64_t S_P = uint64_t(wred_s[0]);  // S_P < V 2^32 < 2^56
    for (int i = 1; i < kWaves; ++i) {
      S_P += uint64_t(wred_s[i]);
      sq += red_s[i][0];
      nanb |= red_s[i][1];
    }
    const uint64_t S_Q = qrow ? sq : 0;
    const bool test = nkid > 0 && qrow != nullptr && S_Q > 0;
    uint32_t flags = ((nanb & 1u) || ((nanb & 2u) && qrow)) ? SPEC_STATUS_NAN_INPUT : 0u;
    if (nkid > 0 && !test) flags |= SPEC_STATUS_ZERO_Q;
    SP_s = S_P;
    SQ_s = S_Q;
    W_s = u128(S_P) * S_Q;
    gamma_s = 0;
    flags_s = flags;
    ki_s = 0;
    tested_s = 0;
    test_s = test;
    src_s = 0;  // the per-slice masses are pass 0's sums of fx(p)
    fastok_s = test && may_win && !(nanb & kWinOverflow);
  }
  __syncthreads();
  // ---- the children in index order: the block tests them one after another (thread 0); after a rejection
  // the next residual mass comes from the window records when they admit the new gamma, else from a pass of
  // this block over the row
  for (;;) {
    if (tid == 0) {
      int act = -2, ki = ki_s, tst = tested_s;
      const u128 W = W_s;
      const uint64_t S_Q = SQ_s;
      uint64_t g = gamma_s;
      for (; test_s && ki < nkid; ++ki) {
        const int c = kid_s[ki];
        const uint64_t pq = kpq_s[ki];
        if (pq == ~0ull) continue;  // invalid draft token: never tested
        tst = 1;
        const uint32_t Pt = uint32_t(pq >> 32), Qt = uint32_t(pq);
        const u128 Nt = residual(Pt, Qt, S_Q, g, false);
        const uint64_t m = km_s[c - 1];
        bool accept = false;
        if (Nt > 0) {
          const U192 lhs = mul_u128_u64(W, m * uint64_t(Qt));  // m Q_t W
          const U192 rhs = shl_u192(mul_u128_u64(Nt, S_Q), 24);  // 2^24 N_t S_Q
          accept = le_u192(lhs, rhs);
        }
        if (accept) {
          act = c;
          break;
        }
        // rejected: residual <- norm(max(0, residual - q)), whose mass is needed next
        g = g + div_u128_u64(W, S_Q);
        act = -1;
        ++ki;
        break;
      }
      ki_s = ki;
      tested_s = tst;
      gamma_s = g;
      act_s = act;
      fast_s = act == -1 && fastok_s && win_admits(g, S_Q);
    }
    __syncthreads();
    if (act_s != -1) break;
    if (fast_s) {  // the mass (and every slice's share, for a resample) from the window records
      const u128 W = win_mass(w, a, node, SQ_s, gamma_s, win_s, ssl_s);
      if (tid == 0) {
        W_s = W;
        src_s = 1;
      }
    } else {
      row_mass<VEC, LG>(w, a, node, prow, qrow, pr, SQ_s, gamma_s, ssl_s, part_s, &W_s);
      if (tid == 0) src_s = 2;
    }
    if (tid == 0 && W_s == 0) flags_s |= SPEC_STATUS_ZERO_RESIDUAL;
    __syncthreads();
  }
  if (tid == 0) {
    plain_s = !tested_s;
    if (!tested_s) W_s = u128(SP_s);
  }
  __syncthreads();
  if (act_s >= 0) {
    sample_finish<VEC, LG>(w, a, b, u, act_s, flags_s, false);
    return;
  }
  // ---- no draft accepted: the bonus is drawn only if the walk stops at this node, by the block that walks the
  // tree (resample_stop); publish what it needs: the final residual mass W, gamma, S_Q, the node's uniform K,
  // whether anything was tested, and where the per-slice masses are (pass 0's sums of fx(p) in
  // ssum, or smass: this block's row pass wrote it; window masses are written there now)
  if (src_s == 1 && tid < a.nsl) {
    uint64_t* sm = w.smass + (node * a.nsl + tid) * 2;
    st_agent(sm, uint64_t(ssl_s[tid]));
    st_agent(sm + 1, uint64_t(ssl_s[tid] >> 64));
  }
  if (tid == 0) {
    uint64_t* rs = w.rstate + node * kRs;
    const u128 W = W_s;
    st_agent(rs, uint64_t(W));
    st_agent(rs + 1, uint64_t(W >> 64));
    st_agent(rs + 2, gamma_s);
    st_agent(rs + 3, SQ_s);
    st_agent(rs + 4, K_s);
    st_agent(rs + 5, uint64_t(plain_s ? 1u : 0u) | (uint64_t(src_s == 0 ? 0u : 2u) << 8));
  }
  wait_global_stores();
  __syncthreads();  // every thread's stores are complete before the ticket
  sample_finish<VEC, LG>(w, a, b, u, -1, flags_s, false);
}

// The smallest index among the largest fx(p) of a node's row (key fx(p) << 32 | ~index, maximum over the row), in
// one pass of the block over the row: the bonus when the residual is zero, the only time it is needed. Every
// thread calls it; the index is returned to every thread.
template <bool VEC, bool LG>
__device__ __forceinline__ int row_argmax(const VerifyArgs& a, size_t node) {
  __shared__ uint64_t am_s[kWaves];
  const float* prow = sample_row(a, node);
  const auto pre = [&] { return prob_row<LG>(a, node); };
  uint64_t am = 0;
  for (int lo = 0; lo < a.V; lo += kSampleSlice)
    slice_for<VEC>(prow, nullptr, lo, min(a.V, lo + kSampleSlice), pre, [&](int v, float x, float) {
      const uint64_t k = (uint64_t(fx(x)) << 32) | uint64_t(0xffffffffu - uint32_t(v));
      am = k > am ? k : am;
    });
  am = wave_max_u64(am);
  __syncthreads();  // every earlier use of am_s is done
  if ((threadIdx.x & (kWave - 1)) == 0) am_s[threadIdx.x / kWave] = am;
  __syncthreads();
  for (int i = 0; i < kWaves; ++i) am = am_s[i] > am ? am_s[i] : am;
  return int(0xffffffffu - uint32_t(am));
}

// The bonus of a sampling sequence whose accepted chain stops at node u, drawn by the block that walks the tree
// from the state u's deciding block published: from the residual after u's rejections (or from p if u tested
// nothing) with u's resampling uniform K, i.e. the smallest v with 2^32 prefix(v) > K W (prefix of the residual
// masses in index order); the slice from the per-slice masses, then one pass over that slice. Every thread calls
// it; the token is returned to every thread.
template <bool VEC, bool LG>
__device__ __forceinline__ int resample_stop(const VerifyWs& w, const VerifyArgs& a, int b, int u) {
  __shared__ u128 W_s, tau_s, run_s, grem_s, wtot_s[kWaves], ssl_s[kThreads];
  __shared__ uint64_t gsp_s[kWaves][kSampleSlice / (4 * kThreads)], gsq_s[kWaves][kSampleSlice / (4 * kThreads)];
  __shared__ uint64_t gamma_s, SQ_s;
  __shared__ int plain_s, src_s, found_s, grp_s, bonus_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, V = a.V;
  const size_t node = size_t(b) * a.max_T + u;
  // the first kThreads slices' masses from both possible sources, in the state's round trip (the state says which)
  uint64_t m0 = 0, m1 = 0, m2 = 0;
  if (tid < a.nsl) {
    const size_t r = node * a.nsl + tid;
    m0 = w.ssum[r];
    m1 = ld_agent(w.smass + r * 2);
    m2 = ld_agent(w.smass + r * 2 + 1);
  }
  if (tid == 0) {
    const uint64_t* rs = w.rstate + node * kRs;
    const u128 W = u128(ld_agent(rs)) | (u128(ld_agent(rs + 1)) << 64);
    const uint64_t K = ld_agent(rs + 4);
    const uint64_t f = ld_agent(rs + 5);
    W_s = W;
    gamma_s = ld_agent(rs + 2);
    SQ_s = ld_agent(rs + 3);
    plain_s = int(f & 1u);
    src_s = int(f >> 8);
    // threshold: smallest v with 2^32 * prefix(v) > K W  <=>  prefix(v) > floor(K W / 2^32)
    const U192 kw = mul_u128_u64(W, K);
    tau_s = (u128(kw.hi) << 96) | (u128(kw.mid) << 32) | u128(kw.lo >> 32);
    run_s = 0;
    found_s = -1;
    bonus_s = -1;
  }
  __syncthreads();
  const u128 W = W_s;
  if (W == 0) return row_argmax<VEC, LG>(a, node);  // zero residual: smallest-index argmax of p
  const bool plain = __builtin_amdgcn_readfirstlane(plain_s) != 0;
  const float* prow = sample_row(a, node);
  const ProbRow<LG> pr = prob_row<LG>(a, node);
  const int qr = a.q_row ? a.q_row[node] : -1;
  const float* qrow = (!plain && a.draft != nullptr && qr >= 0 && qr < a.R) ? a.draft + (size_t(b) * a.R + qr) * V : nullptr;
  // the slice holding the threshold: per-slice masses kThreads at a time, one round trip per chunk
  for (int c0 = 0; c0 < a.nsl; c0 += kThreads) {
    __syncthreads();
    if (found_s >= 0) break;
    const int sl = c0 + tid;
    if (sl < a.nsl) {
      const size_t r = node * a.nsl + sl;
      if (c0 == 0)
        ssl_s[tid] = src_s == 0 ? u128(m0) : (u128(m1) | (u128(m2) << 64));
      else
        ssl_s[tid] = src_s == 0 ? u128(w.ssum[r]) : (u128(ld_agent(w.smass + r * 2)) | (u128(ld_agent(w.smass + r * 2 + 1)) << 64));
    }
    __syncthreads();
    if (tid == 0) {
      u128 run = run_s;
      const int n = min(kThreads, a.nsl - c0);
      for (int i = 0; i < n; ++i) {
        if (run + ssl_s[i] > tau_s) {
          found_s = c0 + i;
          break;
        }
        run += ssl_s[i];
      }
      if (found_s < 0 && c0 + n >= a.nsl) found_s = a.nsl - 1;  // unreachable with exact sums
      run_s = run;
    }
  }
  __syncthreads();
  // the block searches the chosen slice: coalesced loads (thread t holds elements lo + 4 t + 1024 i + k,
  // k < 4, of the slice's 8 groups of 1024), the groups' sums by wave reductions locate the group holding
  // the threshold, one block scan over that group's 256 chunks of 4 elements locates the chunk, and its
  // thread walks the 4 elements it holds
  const uint64_t S_Q = SQ_s, gamma = gamma_s;
  constexpr int NG = kSampleSlice / (4 * kThreads);
  const int lo = found_s * kSampleSlice, whi = min(V, lo + kSampleSlice);
  const u128 rem = tau_s - run_s;  // remaining threshold inside the slice
  // every load issued before any is used: addresses clamped into the row, elements past the slice masked
  float4 x[NG], y[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int v = lo + 4 * tid + 4 * kThreads * i;
    if (VEC) {
      const int vc = v + 4 <= whi ? v : lo;
      x[i] = *reinterpret_cast<const float4*>(prow + vc);
      y[i] = qrow ? *reinterpret_cast<const float4*>(qrow + vc) : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      float e[4], f[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int vk = v + k < whi ? v + k : lo;
        e[k] = prow[vk];
        f[k] = qrow ? qrow[vk] : 0.f;
      }
      x[i] = make_float4(e[0], e[1], e[2], e[3]);
      y[i] = make_float4(f[0], f[1], f[2], f[3]);
    }
  }
  // this thread's 4 elements of group i in fixed point (past the slice: P = Q = 0, no residual) and its sums of P
  // and Q over those with a positive residual. P = 0 is never positive and the fp32 test decides the rest
  // branch-free; an element it cannot decide (products within 1e-6 of each other, rare) is left out of the sums
  // and returned as bit k
  const float fS = float(S_Q), fG = float(gamma);
  auto fast = [&](float4 xv, float4 yv, int i, uint64_t& sp, uint64_t& sq) __attribute__((always_inline)) -> uint32_t {
    const float xs[4] = {xv.x, xv.y, xv.z, xv.w}, ys[4] = {yv.x, yv.y, yv.z, yv.w};
    uint32_t und = 0;
    sp = 0;
    sq = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool in = lo + 4 * tid + 4 * kThreads * i + k < whi;
      const uint32_t P = fx(in ? pr(xs[k]) : 0.f), Q = fx(in ? ys[k] : 0.f);  // fx(0) = 0
      const float fa = float(P) * fS, fc = float(Q) * fG;
      const bool pos = plain ? P != 0u : fa > fc * 1.000001f;
      sp += pos ? P : 0u;
      sq += pos ? Q : 0u;
      und |= (P != 0u && !pos && !(fa < fc * 0.999999f)) ? 1u << k : 0u;  // plain: pos == (P != 0)
    }
    return und;
  };
  // the undecided elements of group i (bits), reloaded from the row: each joins the sums when P S_Q > gamma Q
  auto settle = [&](uint32_t bits, int i, uint64_t& sp, uint64_t& sq) __attribute__((always_inline)) {
    for (; bits != 0u; bits &= bits - 1u) {
      const int v = lo + 4 * tid + 4 * kThreads * i + __builtin_ctz(bits);
      const uint32_t P = fx(pr(prow[v])), Q = qrow ? fx(qrow[v]) : 0u;
      if (mul64x32(S_Q, P) > mul64x32(gamma, Q)) {
        sp += P;
        sq += Q;
      }
    }
  };
  // per group: the wave's sums, four groups' P and Q sums per transposed reduction; undecided elements (bit
  // 4 i + k of amb) are added in a second, rare pass
  static_assert(NG % 4 == 0, "groups in fours");
  uint32_t amb = 0;
#pragma unroll
  for (int h = 0; h < NG; h += 4) {
    uint64_t gs[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) amb |= fast(x[h + i], y[h + i], h + i, gs[i], gs[4 + i]) << (4 * (h + i));
    const uint64_t tot = wave_sum8_u64(gs);
    const int j = lane >> 3;  // value j: the sum of P (j < 4) or of Q of group h + j % 4
    if ((lane & 7) == 0) {
      if (j < 4)
        gsp_s[wave][h + j] = tot;
      else
        gsq_s[wave][h + j - 4] = tot;
    }
  }
  if (__syncthreads_or(amb != 0u)) {
    for (int i = 0; i < NG; ++i) {
      uint64_t sp = 0, sq = 0;
      settle((amb >> (4 * i)) & 0xfu, i, sp, sq);
      sp = wave_sum_u64(sp);
      sq = wave_sum_u64(sq);
      if (lane == 0) {
        gsp_s[wave][i] += sp;
        gsq_s[wave][i] += sq;
      }
    }
    __syncthreads();
  }
  if (wave == 0) {  // group i's residual mass in lane i, an inclusive scan over the NG lanes, the first to pass rem
    u128 t = 0;
    if (lane < NG) {
      uint64_t sp = 0, sq = 0;
      for (int q = 0; q < kWaves; ++q) {
        sp += gsp_s[q][lane];
        sq += gsq_s[q][lane];
      }
      t = res_sum(sp, sq, S_Q, gamma, plain);
    }
    u128 incl = t;
#pragma unroll
    for (int o = 1; o < NG; o <<= 1) {
      const u128 up = shfl_up_u128(incl, o);
      if (lane >= o) incl += up;
    }
    const uint64_t over = __ballot(lane < NG && incl > rem);
    const int g = over ? __builtin_ctzll(over) : NG - 1;  // NG - 1: unreachable with exact sums
    if (lane == g) {
      grp_s = g;
      grem_s = rem - (incl - t);
    }
  }
  __syncthreads();
  const int g = __builtin_amdgcn_readfirstlane(grp_s);
  const u128 grem = grem_s;
  // group g's 4 elements of this thread, loaded again (just read, so from cache): holding all groups' registers
  // until g is known would cost the kernel an occupancy step
  float4 xg, yg;
  {
    const int v = lo + 4 * tid + 4 * kThreads * g;
    if (VEC) {
      const int vc = v + 4 <= whi ? v : lo;
      xg = *reinterpret_cast<const float4*>(prow + vc);
      yg = qrow ? *reinterpret_cast<const float4*>(qrow + vc) : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      float e[4], f[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int vk = v + k < whi ? v + k : lo;
        e[k] = prow[vk];
        f[k] = qrow ? qrow[vk] : 0.f;
      }
      xg = make_float4(e[0], e[1], e[2], e[3]);
      yg = make_float4(f[0], f[1], f[2], f[3]);
    }
  }
  uint64_t sp, sq;
  settle(fast(xg, yg, g, sp, sq), g, sp, sq);
  const u128 mine = res_sum(sp, sq, S_Q, gamma, plain);  // this thread's chunk of group g
  const u128 ex = block_exclusive_scan_u128(mine, wtot_s);
  if (mine > 0 && ex <= grem && grem < ex + mine) {
    const float xs[4] = {xg.x, xg.y, xg.z, xg.w}, ys[4] = {yg.x, yg.y, yg.z, yg.w};
    u128 run = ex;
    int hit = -1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int v = lo + 4 * tid + 4 * kThreads * g + k;
      const uint32_t P = fx(v < whi ? pr(xs[k]) : 0.f), Q = fx(v < whi ? ys[k] : 0.f);
      run += residual(P, Q, S_Q, gamma, plain);
      if (run > grem && hit < 0) hit = v;
    }
    bonus_s = hit;
  }
  __syncthreads();
  const int bn = bonus_s;
  return bn >= 0 ? bn : row_argmax<VEC, LG>(a, node);  // unreachable with exact sums; keeps the output defined
}

// ------------------------------------------------------------------ walk
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  return (uint64_t(uint32_t(__shfl(int(v >> 32), src))) << 32) | uint32_t(__shfl(int(v), src));
}

// Runs in wave 0 of the last block of sequence b to finish (node n in lane n - 1; the root's values are
// read by every lane); reads the other blocks' results with agent-scope loads, one round trip.
// Greedy: a node is accepted when its token is its parent's argmax and so is every node above it;
// validity (AND) and depth (sum) along the path come from pointer doubling over lanes, the deepest
// valid node (ties -> smaller index) from a wave maximum, and the path from its ancestry bits.
// Sampling: the accepted child chain from the root, chased in registers.
__device__ __forceinline__ void walk(const VerifyWs& w, const VerifyArgs& a, int b, int* stop_out = nullptr,
                                     int* nacc_out = nullptr) {
  __shared__ int path_s[65], tok_s[65];
  if (threadIdx.x >= kWave) return;
  const int lane = threadIdx.x, max_T = a.max_T, V = a.V;
  const int T = seq_T(a.T_b, b, max_T);
  const bool greedy = a.mode[b] != SPEC_MODE_SAMPLE;
  const size_t base = size_t(b) * max_T;
  const int n = lane + 1;
  const bool real = n < T;
  uint32_t f = 0;
  int par = 0, tok = 0;
  if (real) {
    par = a.parents[base + n];
    if (par < 0 || par >= n) {
      par = 0;
      f |= SPEC_STATUS_INVALID_PARENT;
    }
    tok = a.tokens[base + n];
    if (tok < 0 || tok >= V) f |= SPEC_STATUS_INVALID_TOKEN;
    tok_s[n] = tok;
  }
  if (lane == 0) path_s[0] = 0;
  int nacc, bonus;
  uint32_t rootf;
  if (greedy) {
    const uint64_t k0 = ld_agent(w.keys + base * kKS);
    const uint32_t rf0 = ld_agent(w.rowflag + base);
    uint64_t k = 0;
    uint32_t rf = 0;
    if (real) {
      k = ld_agent(w.keys + (base + n) * kKS);
      rf = ld_agent(w.rowflag + base + n);
    }
    const int am0 = int(0xffffffffu - uint32_t(k0)), am = int(0xffffffffu - uint32_t(k));
    if (rf) f |= SPEC_STATUS_NAN_INPUT;
    rootf = rf0 ? SPEC_STATUS_NAN_INPUT : 0u;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // every lane has read the root before it is cleared
    if (real) {  // leave the workspace zeroed
      st_agent(w.keys + (base + n) * kKS, uint64_t(0));
      st_agent(w.rowflag + base + n, 0u);
    }
    if (lane == 0) {
      st_agent(w.keys + base * kKS, uint64_t(0));
      st_agent(w.rowflag + base, 0u);
    }
    const int par_am = __shfl(am, par > 0 ? par - 1 : lane);
    int ok = real && tok >= 0 && tok < V && tok == (par > 0 ? par_am : am0);
    int dep = 1, jump = real ? par : 0;  // 0 = reached the root
    uint64_t anc = real ? (1ull << lane) : 0ull;
    while (__ballot(jump != 0)) {
      const int src = jump > 0 ? jump - 1 : lane;
      const int oj = __shfl(ok, src), dj = __shfl(dep, src), jj = __shfl(jump, src);
      const uint64_t aj = shfl_u64(anc, src);
      if (jump != 0) {
        ok &= oj;
        dep += dj;
        anc |= aj;
        jump = jj;
      }
    }
    // deepest valid node, ties -> smaller index; the root (depth 0, index 0) always qualifies
    const uint32_t key = (real && ok) ? (uint32_t(dep + 1) << 8) | uint32_t(255 - n) : 0u;
    const uint32_t best = max(uint32_t(wave_max_u64(key)), (1u << 8) | 255u);
    const int e = 255 - int(best & 255u);
    nacc = int(best >> 8) - 1;
    const uint64_t anc_e = shfl_u64(anc, e > 0 ? e - 1 : 0);
    if (e > 0 && real && ((anc_e >> lane) & 1)) path_s[dep] = n;
    bonus = e > 0 ? __shfl(am, e - 1) : am0;
  } else {
    const uint32_t nf0 = ld_agent(w.nflag + base);
    const int ch0 = ld_agent(w.acc_child + base);
    uint32_t nf = 0;
    int ch = -1;
    if (real) {
      nf = ld_agent(w.nflag + base + n);
      ch = ld_agent(w.acc_child + base + n);
    }
    f |= nf & SPEC_STATUS_NAN_INPUT;
    constexpr uint32_t kPathFlags = SPEC_STATUS_ZERO_Q | SPEC_STATUS_ZERO_RESIDUAL;
    rootf = nf0 & (SPEC_STATUS_NAN_INPUT | kPathFlags);
    int u = 0, c = ch0, cnt = 0;
    while (c > u && c < T && cnt < kWave) {  // uniform: every value comes from a readlane
      u = c;
      ++cnt;
      if (lane == 0) path_s[cnt] = u;
      rootf |= __builtin_amdgcn_readlane(nf, u - 1) & kPathFlags;
      c = __builtin_amdgcn_readlane(ch, u - 1);
    }
    nacc = cnt;
    bonus = -1;  // drawn at the stop node u by the caller (resample_stop), which writes it
    if (lane == 0) {
      *stop_out = u;
      *nacc_out = cnt;
    }
  }
  const uint32_t st = wave_or_u32(f) | rootf;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // path_s / tok_s written by other lanes
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane == 0) {
    a.accept_len[b] = nacc;
    a.status[b] = st;
  }
  for (int k = lane; k < max_T; k += kWave) {
    a.accept_nodes[base + k] = k <= nacc ? path_s[k] : -1;
    if (k != nacc || greedy) a.out_tokens[base + k] = k < nacc ? tok_s[path_s[k + 1]] : (k == nacc ? bonus : -1);
  }
}

// a node's outcome is final: publish it and count it for its sequence; the block finishing a sequence's last
// node walks the tree and then draws the bonus of the node where the accepted chain stops. Rows past T_b are
// counted without outcome (trivial).
template <bool VEC, bool LG>
__device__ __forceinline__ void sample_finish(const VerifyWs& w, const VerifyArgs& a, int b, int u, int acc, uint32_t flags,
                                              bool trivial) {
  __shared__ int last_s, stop_s, nacc_s;
  const size_t node = size_t(b) * a.max_T + u;
  if (threadIdx.x == 0) {
    if (!trivial) {
      st_agent(w.acc_child + node, acc);
      st_agent(w.nflag + node, flags);
    }
    wait_global_stores();
    last_s = ticket_add(&w.tickets[size_t(b) * kQ]) == uint32_t(a.max_T - 1);
  }
  __syncthreads();
  if (!last_s) return;
  if (threadIdx.x == 0) ticket_reset(&w.tickets[size_t(b) * kQ]);
  walk(w, a, b, &stop_s, &nacc_s);
  __syncthreads();
  const int bonus = resample_stop<VEC, LG>(w, a, b, stop_s);
  if (threadIdx.x == 0) a.out_tokens[size_t(b) * a.max_T + nacc_s] = bonus;
}

// The sampling sequences in index order into smap (when there are at most kMaxSampleMap); returns their count
__device__ __forceinline__ int sampling_map(const VerifyArgs& a, int* smap, int* wcnt) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  int nseq = 0;
  for (int b0 = 0; b0 < a.B; b0 += kThreads) {
    const int b = b0 + tid;
    const bool f = b < a.B && a.mode[b] == SPEC_MODE_SAMPLE;
    const uint64_t m = __ballot(f);
    if (lane == 0) wcnt[wave] = __popcll(m);
    __syncthreads();
    int off = nseq, tot = 0;
    for (int i = 0; i < kWaves; ++i) {
      off += i < wave ? wcnt[i] : 0;
      tot += wcnt[i];
    }
    off += __popcll(m & ((1ull << lane) - 1));
    if (f && off < kMaxSampleMap) smap[off] = b;
    nseq += tot;
    __syncthreads();
  }
  return nseq;
}

// sampling slice blocks of the rows kernel: the (node, slice) items of the sampling sequences, taken by a
// fixed stride (items numbered node-major over the listed sampling sequences when they fit, else over every
// sequence with the greedy ones skipped)
template <bool VEC, bool LG>
__device__ __forceinline__ void sample_slices(const VerifyWs& w, const VerifyArgs& a) {
  __shared__ int smap[kMaxSampleMap];
  __shared__ int wcnt[kWaves];
  __shared__ unsigned long long kids_s[kKidsSeqs][2];  // bit u: node u of listed sampling sequence i has a child
  const int nseq = sampling_map(a, smap, wcnt);
  if (nseq == 0) return;
  const bool mapped = nseq <= kMaxSampleMap;
  // which nodes have children (only their q rows and window records are ever read): one pass over the listed
  // sequences' parents (an invalid parent counts as the root, as in the decisions); more sequences than the
  // mask holds: every node counts as having children
  const int tid = threadIdx.x;
  const bool kmap = mapped && nseq <= kKidsSeqs;
  if (kmap) {
    for (int i = tid; i < 2 * nseq; i += kThreads) kids_s[i >> 1][i & 1] = 0ull;
    __syncthreads();
    for (int i = tid; i < nseq * a.max_T; i += kThreads) {
      const int si = i / a.max_T, c = i - si * a.max_T;
      const int b = smap[si];
      if (c >= 1 && c < seq_T(a.T_b, b, a.max_T)) {
        int pc = a.parents[size_t(b) * a.max_T + c];
        if (pc < 0 || pc >= c) pc = 0;
        atomicOr(&kids_s[si][pc >> 6], 1ull << (pc & 63));
      }
    }
    __syncthreads();
  }
  const long long items = (long long)(mapped ? nseq : a.B) * a.max_T * a.nsl;
  const int sb = a.sample_first ? int(blockIdx.x) : int(blockIdx.x) - a.n_greedy_blocks;
  for (long long it = sb; it < items; it += a.n_sample_blocks) {
    const int sl = int(it % a.nsl);
    const long long nd = it / a.nsl;
    const int u = int(nd % a.max_T), si = int(nd / a.max_T);
    const int b = mapped ? smap[si] : si;
    if (a.mode[b] != SPEC_MODE_SAMPLE || u >= seq_T(a.T_b, b, a.max_T)) continue;
    const bool kids = !kmap || ((kids_s[si][u >> 6] >> (u & 63)) & 1ull);
    sample_slice<VEC, LG>(w, a, b, u, sl, kids);
    __syncthreads();  // the slice's LDS is free for the next item
  }
}

// sampling slice blocks and greedy slice blocks; the sampling ones take the first ids when the call carries
// draft rows (their blocks run longest), else the last (a batch without draft rows is usually all greedy, and
// its sampling blocks only find that out)
template <bool VEC, bool LG>
__global__ void __launch_bounds__(kThreads) verify_rows_kernel(VerifyWs w, VerifyArgs a) {
  __shared__ int last_s;
  const bool sampling_block = a.sample_first ? int(blockIdx.x) < a.n_sample_blocks : int(blockIdx.x) >= a.n_greedy_blocks;
  if (sampling_block) {
    sample_slices<VEC, LG>(w, a);
    return;
  }
  const int gb = a.sample_first ? int(blockIdx.x) - a.n_sample_blocks : int(blockIdx.x);
  const int x = gb % a.n_slices, row = gb / a.n_slices;
  const int b = row / a.max_T, u = row - b * a.max_T;
  if (a.mode[b] == SPEC_MODE_SAMPLE) return;
  if (u < seq_T(a.T_b, b, a.max_T)) {
    if (a.slice == kGreedySlice)
      greedy_slice<VEC, kGreedySlice / (4 * kThreads)>(w, a, row, x * a.slice);
    else if (a.slice == 2 * kGreedySlice)
      greedy_slice<VEC, 2 * kGreedySlice / (4 * kThreads)>(w, a, row, x * a.slice);
    else
      greedy_slice<VEC, kGreedySliceMax / (4 * kThreads)>(w, a, row, x * a.slice);
  }
  // the block that completes the sequence walks its tree. With many slice blocks per sequence the
  // count has two levels, so no ticket takes more than max(n_slices, max_T) increments (one counter
  // took n_slices * max_T, over a thousand on a 65-node tree at V = 128256, and those same-address
  // atomics serialised): the last slice block of a row counts the row for its sequence. Each block's
  // argmax atomic has completed (vmcnt) before its row ticket, and a row's before its sequence ticket.
  // A few slice blocks per sequence share one counter (no second atomic round trip).
  wait_global_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    int last = 0;
    if (!a.row_tickets) {
      last = ticket_add(w.tickets + size_t(b) * kQ) == uint32_t(a.n_slices * a.max_T - 1);
    } else if (ticket_add(w.rtick + size_t(row) * kQ) == uint32_t(a.n_slices - 1)) {
      ticket_reset(w.rtick + size_t(row) * kQ);  // leave the workspace ready for the next call
      last = ticket_add(w.tickets + size_t(b) * kQ) == uint32_t(a.max_T - 1);
    }
    last_s = last;
  }
  __syncthreads();
  if (!last_s) return;
  if (threadIdx.x == 0) ticket_reset(w.tickets + size_t(b) * kQ);  // leave the workspace ready for the next call
  walk(w, a, b);
}

// one block per sampling node (the listed sampling sequences node by node, else every row with the greedy
// ones skipped); the rows kernel's slice results are complete at launch
template <bool VEC, bool LG>
__global__ void __launch_bounds__(kThreads) verify_decide_kernel(VerifyWs w, VerifyArgs a) {
  __shared__ int smap[kMaxSampleMap];
  __shared__ int wcnt[kWaves];
  const int nseq = sampling_map(a, smap, wcnt);
  const bool mapped = nseq <= kMaxSampleMap;
  const int i = blockIdx.x;
  if (i >= (mapped ? nseq : a.B) * a.max_T) return;
  const int si = i / a.max_T, u = i - si * a.max_T;
  const int b = mapped ? smap[si] : si;
  if (a.mode[b] != SPEC_MODE_SAMPLE) return;
  const int T = seq_T(a.T_b, b, a.max_T);
  if (u >= T) {
    sample_finish<VEC, LG>(w, a, b, u, -1, 0u, true);
    return;
  }
  decide_node<VEC, LG>(w, a, b, u, T);
}

// ------------------------------------------------------------------ probabilities from logits
// p = softmax(logits / T_b) of every sampling row (b, u < T_b) is never stored: softmax_partial_kernel
// takes each slice of kSmSlice elements to (max of x = l * (1 / T_b), sum of exp(x - max)), in a fixed
// order, and the sampling passes form p from the logits and the row's merged partials as they read it
// (ProbRow). A non-finite x stays out of the maximum and the sum; rows whose temperature is invalid have
// no partials.
constexpr int kSmThreads = 256;
constexpr int kSmPer = 32;                       // elements per thread
constexpr int kSmSlice = kSmThreads * kSmPer;    // elements per block

__device__ __forceinline__ float sm_block_reduce(float x, bool is_max, float* red) {
  constexpr int NW = kSmThreads / kWave;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float y = __shfl_xor(x, o, kWave);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  __syncthreads();  // the previous reduction's reads of red are done
  if (lane == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

__device__ __forceinline__ bool sm_row(const int32_t* T_b, const int8_t* mode, int max_T, int row) {
  const int b = row / max_T, u = row - b * max_T;
  return mode[b] == SPEC_MODE_SAMPLE && u < seq_T(T_b, b, max_T);
}

// VEC: each thread loads its 32 elements as 8 float4 (V a multiple of 4, logits 16-byte aligned), else
// one float per lane and load
template <bool VEC>
__global__ void __launch_bounds__(kSmThreads) softmax_partial_kernel(const float* logits, const float* temperature,
                                                                      const int32_t* T_b, const int8_t* mode,
                                                                      int max_T, int V, float2* part) {
  __shared__ float red[kSmThreads / kWave];
  const int s = blockIdx.x, row = blockIdx.y, nsl = gridDim.x, tid = threadIdx.x;
  if (!sm_row(T_b, mode, max_T, row)) return;
  const float T = sm_temperature(temperature, row / max_T);
  if (T == 0.f) return;  // no partials: every probability of the row is NaN
  const float inv = 1.f / T;
  const float* l = logits + size_t(row) * V;
  float x[kSmPer];
  if (VEC) {
#pragma unroll
    for (int i = 0; i < kSmPer / 4; ++i) {
      const int v = s * kSmSlice + 4 * (i * kSmThreads + tid);
      const float4 q = v < V ? *reinterpret_cast<const float4*>(l + v) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      x[4 * i] = q.x * inv;
      x[4 * i + 1] = q.y * inv;
      x[4 * i + 2] = q.z * inv;
      x[4 * i + 3] = q.w * inv;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kSmPer; ++i) {
      const int v = s * kSmSlice + i * kSmThreads + tid;
      x[i] = v < V ? l[v] * inv : -INFINITY;
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSmPer; ++i)
    if (isfinite(x[i])) m = fmaxf(m, x[i]);
  m = sm_block_reduce(m, true, red);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kSmPer; ++i)
    if (isfinite(x[i])) sum += exp_nonpos(x[i] - m);
  sum = sm_block_reduce(sum, false, red);
  if (tid == 0) part[size_t(row) * nsl + s] = make_float2(m, sum);
}

}  // namespace
}  // namespace spectree

using namespace spectree;

extern "C" size_t spec_tree_verify_workspace_size(int32_t B, int32_t max_T, int32_t V) {
  if (B < 1 || max_T < 1 || max_T > 65 || V < 1) return 0;
  size_t total = 0;
  carve(nullptr, 0, B, max_T, V, &total);
  return total;
}

// SPEC_TREE_VERIFY_FAST=0 (read at each call, for measurements and tests) takes every residual mass from a
// pass of the deciding block over the row, with no window records.
static int verify_fast_enabled() {
  const char* e = getenv("SPEC_TREE_VERIFY_FAST");
  return !(e && e[0] == '0' && e[1] == 0);
}

static int32_t verify_impl(const char* who, const float* target, float2* sm_part, const float* temperature,
                           const float* draft_probs, const int32_t* q_row,
                                    const int32_t* tokens, const int32_t* parents, const int32_t* T_b,
                                    const int8_t* mode, uint64_t philox_key0, uint64_t philox_key1,
                                    uint64_t philox_offset, int32_t B, int32_t max_T, int32_t R, int32_t V,
                                    int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens, uint32_t* status,
                                    void* ws, size_t ws_bytes, void* stream) {
  if (B < 1 || max_T < 1) return fail(SPEC_E_INVAL, "%s: B=%d max_T=%d", who, B, max_T);
  if (max_T > 65) return fail(SPEC_E_UNSUPPORTED, "%s: max_T=%d > 65", who, max_T);
  if (V < 1 || V >= (1 << 24)) return fail(SPEC_E_UNSUPPORTED, "%s: V=%d not in [1, 2^24)", who, V);
  if (draft_probs && (R < 1 || !q_row)) return fail(SPEC_E_INVAL, "%s: draft_probs needs R >= 1 and q_row", who);
  if (!target || !tokens || !parents || !mode || !accept_len || !accept_nodes || !out_tokens || !status)
    return fail(SPEC_E_INVAL, "%s: null pointer", who);
  const long long rows = (long long)B * max_T;
  const long long nsl = sample_slices(V);
  if (rows * nsl >= (1LL << 31)) return fail(SPEC_E_UNSUPPORTED, "%s: B*max_T*ceil(V/%d) too large", who, kSampleSlice);
  size_t need = 0;
  VerifyWs w = carve(ws, ws_bytes, B, max_T, V, &need);
  if (!ws || ws_bytes < need) return fail(SPEC_E_WORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 15) return fail(SPEC_E_INVAL, "%s: ws must be 16-byte aligned", who);
  // greedy slices of kGreedySlice elements (one round trip of loads per block), doubled or tripled when
  // the rows would otherwise need more blocks than a launch keeps resident (2 per CU at this kernel's
  // register count): a 65-node tree at V = 128256 takes 390 blocks of 24 K instead of 1040 of 8 K
  long long sl = kGreedySlice;
  while (sl < kGreedySliceMax && rows * ((V + sl - 1) / sl) > kGreedyBlocksTarget) sl += kGreedySlice;
  VerifyArgs a;
  a.target = target;
  a.sm_part = sm_part;
  a.temperature = temperature;
  a.sm_nsl = int((V + kSmSlice - 1) / kSmSlice);
  a.draft = draft_probs;
  a.q_row = q_row;
  a.tokens = tokens;
  a.parents = parents;
  a.T_b = T_b;
  a.mode = mode;
  a.key0 = philox_key0;
  a.key1 = philox_key1;
  a.offset = philox_offset;
  a.B = B;
  a.max_T = max_T;
  a.R = draft_probs ? R : 0;
  a.V = V;
  a.slice = int(sl);
  a.n_slices = int((V + sl - 1) / sl);
  a.nsl = int(nsl);
  a.n_greedy_blocks = int(rows) * a.n_slices;
  a.row_tickets = (long long)a.n_slices * max_T > 256;
  long long max_sblocks = kMaxSampleBlocks;
  if (const char* env = getenv("SPEC_TREE_VERIFY_SBLOCKS")) {  // sampling slice blocks per launch, for sweeps
    const long long v = atoll(env);
    if (v >= 256 && v <= (1LL << 20)) max_sblocks = v;
  }
  a.n_sample_blocks = int(std::min<long long>(max_sblocks, rows * nsl));
  a.sample_first = draft_probs != nullptr;
  a.fast = verify_fast_enabled();
  a.accept_len = accept_len;
  a.accept_nodes = accept_nodes;
  a.out_tokens = out_tokens;
  a.status = status;
  if ((long long)a.n_greedy_blocks + a.n_sample_blocks >= (1LL << 31))
    return fail(SPEC_E_UNSUPPORTED, "%s: grid too large", who);
  const bool vec = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(target) | reinterpret_cast<uintptr_t>(draft_probs)) & 15) == 0;
  const dim3 grid(a.n_greedy_blocks + a.n_sample_blocks);
  const dim3 dgrid{unsigned(rows), 1, 1};
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (sm_part) {  // the sampling rows' softmax partials first (same stream: the verify launches wait)
    const dim3 sgrid(unsigned(a.sm_nsl), unsigned(rows));
    if ((V % 4 == 0) && (reinterpret_cast<uintptr_t>(target) & 15) == 0)
      hipLaunchKernelGGL(softmax_partial_kernel<true>, sgrid, dim3(kSmThreads), 0, st, target, temperature, T_b, mode,
                         max_T, V, sm_part);
    else
      hipLaunchKernelGGL(softmax_partial_kernel<false>, sgrid, dim3(kSmThreads), 0, st, target, temperature, T_b, mode,
                         max_T, V, sm_part);
    if (vec) {
      hipLaunchKernelGGL((verify_rows_kernel<true, true>), grid, dim3(kThreads), 0, st, w, a);
      hipLaunchKernelGGL((verify_decide_kernel<true, true>), dgrid, dim3(kThreads), 0, st, w, a);
    } else {
      hipLaunchKernelGGL((verify_rows_kernel<false, true>), grid, dim3(kThreads), 0, st, w, a);
      hipLaunchKernelGGL((verify_decide_kernel<false, true>), dgrid, dim3(kThreads), 0, st, w, a);
    }
  } else if (vec) {
    hipLaunchKernelGGL((verify_rows_kernel<true, false>), grid, dim3(kThreads), 0, st, w, a);
    hipLaunchKernelGGL((verify_decide_kernel<true, false>), dgrid, dim3(kThreads), 0, st, w, a);
  } else {
    hipLaunchKernelGGL((verify_rows_kernel<false, false>), grid, dim3(kThreads), 0, st, w, a);
    hipLaunchKernelGGL((verify_decide_kernel<false, false>), dgrid, dim3(kThreads), 0, st, w, a);
  }
  return check_launch(who);
}

extern "C" int32_t spec_tree_verify(const float* target, const float* draft_probs, const int32_t* q_row,
                                    const int32_t* tokens, const int32_t* parents, const int32_t* T_b,
                                    const int8_t* mode, uint64_t philox_key0, uint64_t philox_key1,
                                    uint64_t philox_offset, int32_t B, int32_t max_T, int32_t R, int32_t V,
                                    int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens, uint32_t* status,
                                    void* ws, size_t ws_bytes, void* stream) {
  return verify_impl("spec_tree_verify", target, nullptr, nullptr, draft_probs, q_row, tokens, parents, T_b, mode, philox_key0,
                     philox_key1, philox_offset, B, max_T, R, V, accept_len, accept_nodes, out_tokens, status, ws,
                     ws_bytes, stream);
}

// the logits entry point's workspace: the verify workspace, then the slices' softmax partials at its very
// end (they need not start at zero); the verify part is everything below them
static size_t logits_part_bytes(int32_t B, int32_t max_T, int32_t V) {
  const size_t nsl = (size_t(V) + kSmSlice - 1) / kSmSlice;
  return align_up(size_t(B) * max_T * nsl * sizeof(float2), 256);
}

extern "C" size_t spec_tree_verify_logits_workspace_size(int32_t B, int32_t max_T, int32_t V) {
  const size_t verify = spec_tree_verify_workspace_size(B, max_T, V);
  return verify ? verify + logits_part_bytes(B, max_T, V) : 0;
}

extern "C" int32_t spec_tree_verify_logits(const float* logits, const float* temperature, const float* draft_probs,
                                           const int32_t* q_row, const int32_t* tokens, const int32_t* parents,
                                           const int32_t* T_b, const int8_t* mode, uint64_t philox_key0,
                                           uint64_t philox_key1, uint64_t philox_offset, int32_t B, int32_t max_T,
                                           int32_t R, int32_t V, int32_t* accept_len, int32_t* accept_nodes,
                                           int32_t* out_tokens, uint32_t* status, void* ws, size_t ws_bytes,
                                           void* stream) {
  const char* who = "spec_tree_verify_logits";
  if (B < 1 || max_T < 1) return fail(SPEC_E_INVAL, "%s: B=%d max_T=%d", who, B, max_T);
  if (max_T > 65) return fail(SPEC_E_UNSUPPORTED, "%s: max_T=%d > 65", who, max_T);
  if (V < 1 || V >= (1 << 24)) return fail(SPEC_E_UNSUPPORTED, "%s: V=%d not in [1, 2^24)", who, V);
  if ((long long)B * max_T > 65535) return fail(SPEC_E_UNSUPPORTED, "%s: B*max_T=%lld > 65535", who, (long long)B * max_T);
  const size_t need = spec_tree_verify_logits_workspace_size(B, max_T, V);
  if (!ws || ws_bytes < need) return fail(SPEC_E_WORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 15) return fail(SPEC_E_INVAL, "%s: ws must be 16-byte aligned", who);
  const size_t off = (ws_bytes - logits_part_bytes(B, max_T, V)) & ~size_t(255);
  float2* part = reinterpret_cast<float2*>(static_cast<char*>(ws) + off);
  return verify_impl(who, logits, part, temperature, draft_probs, q_row, tokens, parents, T_b, mode, philox_key0, philox_key1,
                     philox_offset, B, max_T, R, V, accept_len, accept_nodes, out_tokens, status, ws, off, stream);
}
