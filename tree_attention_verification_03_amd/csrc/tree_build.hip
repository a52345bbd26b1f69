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
#include "api_common.h"
#include "spec_common.h"

namespace spectree {
namespace {

constexpr int kMaxTopk = 8;
constexpr int kMaxDepth = 16;
constexpr int kRowThreads = 256;
constexpr int kMaxSlices = 128;  // blocks per draft row (n_slices * max_topk <= 128 candidates per row)
constexpr int kBatch = 8 * 4 * kRowThreads;  // row elements whose loads a block issues together (8 float4 per thread)
constexpr int kFinishThreads = 256;

struct BuildWs {
  int32_t* tok;    // [B, P]
  int32_t* par;    // [B, P] parent pool index, -1 = root
  int32_t* depth;  // [B, P]
  int32_t* fslot;  // [B, P] frontier slot held at its own step, -1 if never frontier
  double* score;   // [B, P]
  int32_t* frontier;  // [B, max_topk] pool indices, rank order
  uint32_t* ticket;   // [B] blocks of the sequence's step that have finished
  uint64_t* cand;     // [B, max_topk, kMaxSlices, kMaxTopk] per-slice top-k keys
};

size_t pool_cap(int max_topk, int max_depth) {
  return size_t(max_topk) + size_t(max_depth - 1) * max_topk * max_topk;
}

BuildWs carve(void* ws, int B, int max_topk, int max_depth, size_t* total) {
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
  w.ticket = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * B));
  w.cand = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * B * max_topk * kMaxSlices * kMaxTopk));
  *total = off;
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

// Block-wide top-k (k <= 8) of row[lo, hi); results (rank order, 0 = none) in out_key[0..k).
template <bool VEC>
__device__ void block_slice_topk(const float* row, int lo, int hi, int k, uint64_t* out_key) {
  __shared__ uint64_t wtop[(kRowThreads / kWave) * kMaxTopk];
  uint64_t best[kMaxTopk];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) best[j] = 0;
  auto insert = [&](uint64_t key) {
    if (key > best[kMaxTopk - 1]) {
#pragma unroll
      for (int j = 0; j < kMaxTopk; ++j) {
        if (key > best[j]) {
          const uint64_t t = best[j];
          best[j] = key;
          key = t;
        }
      }
    }
  };
  if (VEC) {  // kBatch elements per round trip (a slice is normally one batch)
    for (int base = lo; base < hi; base += kBatch) {
      float4 xs[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int v = base + 4 * threadIdx.x + 4 * kRowThreads * i;
        xs[i] = v < hi ? *reinterpret_cast<const float4*>(row + v) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int v = base + 4 * threadIdx.x + 4 * kRowThreads * i;
        if (v >= hi) continue;
        insert(lp_key(xs[i].x, v));
        insert(lp_key(xs[i].y, v + 1));
        insert(lp_key(xs[i].z, v + 2));
        insert(lp_key(xs[i].w, v + 3));
      }
    }
  } else {
#pragma unroll 4
    for (int v = lo + threadIdx.x; v < hi; v += kRowThreads) insert(lp_key(row[v], v));
  }
  // each wave pops its own top k (wave maxima, no barriers; keys are unique, so exactly one lane owns
  // each maximum), then the block ranks the waves' 4k candidates: rank = number of larger candidates
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int r = 0; r < k; ++r) {
    const uint64_t m = wave_max_u64(best[0]);
    if (lane == 0) wtop[wave * kMaxTopk + r] = m;
    if (best[0] == m && m != 0) {
#pragma unroll
      for (int j = 0; j < kMaxTopk - 1; ++j) best[j] = best[j + 1];
      best[kMaxTopk - 1] = 0;
    }
  }
  if (threadIdx.x < k) out_key[threadIdx.x] = 0;  // fewer than k keys in the slice: the rest stay empty
  __syncthreads();
  constexpr int NWV = kRowThreads / kWave;
  if (threadIdx.x < NWV * k) {
    const int wv = threadIdx.x / k, r = threadIdx.x - wv * k;
    const uint64_t key = wtop[wv * kMaxTopk + r];
    int rank = 0;
    for (int o = 0; o < NWV * k; ++o) rank += wtop[(o / k) * kMaxTopk + o % k] > key;
    if (key != 0 && rank < k) out_key[rank] = key;  // nonzero keys are unique
  }
  __syncthreads();
}

// One kernel for every step. Block (slice x, frontier slot f, sequence b) reduces a slice of
// step-`step` draft row f to its top-k keys and publishes them; the last block of the sequence's
// step to finish (ticket) merges, in LDS, the slices of every row: at step 1 the root row fills the
// pool and the frontier; at step >= 2 the k rows' k children join the pool (score = parent score +
// log-prob, an fp64 left fold), the k*k children are ranked and the best k form the next frontier.
template <bool VEC>
__global__ void __launch_bounds__(kRowThreads) build_step_kernel(BuildWs w, int P, int step, const float* draft,
                                                                  int64_t seq_stride, const int32_t* topk,
                                                                  const int32_t* depth, int max_topk, int max_depth,
                                                                  int V, int slice, int32_t* frontier_tokens) {
  constexpr int kCand = 128;  // candidates per row (n_slices * k)
  __shared__ uint64_t keys[kMaxTopk];
  __shared__ uint64_t ck[kMaxTopk * kCand];     // [row][slice * k + j]
  __shared__ uint64_t top[kMaxTopk * kMaxTopk];  // [row][rank]
  __shared__ double csc[kMaxTopk * kMaxTopk];    // child scores [row * k + c]
  __shared__ int cpar[kMaxTopk];
  __shared__ int last;
  const int x = blockIdx.x, f = blockIdx.y, b = blockIdx.z;
  const int n_slices = gridDim.x;
  const int k = clamp_i(topk[b], 1, max_topk);
  const int D = clamp_i(depth[b], 1, max_depth);
  const int rows = step == 1 ? 1 : k;
  if (step > D || f >= rows) return;
  const float* row = draft + b * seq_stride + int64_t(f) * V;
  const int lo = x * slice, hi = min(V, lo + slice);
  uint64_t* cand = w.cand + ((size_t(b) * max_topk + f) * kMaxSlices + x) * kMaxTopk;
  block_slice_topk<VEC>(row, lo, hi, k, keys);
  if (threadIdx.x < k) st_agent(cand + threadIdx.x, keys[threadIdx.x]);
  wait_global_stores();
  __syncthreads();
  if (threadIdx.x == 0) last = (ticket_add(w.ticket + b) == uint32_t(n_slices * rows - 1));
  __syncthreads();
  if (!last) return;
  if (threadIdx.x == 0) ticket_reset(w.ticket + b);  // leave the workspace ready for the next step

  // every row's candidates (0 = empty), and at step >= 2 the rows' parents and their scores
  const int nc = n_slices * k;
  for (int i = threadIdx.x; i < rows * nc; i += kRowThreads) {
    const int r = i / nc, j = i - r * nc;
    ck[r * kCand + j] = ld_agent(w.cand + ((size_t(b) * max_topk + r) * kMaxSlices + j / k) * kMaxTopk + j % k);
  }
  const int base = k + (step - 2) * k * k;  // pool index of this step's first child (step >= 2)
  double psc = 0.0;
  if (step >= 2 && threadIdx.x < k) {
    cpar[threadIdx.x] = w.frontier[b * max_topk + threadIdx.x];
  }
  __syncthreads();
  // per row top-k: rank = number of larger keys (keys of one row are unique; 0 = empty)
  for (int i = threadIdx.x; i < rows * nc; i += kRowThreads) {
    const int r = i / nc;
    const uint64_t ki = ck[r * kCand + (i - r * nc)];
    if (ki == 0) continue;
    int rank = 0;
    for (int j = 0; j < nc; ++j) rank += ck[r * kCand + j] > ki;
    if (rank < k) top[r * kMaxTopk + rank] = ki;
  }
  if (step >= 2 && threadIdx.x < k * k) psc = w.score[size_t(b) * P + cpar[threadIdx.x / k]];
  __syncthreads();

  if (step == 1) {
    if (threadIdx.x < max_topk) {
      const int c = threadIdx.x;
      int tok = -1;
      if (c < k) {
        const size_t e = size_t(b) * P + c;
        tok = key_token(top[c]);
        w.tok[e] = tok;
        w.par[e] = -1;
        w.depth[e] = 1;
        w.fslot[e] = c;
        w.score[e] = 0.0 + double(key_value(top[c]));
        w.frontier[b * max_topk + c] = c;
      }
      frontier_tokens[b * max_topk + c] = tok;
    }
    return;
  }

  // children: row r's c-th best token becomes pool entry base + r * k + c
  const int n = k * k;
  if (threadIdx.x < n) {
    const int r = threadIdx.x / k, c = threadIdx.x - r * k;
    const uint64_t key = top[r * kMaxTopk + c];
    const size_t e = size_t(b) * P + base + threadIdx.x;
    const double sc = psc + double(key_value(key));
    csc[threadIdx.x] = sc;
    w.tok[e] = key_token(key);
    w.par[e] = cpar[r];
    w.depth[e] = step;
    w.score[e] = sc;
  }
  __syncthreads();
  // rank the k*k children: rank(c) = #children that beat c (higher score, ties -> smaller pool index)
  if (threadIdx.x < n) {
    const int c = threadIdx.x;
    const double sc = csc[c];
    int rank = 0;
    for (int o = 0; o < n; ++o) rank += (csc[o] > sc) || (csc[o] == sc && o < c);
    w.fslot[size_t(b) * P + base + c] = rank < k ? rank : -1;
    if (rank < k) {
      w.frontier[b * max_topk + rank] = base + c;
      frontier_tokens[b * max_topk + rank] = key_token(top[(c / k) * kMaxTopk + c % k]);
    }
  }
  if (threadIdx.x >= k && threadIdx.x < max_topk) frontier_tokens[b * max_topk + threadIdx.x] = -1;
}

__global__ void __launch_bounds__(kFinishThreads) build_finish_kernel(BuildWs w, int P, const int32_t* root_tokens,
                                                                       const int32_t* topk, const int32_t* depth,
                                                                       const int32_t* num_draft, int max_topk,
                                                                       int max_depth, int max_T, int32_t* tokens,
                                                                       int32_t* parents, int32_t* depth_out,
                                                                       uint64_t* anc_mask, int32_t* q_row) {
  constexpr int kPool = kMaxTopk + (kMaxDepth - 1) * kMaxTopk * kMaxTopk;
  __shared__ double sc[kPool];
  __shared__ int rank_s[kPool];  // pool rank, then node number (0 = not kept)
  __shared__ int par_e[kPool], dep_e[kPool], fs_e[kPool], tok_e[kPool];
  __shared__ int pool_of[65];
  __shared__ int node_par[65];
  __shared__ uint64_t anc_s[65];
  __shared__ int jump_s[65];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int k = clamp_i(topk[b], 1, max_topk);
  const int D = clamp_i(depth[b], 1, max_depth);
  const int pool = k + (D - 1) * k * k;
  const int N = clamp_i(num_draft[b], 1, min(pool, max_T - 1));
  const int T = N + 1;
  const size_t row = size_t(b) * P;

  // one round trip: every field of the pool
  for (int e = tid; e < pool; e += blockDim.x) {
    sc[e] = w.score[row + e];
    par_e[e] = w.par[row + e];
    dep_e[e] = w.depth[row + e];
    fs_e[e] = w.fslot[row + e];
    tok_e[e] = w.tok[row + e];
  }
  __syncthreads();
  for (int e = tid; e < pool; e += blockDim.x) {
    const double s = sc[e];
    int r = 0;
    for (int o = 0; o < pool; ++o) r += (sc[o] > s) || (sc[o] == s && o < e);
    rank_s[e] = r;
  }
  __syncthreads();
  // kept entries, numbered 1..N in pool order (wave 0 scans the pool 64 at a time)
  if (tid < kWave) {
    int base = 0;
    for (int c0 = 0; c0 < pool; c0 += kWave) {
      const int e = c0 + tid;
      const bool kept = e < pool && rank_s[e] < N;
      const uint64_t m = __ballot(kept);
      if (kept) pool_of[1 + base + __popcll(m & ((1ull << tid) - 1))] = e;
      base += __popcll(m);
    }
  }
  __syncthreads();
  if (tid >= 1 && tid < T) rank_s[pool_of[tid]] = -tid;  // kept entry -> -(node number)
  __syncthreads();
  // parents as node numbers: the parent entry of a kept entry is kept (scores never increase
  // down a path and the parent has the smaller pool index), so it carries a node number
  if (tid < T) {
    const int n = tid;
    int par_node = -1;
    if (n > 0) {
      const int pe = par_e[pool_of[n]];
      par_node = 0;
      if (pe >= 0 && rank_s[pe] < 0) par_node = -rank_s[pe];
    }
    node_par[n] = par_node;
    jump_s[n] = n > 0 ? par_node : 0;
    anc_s[n] = n > 0 ? (1ull << (n - 1)) : 0ull;
  }
  __syncthreads();
#pragma unroll 1
  for (int it = 0; it < 7; ++it) {
    uint64_t na = 0;
    int nj = 0;
    if (tid < T) {
      const int j = jump_s[tid];
      na = anc_s[tid] | anc_s[j];
      nj = jump_s[j];
    }
    __syncthreads();
    if (tid < T) {
      anc_s[tid] = na;
      jump_s[tid] = nj;
    }
    __syncthreads();
  }
  for (int n = tid; n < max_T; n += blockDim.x) {
    const size_t o = size_t(b) * max_T + n;
    if (n == 0) {
      tokens[o] = root_tokens[b];
      parents[o] = -1;
      depth_out[o] = 0;
      anc_mask[o] = 0;
      q_row[o] = 0;
    } else if (n < T) {
      const int e = pool_of[n];
      const int d = dep_e[e];
      const int fs = fs_e[e];
      tokens[o] = tok_e[e];
      parents[o] = node_par[n];
      depth_out[o] = d;
      anc_mask[o] = anc_s[n];
      q_row[o] = (fs >= 0 && d < D) ? 1 + (d - 1) * max_topk + fs : -1;
    } else {
      tokens[o] = -1;
      parents[o] = -1;
      depth_out[o] = 0;
      anc_mask[o] = 0;
      q_row[o] = -1;
    }
  }
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
  carve(nullptr, B, max_topk, max_depth, &total);
  return total;
}

extern "C" int32_t spec_tree_build_step(void* ws, size_t ws_bytes, int32_t step, const float* draft_logprobs,
                                        int64_t seq_stride, const int32_t* topk, const int32_t* depth, int32_t B,
                                        int32_t max_topk, int32_t max_depth, int32_t V, int32_t* frontier_tokens,
                                        void* stream) {
  int32_t rc = check_build("spec_tree_build_step", B, max_topk, max_depth);
  if (rc != SPEC_OK) return rc;
  if (step < 1 || step > max_depth) return fail(SPEC_E_INVAL, "spec_tree_build_step: step=%d not in [1, %d]", step, max_depth);
  if (V < max_topk || V >= (1 << 30)) return fail(SPEC_E_INVAL, "spec_tree_build_step: V=%d must be in [max_topk, 2^30)", V);
  if (!draft_logprobs || !topk || !depth || !frontier_tokens) return fail(SPEC_E_INVAL, "spec_tree_build_step: null pointer");
  const int64_t min_stride = (step == 1 ? 1 : max_topk) * int64_t(V);
  if (B > 1 && seq_stride < min_stride)
    return fail(SPEC_E_INVAL, "spec_tree_build_step: seq_stride=%lld < %lld", (long long)seq_stride, (long long)min_stride);
  size_t need = 0;
  BuildWs w = carve(ws, B, max_topk, max_depth, &need);
  if (!ws || ws_bytes < need) return fail(SPEC_E_WORKSPACE, "spec_tree_build_step: workspace %zu < %zu bytes", ws_bytes, need);
  const int P = int(pool_cap(max_topk, max_depth));
  hipStream_t st = static_cast<hipStream_t>(stream);
  // about 64 blocks per sequence and step, and slices of at most one load batch (8 K elements) where
  // possible; at most 128 / max_topk slices per row, so a row has <= 128 candidates; >= 1 K per slice
  const int max_sl = std::max(1, 128 / max_topk);
  const int rows = step == 1 ? 1 : max_topk;
  int n_slices = std::max(64 / rows, (V + kBatch - 1) / kBatch);
  n_slices = std::max(1, std::min(std::min(n_slices, max_sl), (V + 1023) / 1024));
  int slice = (V + n_slices - 1) / n_slices;
  slice = (slice + 1023) / 1024 * 1024;
  n_slices = (V + slice - 1) / slice;
  const dim3 grid(n_slices, step == 1 ? 1 : max_topk, B);
  const bool vec = (V % 4 == 0) && (seq_stride % 4 == 0) && ((reinterpret_cast<uintptr_t>(draft_logprobs) & 15) == 0);
  if (vec)
    hipLaunchKernelGGL(build_step_kernel<true>, grid, dim3(kRowThreads), 0, st, w, P, step, draft_logprobs, seq_stride,
                       topk, depth, max_topk, max_depth, V, slice, frontier_tokens);
  else
    hipLaunchKernelGGL(build_step_kernel<false>, grid, dim3(kRowThreads), 0, st, w, P, step, draft_logprobs, seq_stride,
                       topk, depth, max_topk, max_depth, V, slice, frontier_tokens);
  return check_launch("spec_tree_build_step");
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
  BuildWs w = carve(ws, B, max_topk, max_depth, &need);
  if (!ws || ws_bytes < need) return fail(SPEC_E_WORKSPACE, "spec_tree_build_finish: workspace %zu < %zu bytes", ws_bytes, need);
  const int P = int(pool_cap(max_topk, max_depth));
  hipLaunchKernelGGL(build_finish_kernel, dim3(B), dim3(kFinishThreads), 0, static_cast<hipStream_t>(stream), w, P,
                     root_tokens, topk, depth, num_draft, max_topk, max_depth, max_T, tokens, parents, depth_out,
                     anc_mask, q_row);
  return check_launch("spec_tree_build_finish");
}
