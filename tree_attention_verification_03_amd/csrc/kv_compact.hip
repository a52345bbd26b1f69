// Accepted-path KV compaction and the standalone tree-mask kernel.
//
// Compaction: tanhdev "Tech Radar: SGLang EAGLE-2", section 2 sequence diagram
// (retain the accepted path's KV, discard rejected branches); lesty.tech
// "EAGLE-2 & Lookahead Decoding", section 6 "Paged Tree KV-Cache Allocation".
// Node j's K/V sits at slot L_b + j; the k-th accepted draft moves to slot
// L_b + k. One block per (sequence, layer, KV head) loads every source row
// into LDS before it stores any destination, so overlapping moves are safe.
//
// Pruning: tanhdev section 4 "Production Failure Modes", Failure Mode 2 "KV
// Cache Memory Fragmentation" (discarded branches pruned without copies);
// lesty.tech section 6 (rejected candidates' blocks go back to the free pool).
// Only the page table changes: one wave per sequence rewrites its tree region
// and packs the released entries with a ballot prefix count.
//
// Mask: tanhdev section 2 "Dynamic Tree-Attention Verification" and section 5
// "FlashAttention-3 Tree Kernel Design" (one 64-bit ancestry word per node).
#include "api_common.h"
#include "spec_common.h"

namespace spectree {
namespace {

constexpr int kCompactThreads = 256;
constexpr int kMaskThreads = 128;
constexpr int kPruneThreads = 64;  // one wave: a tree has at most 64 drafts, and its tail at most 64 pages

template <int D>
__global__ void __launch_bounds__(kCompactThreads) kv_compact_kernel(uint16_t* k, uint16_t* v, const int32_t* page_table,
                                                                      const int32_t* prefix_lens, const int32_t* accept_nodes,
                                                                      const int32_t* accept_len, int max_T, int Hkv,
                                                                      int page_shift, int max_pages, int num_pages,
                                                                      int64_t layer_stride, int32_t* new_prefix_lens) {
  constexpr int CH = D / 8;  // 16-byte chunks per (slot, head) row
  __shared__ uint4 stage[2][64][CH];
  __shared__ int src_s[65], dst_s[65];
  __shared__ int n_s;
  const int b = blockIdx.x, layer = blockIdx.y, g = blockIdx.z, tid = threadIdx.x;
  const int cap = max_pages << page_shift;
  const int L = prefix_lens[b];
  int a = accept_len[b];
  const size_t base = size_t(b) * max_T;
  if (tid == 0) {
    bool ok = a >= 0 && a < max_T && L >= 0 && L + max_T <= cap;
    int prev = 0;
    for (int j = 1; ok && j <= a; ++j) {
      const int n = accept_nodes[base + j];
      ok = n > prev && n < max_T;
      prev = n;
    }
    n_s = ok ? a : 0;
    if (layer == 0 && g == 0) new_prefix_lens[b] = ok ? L + 1 + a : (L < 0 ? 0 : L);
  }
  __syncthreads();
  a = n_s;
  if (a == 0) return;
  if (tid < a) {
    const int j = tid + 1;
    const int ss = L + accept_nodes[base + j], ds = L + j;
    const int ps = page_table[size_t(b) * max_pages + (ss >> page_shift)];
    const int pd = page_table[size_t(b) * max_pages + (ds >> page_shift)];
    const bool ok = ps >= 0 && ps < num_pages && pd >= 0 && pd < num_pages;
    const int pm = (1 << page_shift) - 1;
    src_s[j] = ok ? ((ps << page_shift) | (ss & pm)) : -1;  // physical row index
    dst_s[j] = ok ? ((pd << page_shift) | (ds & pm)) : -1;
  }
  __syncthreads();
  const size_t row_stride = size_t(Hkv) * D;  // elements between physical rows
  uint16_t* kl = k + layer * layer_stride + size_t(g) * D;
  uint16_t* vl = v + layer * layer_stride + size_t(g) * D;
  for (int idx = tid; idx < a * CH; idx += kCompactThreads) {
    const int j = 1 + idx / CH, c = idx % CH;
    const int s = src_s[j];
    if (s < 0) continue;
    stage[0][j - 1][c] = reinterpret_cast<const uint4*>(kl + size_t(s) * row_stride)[c];
    stage[1][j - 1][c] = reinterpret_cast<const uint4*>(vl + size_t(s) * row_stride)[c];
  }
  __syncthreads();
  for (int idx = tid; idx < a * CH; idx += kCompactThreads) {
    const int j = 1 + idx / CH, c = idx % CH;
    const int s = src_s[j], d = dst_s[j];
    if (s < 0 || d < 0) continue;
    reinterpret_cast<uint4*>(kl + size_t(d) * row_stride)[c] = stage[0][j - 1][c];
    reinterpret_cast<uint4*>(vl + size_t(d) * row_stride)[c] = stage[1][j - 1][c];
  }
}

// REMAP (one slot per entry): lane i handles draft node i + 1; the k-th accepted node's entry moves to slot L + k.
// TAIL: lane i handles logical page ceil(L' / page) + i, which holds only rejected slots once the accepted KV has
// been compacted below L' = L + 1 + accept_len.
__global__ void __launch_bounds__(kPruneThreads) kv_prune_kernel(int32_t* page_table, const int32_t* prefix_lens,
                                                                  const int32_t* T_b, const int32_t* accept_nodes,
                                                                  const int32_t* accept_len, int max_T, int page_shift,
                                                                  int max_pages, int num_pages, int remap, int32_t* freed,
                                                                  int32_t* freed_count, int32_t* new_prefix_lens,
                                                                  uint32_t* status) {
  __shared__ int on_path[kPruneThreads + 1];
  const int b = blockIdx.x, lane = threadIdx.x;
  const int L = prefix_lens[b], T = T_b[b], a = accept_len[b];
  const size_t nb = size_t(b) * max_T;
  int32_t* row = page_table + size_t(b) * max_pages;
  const bool len_ok = T >= 1 && T <= max_T && L >= 0 && int64_t(L) + T <= (int64_t(max_pages) << page_shift);
  bool path_ok = len_ok && a >= 0 && a <= T - 1;
  const int j = lane + 1;  // path position of this lane, and its draft node in REMAP
  int n = 0;
  if (path_ok && j <= a) n = accept_nodes[nb + j];
  int prev = __shfl_up(n, 1);
  if (lane == 0) prev = 0;
  path_ok = path_ok && __ballot(j <= a && !(prev < n && n < T)) == 0;
  if (!path_ok) {
    for (int i = lane; i < max_T; i += kPruneThreads) freed[nb + i] = -1;
    if (lane == 0) {
      new_prefix_lens[b] = L < 0 ? 0 : L;
      freed_count[b] = 0;
      if (status) status[b] = len_ok ? SPEC_STATUS_INVALID_PATH : SPEC_STATUS_INVALID_LENGTH;
    }
    return;
  }
  int32_t old = -1;
  bool put = false, bad = false;
  if (remap) {
    on_path[j] = 0;
    __syncthreads();
    if (j <= a) on_path[n] = 1;
    const bool in = j < T;
    if (in) old = row[L + j];
    __syncthreads();
    const int32_t moved = __shfl(old, (j <= a ? n : 1) - 1);  // the entry of accepted node n sits in lane n - 1
    if (j <= a)
      row[L + j] = moved;
    else if (in)
      row[L + j] = -1;
    bad = in && (old < 0 || old >= num_pages);
    put = in && !bad && !on_path[j];
  } else {
    const int first = (L + a + (1 << page_shift)) >> page_shift;  // ceil((L + 1 + a) / page)
    const int last = (L + T - 1) >> page_shift;
    const int pidx = first + lane;
    if (pidx <= last) {
      old = row[pidx];
      row[pidx] = -1;
      bad = old < 0 || old >= num_pages;
      put = !bad;
    }
  }
  const uint64_t mask = __ballot(put);
  const int cnt = __popcll(mask);
  if (put) freed[nb + __popcll(mask & ((1ull << lane) - 1))] = old;
  for (int i = cnt + lane; i < max_T; i += kPruneThreads) freed[nb + i] = -1;
  const bool any_bad = __ballot(bad) != 0;
  if (lane == 0) {
    new_prefix_lens[b] = L + 1 + a;
    freed_count[b] = cnt;
    if (status) status[b] = any_bad ? SPEC_STATUS_INVALID_PAGE : 0u;
  }
}

__global__ void __launch_bounds__(kMaskThreads) tree_mask_kernel(const int32_t* parents, const int32_t* T_b, int max_T,
                                                                  uint64_t* anc_mask, int32_t* depth, uint32_t* status) {
  __shared__ uint64_t anc_s[65];
  __shared__ int jmp_s[65], dep_s[65];
  __shared__ uint32_t bad_s;
  const int b = blockIdx.x, tid = threadIdx.x;
  int T = T_b ? T_b[b] : max_T;
  T = T < 1 ? 1 : (T > max_T ? max_T : T);
  if (tid == 0) bad_s = 0;
  __syncthreads();
  if (tid < T) {
    int p = 0;
    if (tid > 0) {
      p = parents[size_t(b) * max_T + tid];
      if (p < 0 || p >= tid) {
        p = 0;
        atomicOr(&bad_s, SPEC_STATUS_INVALID_PARENT);
      }
    }
    jmp_s[tid] = p;
    anc_s[tid] = tid > 0 ? (1ull << (tid - 1)) : 0ull;
    dep_s[tid] = tid > 0;
  }
  __syncthreads();
  for (int it = 0; it < 7; ++it) {
    uint64_t na = 0;
    int nj = 0, nd = 0;
    if (tid < T) {
      const int j = jmp_s[tid];
      na = anc_s[tid] | anc_s[j];
      nd = dep_s[tid] + dep_s[j];
      nj = jmp_s[j];
    }
    __syncthreads();
    if (tid < T) {
      anc_s[tid] = na;
      dep_s[tid] = nd;
      jmp_s[tid] = nj;
    }
    __syncthreads();
  }
  for (int i = tid; i < max_T; i += kMaskThreads) {
    const size_t o = size_t(b) * max_T + i;
    anc_mask[o] = i < T ? anc_s[i] : 0ull;
    if (depth) depth[o] = i < T ? dep_s[i] : 0;
  }
  if (status && tid == 0) status[b] = bad_s;
}

}  // namespace
}  // namespace spectree

using namespace spectree;

extern "C" int32_t spec_kv_compact(void* k_pages, void* v_pages, const int32_t* page_table, const int32_t* prefix_lens,
                                   const int32_t* accept_nodes, const int32_t* accept_len, int32_t B, int32_t max_T,
                                   int32_t Hkv, int32_t d, int32_t page, int32_t max_pages, int32_t num_pages,
                                   int32_t num_layers, int64_t layer_stride_elems, int32_t* new_prefix_lens,
                                   void* stream) {
  if (B < 1 || max_T < 1 || Hkv < 1 || max_pages < 1 || num_pages < 1 || num_layers < 1)
    return fail(SPEC_E_INVAL, "spec_kv_compact: sizes must be positive");
  if (max_T > 65) return fail(SPEC_E_UNSUPPORTED, "spec_kv_compact: max_T=%d > 65", max_T);
  if (d != 64 && d != 128) return fail(SPEC_E_UNSUPPORTED, "spec_kv_compact: head dim %d not in {64, 128}", d);
  if (!is_pow2(page) || page > 1024) return fail(SPEC_E_UNSUPPORTED, "spec_kv_compact: page %d not a power of two <= 1024", page);
  if (!k_pages || !v_pages || !page_table || !prefix_lens || !accept_nodes || !accept_len || !new_prefix_lens)
    return fail(SPEC_E_INVAL, "spec_kv_compact: null pointer");
  {  // new_prefix_lens is written while other blocks still read prefix_lens: the two must not overlap
    const uintptr_t n0 = reinterpret_cast<uintptr_t>(new_prefix_lens), p0 = reinterpret_cast<uintptr_t>(prefix_lens);
    const uintptr_t nb = sizeof(int32_t) * size_t(B);
    if (n0 < p0 + nb && p0 < n0 + nb) return fail(SPEC_E_INVAL, "spec_kv_compact: new_prefix_lens overlaps prefix_lens");
  }
  const int64_t pool_elems = int64_t(num_pages) * page * Hkv * d;
  if (num_layers > 1 && layer_stride_elems < pool_elems)
    return fail(SPEC_E_INVAL, "spec_kv_compact: layer_stride_elems %lld < pool size %lld", (long long)layer_stride_elems,
                (long long)pool_elems);
  if ((reinterpret_cast<uintptr_t>(k_pages) | reinterpret_cast<uintptr_t>(v_pages)) & 15 || (layer_stride_elems % 8))
    return fail(SPEC_E_INVAL, "spec_kv_compact: pools and layer stride must be 16-byte aligned");
  if (B > 65535 || Hkv > 65535 || num_layers > 65535) return fail(SPEC_E_UNSUPPORTED, "spec_kv_compact: grid too large");
  const dim3 grid(B, num_layers, Hkv);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int ps = ilog2(page);
  if (d == 64)
    hipLaunchKernelGGL(kv_compact_kernel<64>, grid, dim3(kCompactThreads), 0, st, static_cast<uint16_t*>(k_pages),
                       static_cast<uint16_t*>(v_pages), page_table, prefix_lens, accept_nodes, accept_len, max_T, Hkv, ps,
                       max_pages, num_pages, layer_stride_elems, new_prefix_lens);
  else
    hipLaunchKernelGGL(kv_compact_kernel<128>, grid, dim3(kCompactThreads), 0, st, static_cast<uint16_t*>(k_pages),
                       static_cast<uint16_t*>(v_pages), page_table, prefix_lens, accept_nodes, accept_len, max_T, Hkv, ps,
                       max_pages, num_pages, layer_stride_elems, new_prefix_lens);
  return check_launch("spec_kv_compact");
}

extern "C" int32_t spec_kv_prune(int32_t* page_table, const int32_t* prefix_lens, const int32_t* T_b,
                                 const int32_t* accept_nodes, const int32_t* accept_len, int32_t B, int32_t max_T,
                                 int32_t page, int32_t max_pages, int32_t num_pages, int32_t mode, int32_t* freed,
                                 int32_t* freed_count, int32_t* new_prefix_lens, uint32_t* status, void* stream) {
  if (B < 1 || max_T < 1 || max_pages < 1 || num_pages < 1)
    return fail(SPEC_E_INVAL, "spec_kv_prune: sizes must be positive (B=%d max_T=%d max_pages=%d num_pages=%d)", B, max_T,
                max_pages, num_pages);
  if (max_T > 65) return fail(SPEC_E_UNSUPPORTED, "spec_kv_prune: max_T=%d > 65", max_T);
  if (!is_pow2(page) || page > 1024) return fail(SPEC_E_UNSUPPORTED, "spec_kv_prune: page %d not a power of two <= 1024", page);
  if (mode != SPEC_PRUNE_TAIL && mode != SPEC_PRUNE_REMAP) return fail(SPEC_E_INVAL, "spec_kv_prune: mode %d", mode);
  if (mode == SPEC_PRUNE_REMAP && page != 1)
    return fail(SPEC_E_INVAL, "spec_kv_prune: SPEC_PRUNE_REMAP needs one slot per page-table entry (page %d)", page);
  if ((long long)max_pages * page > (1LL << 30)) return fail(SPEC_E_UNSUPPORTED, "spec_kv_prune: more than 2^30 slots per sequence");
  if (!page_table || !prefix_lens || !T_b || !accept_nodes || !accept_len || !freed || !freed_count || !new_prefix_lens)
    return fail(SPEC_E_INVAL, "spec_kv_prune: null pointer");
  hipLaunchKernelGGL(kv_prune_kernel, dim3(B), dim3(kPruneThreads), 0, static_cast<hipStream_t>(stream), page_table,
                     prefix_lens, T_b, accept_nodes, accept_len, max_T, ilog2(page), max_pages, num_pages,
                     mode == SPEC_PRUNE_REMAP ? 1 : 0, freed, freed_count, new_prefix_lens, status);
  return check_launch("spec_kv_prune");
}

extern "C" int32_t spec_tree_mask(const int32_t* parents, const int32_t* T_b, int32_t B, int32_t max_T,
                                  uint64_t* anc_mask, int32_t* depth, uint32_t* status, void* stream) {
  if (B < 1 || max_T < 1) return fail(SPEC_E_INVAL, "spec_tree_mask: B=%d max_T=%d", B, max_T);
  if (max_T > 65) return fail(SPEC_E_UNSUPPORTED, "spec_tree_mask: max_T=%d > 65", max_T);
  if (!parents || !anc_mask) return fail(SPEC_E_INVAL, "spec_tree_mask: null pointer");
  hipLaunchKernelGGL(tree_mask_kernel, dim3(B), dim3(kMaskThreads), 0, static_cast<hipStream_t>(stream), parents, T_b,
                     max_T, anc_mask, depth, status);
  return check_launch("spec_tree_mask");
}
