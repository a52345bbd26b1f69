// Tree attention over a paged prefix KV cache plus each node's ancestors.
//
// Computes, for every sequence b, query head h and tree node i < T_b, softmax
// attention of q[b, i, h] over all prefix slots 0..L_b-1 and over the tree
// slots L_b + j for the root, the ancestors of i and i itself (tanhdev "Tech
// Radar: SGLang EAGLE-2", section 2 "Dynamic Tree-Attention Verification";
// section 5 "FlashAttention-3 Tree Kernel Design": 64-bit ancestry word per
// node, no K x K mask in HBM).
//
// Work decomposition (one launch):
//   grid.z = (b, kv head g); grid.y = block of up to 64 packed rows; grid.x =
//   prefix chunk s (keys [s*chunk, min((s+1)*chunk, L_b))) or, for the last x,
//   the tree slots [L_b, L_b + T_b).
//   Rows r = i * G + h' pack the G query heads sharing KV head g with the tree
//   nodes, so every K/V tile fetched from HBM serves all G*T rows of (b, g).
//   Each of the 4 waves takes 32-key sub-tiles of the item's range:
//     S^T = K Q^T  : bf16 MFMA 16x16x32, keys are the A operand (rows), so K
//                    goes from HBM straight into the A registers (8 consecutive
//                    head-dim elements per lane = one 16-byte load);
//     online softmax on S^T columns (each lane owns one query row; row max
//                    across the 4 lanes sharing it via two xor-shuffles);
//     O^T += V^T P^T: P^T is the S^T accumulator re-packed to bf16 in place
//                    (keys permuted identically in both operands), V^T is read
//                    from a per-wave LDS copy of the V sub-tile.
//   Waves merge (m, l, O) in LDS in fixed order; the item writes its partial
//   to the workspace; the last item of (b, g, row block) to arrive (atomic
//   ticket) merges all partials in fixed item order and writes out / lse.
//   Run-to-run deterministic; no float atomics.
#include "api_common.h"
#include "spec_common.h"

namespace spectree {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kSubKeys = 32;  // keys per wave sub-tile
constexpr int kMaxItems = 64; // prefix chunks + the tree item, per (b, g, row block)

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* page_table;
  const int32_t* prefix_lens;
  const int32_t* parents;
  const int32_t* T_b;
  uint16_t* out;
  float* lse;
  uint32_t* status;
  float* part;
  uint32_t* tickets;
  int max_T, Hq, Hkv, G;
  int page_shift, max_pages, num_pages;
  int chunk, n_splits, n_rb;
  float scale_log2;
};

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const uint16_t (&e)[8]) {
  uint4 u;
  u.x = uint32_t(e[0]) | (uint32_t(e[1]) << 16);
  u.y = uint32_t(e[2]) | (uint32_t(e[3]) << 16);
  u.z = uint32_t(e[4]) | (uint32_t(e[5]) << 16);
  u.w = uint32_t(e[6]) | (uint32_t(e[7]) << 16);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D, int RT>
__global__ void __launch_bounds__(kThreads) tree_attn_kernel(AttnParams p) {
  constexpr int KK = D / 32;       // MFMA k-steps over the head dim
  constexpr int DT = D / 16;       // 16-wide head-dim tiles of O^T
  constexpr int ROWS = RT * 16;    // packed rows per block
  constexpr int VROW = D + 4;      // LDS row stride of a V sub-tile (elements); +8 B staggers banks
  constexpr int OROW = D + 4;      // LDS row stride of the merged O (floats)
  constexpr int ITEM = ROWS * D + 2 * ROWS;  // floats per partial: O[ROWS][D], m[ROWS], l[ROWS]
  constexpr int V_BYTES = 4 * kSubKeys * VROW * 2;
  constexpr int O_BYTES = ROWS * OROW * 4;
  constexpr int W_BYTES = kMaxItems * ROWS * 4 * 3;  // merge weights + staged (m, l)
  constexpr int SMEM = V_BYTES > O_BYTES ? (V_BYTES > W_BYTES ? V_BYTES : W_BYTES)
                                         : (O_BYTES > W_BYTES ? O_BYTES : W_BYTES);
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  __shared__ float red_m[4][ROWS], red_l[4][ROWS];
  __shared__ float row_m[ROWS], row_l[ROWS];
  __shared__ uint64_t anc_s[65];
  __shared__ int par_s[65];
  __shared__ int flag_s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.x, rb = blockIdx.y, bg = blockIdx.z;
  const int b = bg / p.Hkv, g = bg - b * p.Hkv;

  int T = p.T_b ? p.T_b[b] : p.max_T;
  T = min(max(T, 1), p.max_T);
  int L = p.prefix_lens[b];
  const int cap = p.max_pages << p.page_shift;
  if (L < 0 || L > cap - T) {
    if (p.status && s == p.n_splits - 1 && rb == 0 && g == 0 && tid == 0)
      atomicOr(p.status + b, SPEC_STATUS_INVALID_LENGTH);
    L = min(max(L, 0), cap - T);
  }
  const int M = p.G * T;
  const int row0 = rb * ROWS;
  if (row0 >= M) return;
  const int nrows = min(ROWS, M - row0);
  const int nsp = (L + p.chunk - 1) / p.chunk;
  const bool is_tree = (s == p.n_splits - 1);
  if (!is_tree && s >= nsp) return;
  const int n_items = nsp + 1;
  const int key_lo = is_tree ? L : s * p.chunk;
  const int key_hi = is_tree ? L + T : min(L, key_lo + p.chunk);

  // ---- ancestry words of the tree nodes (pointer doubling, tree item only)
  if (is_tree) {
    if (tid < T) {
      int par = 0;
      uint64_t a = 0;
      if (tid > 0) {
        par = p.parents[size_t(b) * p.max_T + tid];
        if (par < 0 || par >= tid) {
          par = 0;
          if (p.status && rb == 0 && g == 0) atomicOr(p.status + b, SPEC_STATUS_INVALID_PARENT);
        }
        a = 1ull << (tid - 1);
      }
      par_s[tid] = par;
      anc_s[tid] = a;
    }
    __syncthreads();
#pragma unroll 1
    for (int it = 0; it < 7; ++it) {  // 2^7 > 64: every chain is covered
      uint64_t na = 0;
      int np = 0;
      if (tid < T) {
        const int pp = par_s[tid];
        na = anc_s[tid] | anc_s[pp];
        np = par_s[pp];
      }
      __syncthreads();
      if (tid < T) {
        anc_s[tid] = na;
        par_s[tid] = np;
      }
      __syncthreads();
    }
  }

  // ---- Q operands (B operand of S^T = K Q^T): lane holds row (lane & 15), 8 head-dim elements
  bf16x8 qop[RT][KK];
  uint64_t row_anc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = row0 + rt * 16 + (lane & 15);
    const bool ok = r < M;
    const int i = ok ? r / p.G : 0;
    const int h = g * p.G + (ok ? r - i * p.G : 0);
    const uint16_t* qp = p.q + ((size_t(b) * p.max_T + i) * p.Hq + h) * D + 8 * (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qop[rt][kk] = ok ? load_bf16x8(qp + 32 * kk) : bf16x8{};
    row_anc[rt] = (is_tree && ok) ? anc_s[i] : 0ull;
  }

  float m_run[RT], l_run[RT];
  f32x4 acc[RT][DT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  uint16_t* vs = reinterpret_cast<uint16_t*>(smem) + wave * kSubKeys * VROW;
  const int pmask = (1 << p.page_shift) - 1;
  const int32_t* ptab = p.page_table + size_t(b) * p.max_pages;
  const size_t tok_stride = size_t(p.Hkv) * D;
  const size_t page_stride = tok_stride << p.page_shift;
  const uint16_t* kbase = p.k + size_t(g) * D;
  const uint16_t* vbase = p.v + size_t(g) * D;
  const int g4 = 4 * (lane >> 4);
  bool bad_page = false;

#pragma unroll 1
  for (int st = key_lo + kSubKeys * wave; st < key_hi; st += 4 * kSubKeys) {
    // K tile: A operand, lane = key (lane & 15) of key tile kt, head-dim chunk 8*(lane>>4) + 32*kk
    bf16x8 kop[2][KK];
    uint32_t kvalid[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int slot = st + 16 * kt + (lane & 15);
      bool ok = slot < key_hi;
      const int phys = ok ? ptab[slot >> p.page_shift] : 0;
      if (ok && (phys < 0 || phys >= p.num_pages)) {
        ok = false;
        bad_page = true;
      }
      const uint16_t* kp = kbase + size_t(ok ? phys : 0) * page_stride + size_t(slot & pmask) * tok_stride + 8 * (lane >> 4);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kop[kt][kk] = ok ? load_bf16x8(kp + 32 * kk) : bf16x8{};
      kvalid[kt] = uint32_t(__ballot(ok) & 0xffffull);
    }
    // V sub-tile -> this wave's LDS slice, row-major [key][d]
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const int idx = lane + 64 * c;
      const int key = idx / (D / 8);
      const int dch = idx - key * (D / 8);
      const int slot = st + key;
      bool ok = slot < key_hi;
      const int phys = ok ? ptab[slot >> p.page_shift] : 0;
      ok = ok && phys >= 0 && phys < p.num_pages;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (ok)
        val = *reinterpret_cast<const uint4*>(vbase + size_t(phys) * page_stride + size_t(slot & pmask) * tok_stride + dch * 8);
      uint2* dst = reinterpret_cast<uint2*>(vs + key * VROW + dch * 8);
      dst[0] = make_uint2(val.x, val.y);
      dst[1] = make_uint2(val.z, val.w);
    }

    // S^T tiles: lane holds keys 16*kt + 4*(lane>>4) + j for query row (lane & 15) of tile rt
    f32x4 sc[2][RT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kt][kk], qop[rt][kk], a, 0, 0, 0);
        sc[kt][rt] = a;
      }

    // online softmax (base 2, scores pre-scaled by sm_scale*log2(e)); P rounded to bf16
    bf16x8 pop[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float sv[8];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kidx = g4 + j;
          bool vis = (kvalid[kt] >> kidx) & 1u;
          if (is_tree && vis) {
            const int jn = st + 16 * kt + kidx - L;  // tree node index of this key
            vis = (jn == 0) || ((row_anc[rt] >> (jn - 1)) & 1ull);
          }
          sv[kt * 4 + j] = vis ? sc[kt][rt][j] * p.scale_log2 : -INFINITY;
        }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float mnew = fmaxf(m_run[rt], mx);
      const bool none = (mnew == -INFINITY);
      const float alpha = none ? 1.f : fast_exp2(m_run[rt] - mnew);
      uint16_t pb[8];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = none ? 0.f : fast_exp2(sv[e] - mnew);
        pb[e] = f32_to_bf16(pe);
        psum += bf16_to_f32(pb[e]);
      }
      l_run[rt] = l_run[rt] * alpha + psum;
      m_run[rt] = mnew;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[rt][dt] *= alpha;
      pop[rt] = pack_bf16x8(pb);
    }

    // O^T += V^T P^T. A operand: lane holds head-dim row dt*16 + (lane & 15) and the same 8 keys
    // (4*(lane>>4) + {0..3}, 16 + 4*(lane>>4) + {0..3}) that the lane's P^T column holds.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int dcol = dt * 16 + (lane & 15);
      uint16_t ve[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ve[j] = vs[(g4 + j) * VROW + dcol];
        ve[4 + j] = vs[(16 + g4 + j) * VROW + dcol];
      }
      const bf16x8 vop = pack_bf16x8(ve);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[rt], acc[rt][dt], 0, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }

  if (bad_page && p.status) atomicOr(p.status + b, SPEC_STATUS_INVALID_PAGE);

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    l_run[rt] += __shfl_xor(l_run[rt], 16, kWave);
    l_run[rt] += __shfl_xor(l_run[rt], 32, kWave);
  }

  // ---- merge the 4 waves (fixed order)
  __syncthreads();
  if (lane < 16) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      red_m[wave][rt * 16 + lane] = m_run[rt];
      red_l[wave][rt * 16 + lane] = l_run[rt];
    }
  }
  __syncthreads();
  float fac[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + (lane & 15);
    float mx = red_m[0][row];
#pragma unroll
    for (int w = 1; w < 4; ++w) mx = fmaxf(mx, red_m[w][row]);
    float ls = 0.f, mine = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (red_m[w][row] == -INFINITY) ? 0.f : fast_exp2(red_m[w][row] - mx);
      ls += red_l[w][row] * f;
      if (w == wave) mine = f;
    }
    fac[rt] = mine;
    if (wave == 0 && lane < 16) {
      row_m[row] = mx;
      row_l[row] = ls;
    }
  }
  float* obuf = reinterpret_cast<float*>(smem);
#pragma unroll 1
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int row = rt * 16 + (lane & 15);
          float4* o = reinterpret_cast<float4*>(obuf + row * OROW + dt * 16 + g4);
          const f32x4 v4 = acc[rt][dt] * fac[rt];
          if (w == 0) {
            *o = make_float4(v4[0], v4[1], v4[2], v4[3]);
          } else {
            float4 t = *o;
            *o = make_float4(t.x + v4[0], t.y + v4[1], t.z + v4[2], t.w + v4[3]);
          }
        }
    }
    __syncthreads();
  }

  constexpr float kLn2 = 0.69314718055994530942f;
  if (n_items == 1) {  // no prefix: this item is the whole answer
    for (int idx = tid; idx < nrows * D; idx += kThreads) {
      const int row = idx / D, d = idx - row * D;
      const int r = row0 + row, i = r / p.G, h = g * p.G + (r - i * p.G);
      const float ls = row_l[row];
      const float o = ls > 0.f ? obuf[row * OROW + d] / ls : 0.f;
      p.out[((size_t(b) * p.max_T + i) * p.Hq + h) * D + d] = f32_to_bf16(o);
    }
    if (p.lse && tid < nrows) {
      const int r = row0 + tid, i = r / p.G, h = g * p.G + (r - i * p.G);
      const float ls = row_l[tid];
      p.lse[(size_t(b) * p.max_T + i) * p.Hq + h] = ls > 0.f ? (row_m[tid] + __log2f(ls)) * kLn2 : -INFINITY;
    }
    return;
  }

  // ---- publish this item's partial (write-through stores), then the last arrival merges all items
  float* const grp = p.part + (size_t(bg) * p.n_rb + rb) * size_t(p.n_splits) * ITEM;
  float* const mine = grp + size_t(s) * ITEM;
  constexpr int D2 = D / 2;
  for (int idx = tid; idx < nrows * D2; idx += kThreads) {
    const int row = idx / D2, c2 = idx - row * D2;
    const float2 v2 = *reinterpret_cast<const float2*>(obuf + row * OROW + 2 * c2);
    st_agent(reinterpret_cast<uint64_t*>(mine + row * D) + c2, __builtin_bit_cast(uint64_t, v2));
  }
  if (tid < nrows) {
    st_agent(mine + ROWS * D + tid, row_m[tid]);
    st_agent(mine + ROWS * D + ROWS + tid, row_l[tid]);
  }
  wait_global_stores();
  __syncthreads();
  uint32_t* ticket = p.tickets + size_t(bg) * p.n_rb + rb;
  if (tid == 0) flag_s = (ticket_add(ticket) == uint32_t(n_items - 1));
  __syncthreads();
  if (!flag_s) return;
  if (tid == 0) ticket_reset(ticket);  // leave the workspace ready for the next call

  // merge: stage every item's (m, l) in LDS with all threads, then weights, then O in float4 columns
  float* wts = reinterpret_cast<float*>(smem);                // [item][ROWS] normalised weights
  float* ml = wts + kMaxItems * ROWS;                         // [item][2][ROWS] raw (m, l)
  for (int idx = tid; idx < n_items * 2 * ROWS; idx += kThreads) {
    const int it = idx / (2 * ROWS), r2 = idx - it * 2 * ROWS;
    const int si = it < nsp ? it : p.n_splits - 1;
    ml[idx] = (r2 % ROWS) < nrows ? ld_agent(grp + size_t(si) * ITEM + ROWS * D + r2) : 0.f;
  }
  __syncthreads();
  if (tid < nrows) {
    float mx = -INFINITY;
    for (int it = 0; it < n_items; ++it) mx = fmaxf(mx, ml[it * 2 * ROWS + tid]);
    float ls = 0.f;
    for (int it = 0; it < n_items; ++it) {
      const float m = ml[it * 2 * ROWS + tid];
      const float f = (m == -INFINITY) ? 0.f : fast_exp2(m - mx);
      ls += ml[it * 2 * ROWS + ROWS + tid] * f;
      wts[it * ROWS + tid] = f;
    }
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
    for (int it = 0; it < n_items; ++it) wts[it * ROWS + tid] *= inv;
    if (p.lse) {
      const int r = row0 + tid, i = r / p.G, h = g * p.G + (r - i * p.G);
      p.lse[(size_t(b) * p.max_T + i) * p.Hq + h] = ls > 0.f ? (mx + __log2f(ls)) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();
  constexpr int D4 = D / 4;
  for (int idx = tid; idx < nrows * D4; idx += kThreads) {
    const int row = idx / D4, c4 = idx - row * D4;
    const float* src = grp + row * D + 4 * c4;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    int it = 0;
    for (; it + 4 <= n_items; it += 4) {  // four independent loads in flight per step
      float4 a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int si = (it + u) < nsp ? (it + u) : p.n_splits - 1;
        const uint64_t* q2 = reinterpret_cast<const uint64_t*>(src + size_t(si) * ITEM);
        const float2 lo2 = __builtin_bit_cast(float2, ld_agent(q2)), hi2 = __builtin_bit_cast(float2, ld_agent(q2 + 1));
        a[u] = make_float4(lo2.x, lo2.y, hi2.x, hi2.y);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wv = wts[(it + u) * ROWS + row];
        o.x += a[u].x * wv;
        o.y += a[u].y * wv;
        o.z += a[u].z * wv;
        o.w += a[u].w * wv;
      }
    }
    for (; it < n_items; ++it) {
      const int si = it < nsp ? it : p.n_splits - 1;
      const uint64_t* q2 = reinterpret_cast<const uint64_t*>(src + size_t(si) * ITEM);
      const float2 lo2 = __builtin_bit_cast(float2, ld_agent(q2)), hi2 = __builtin_bit_cast(float2, ld_agent(q2 + 1));
      const float4 a = make_float4(lo2.x, lo2.y, hi2.x, hi2.y);
      const float wv = wts[it * ROWS + row];
      o.x += a.x * wv;
      o.y += a.y * wv;
      o.z += a.z * wv;
      o.w += a.w * wv;
    }
    const int r = row0 + row, i = r / p.G, h = g * p.G + (r - i * p.G);
    uint16_t* dst = p.out + ((size_t(b) * p.max_T + i) * p.Hq + h) * D + 4 * c4;
    const uint32_t lo = uint32_t(f32_to_bf16(o.x)) | (uint32_t(f32_to_bf16(o.y)) << 16);
    const uint32_t hi = uint32_t(f32_to_bf16(o.z)) | (uint32_t(f32_to_bf16(o.w)) << 16);
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  }
}

struct AttnPlan {
  int G, RT, rows, n_rb, chunk, n_splits;
  size_t part_bytes, ticket_bytes;
};

AttnPlan make_plan(int B, int max_T, int Hq, int Hkv, int d, int page, int max_pages) {
  AttnPlan pl;
  pl.G = Hq / Hkv;
  const int M = pl.G * max_T;
  pl.RT = (M + 15) / 16;
  if (pl.RT > 4) pl.RT = 4;
  pl.rows = pl.RT * 16;
  pl.n_rb = (M + pl.rows - 1) / pl.rows;
  const long long slots = (long long)max_pages * page;
  const long long groups = (long long)B * Hkv * pl.n_rb;
  long long chunk = (slots * groups + 4095) / 4096;  // aim at ~4k work items
  if (chunk < 4LL * pl.rows) chunk = 4LL * pl.rows;  // keep partials small next to the KV they summarise
  chunk = (chunk + 127) / 128 * 128;
  if (chunk < 128) chunk = 128;
  if (chunk > 2048) chunk = 2048;
  if (const char* env = getenv("SPEC_TREE_ATTN_CHUNK")) {
    const long long c = atoll(env);
    if (c >= 128) chunk = c / 128 * 128;
  }
  while ((slots + chunk - 1) / chunk + 1 > kMaxItems) chunk += 128;
  pl.chunk = int(chunk);
  pl.n_splits = int((slots + chunk - 1) / chunk) + 1;
  const size_t item = size_t(pl.rows) * d + 2 * size_t(pl.rows);
  pl.part_bytes = align_up(size_t(groups) * pl.n_splits * item * sizeof(float), 256);
  pl.ticket_bytes = align_up(size_t(groups) * sizeof(uint32_t), 256);
  return pl;
}

template <int D>
void launch_d(const AttnPlan& pl, const AttnParams& prm, dim3 grid, hipStream_t st) {
  switch (pl.RT) {
    case 1: hipLaunchKernelGGL((tree_attn_kernel<D, 1>), grid, dim3(kThreads), 0, st, prm); break;
    case 2: hipLaunchKernelGGL((tree_attn_kernel<D, 2>), grid, dim3(kThreads), 0, st, prm); break;
    case 3: hipLaunchKernelGGL((tree_attn_kernel<D, 3>), grid, dim3(kThreads), 0, st, prm); break;
    default: hipLaunchKernelGGL((tree_attn_kernel<D, 4>), grid, dim3(kThreads), 0, st, prm); break;
  }
}

int32_t check_shapes(int32_t B, int32_t max_T, int32_t Hq, int32_t Hkv, int32_t d, int32_t page, int32_t max_pages) {
  if (B < 1 || max_T < 1 || Hq < 1 || Hkv < 1 || max_pages < 1 || page < 1)
    return fail(SPEC_E_INVAL, "spec_tree_attention: sizes must be positive (B=%d max_T=%d Hq=%d Hkv=%d page=%d max_pages=%d)",
                B, max_T, Hq, Hkv, page, max_pages);
  if (max_T > 65) return fail(SPEC_E_UNSUPPORTED, "spec_tree_attention: max_T=%d > 65 (root + 64 drafts)", max_T);
  if (Hq % Hkv) return fail(SPEC_E_INVAL, "spec_tree_attention: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if (Hq / Hkv > 16) return fail(SPEC_E_UNSUPPORTED, "spec_tree_attention: group size %d > 16", Hq / Hkv);
  if (d != 64 && d != 128) return fail(SPEC_E_UNSUPPORTED, "spec_tree_attention: head dim %d not in {64, 128}", d);
  if (!is_pow2(page) || page > 1024) return fail(SPEC_E_UNSUPPORTED, "spec_tree_attention: page %d not a power of two <= 1024", page);
  if ((long long)max_pages * page < max_T)
    return fail(SPEC_E_INVAL, "spec_tree_attention: page table holds %lld slots < max_T=%d", (long long)max_pages * page, max_T);
  if ((long long)max_pages * page > (1LL << 30)) return fail(SPEC_E_UNSUPPORTED, "spec_tree_attention: more than 2^30 slots per sequence");
  return SPEC_OK;
}

}  // namespace
}  // namespace spectree

using namespace spectree;

extern "C" size_t spec_tree_attention_workspace_size(int32_t B, int32_t max_T, int32_t Hq, int32_t Hkv, int32_t d,
                                                     int32_t page, int32_t max_pages) {
  if (check_shapes(B, max_T, Hq, Hkv, d, page, max_pages) != SPEC_OK) return 0;
  const AttnPlan pl = make_plan(B, max_T, Hq, Hkv, d, page, max_pages);
  return pl.part_bytes + pl.ticket_bytes;
}

extern "C" int32_t spec_tree_attention(const void* q, const void* k_pages, const void* v_pages, const int32_t* page_table,
                                       const int32_t* prefix_lens, const int32_t* parents, const int32_t* T_b, int32_t B,
                                       int32_t max_T, int32_t Hq, int32_t Hkv, int32_t d, int32_t page, int32_t max_pages,
                                       int32_t num_pages, float sm_scale, void* out, float* lse, uint32_t* status, void* ws,
                                       size_t ws_bytes, void* stream) {
  int32_t rc = check_shapes(B, max_T, Hq, Hkv, d, page, max_pages);
  if (rc != SPEC_OK) return rc;
  if (!q || !k_pages || !v_pages || !page_table || !prefix_lens || !parents || !out)
    return fail(SPEC_E_INVAL, "spec_tree_attention: null tensor pointer");
  if (num_pages < 1) return fail(SPEC_E_INVAL, "spec_tree_attention: num_pages=%d", num_pages);
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(SPEC_E_INVAL, "spec_tree_attention: sm_scale must be finite and > 0");
  const AttnPlan pl = make_plan(B, max_T, Hq, Hkv, d, page, max_pages);
  if (!ws || ws_bytes < pl.part_bytes + pl.ticket_bytes)
    return fail(SPEC_E_WORKSPACE, "spec_tree_attention: workspace %zu bytes < %zu", ws_bytes, pl.part_bytes + pl.ticket_bytes);
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pages) | reinterpret_cast<uintptr_t>(v_pages) |
       reinterpret_cast<uintptr_t>(ws)) & 15)
    return fail(SPEC_E_INVAL, "spec_tree_attention: q, k_pages, v_pages and ws must be 16-byte aligned");

  AttnParams prm;
  prm.q = static_cast<const uint16_t*>(q);
  prm.k = static_cast<const uint16_t*>(k_pages);
  prm.v = static_cast<const uint16_t*>(v_pages);
  prm.page_table = page_table;
  prm.prefix_lens = prefix_lens;
  prm.parents = parents;
  prm.T_b = T_b;
  prm.out = static_cast<uint16_t*>(out);
  prm.lse = lse;
  prm.status = status;
  prm.part = static_cast<float*>(ws);
  prm.tickets = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + pl.part_bytes);
  prm.max_T = max_T;
  prm.Hq = Hq;
  prm.Hkv = Hkv;
  prm.G = pl.G;
  prm.page_shift = ilog2(page);
  prm.max_pages = max_pages;
  prm.num_pages = num_pages;
  prm.chunk = pl.chunk;
  prm.n_splits = pl.n_splits;
  prm.n_rb = pl.n_rb;
  prm.scale_log2 = sm_scale * 1.4426950408889634f;
  const dim3 grid(pl.n_splits, pl.n_rb, B * Hkv);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (d == 64)
    launch_d<64>(pl, prm, grid, st);
  else
    launch_d<128>(pl, prm, grid, st);
  return check_launch("spec_tree_attention");
}
