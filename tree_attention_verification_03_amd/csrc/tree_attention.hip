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
//   grid.z = (b, kv head g); grid.y = block of up to 48 packed rows; grid.x =
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
constexpr int kMaxChunk = 2048;
constexpr int kMergeItems = 32;  // items whose (m, l) the merge stages in LDS at a time
constexpr int kMaxPageIds = kMaxChunk + 2;  // page ids of one chunk (page size 1) or of the tree slots

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
  const uint16_t* zeros;  // a zero-filled (token, head) row in the workspace: target of masked loads
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair, hardware round-to-nearest-even
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// LDS address space pointer for the direct global->LDS loads
typedef __attribute__((address_space(3))) void lds_void;

// Chunk swizzle of a V row in LDS (16-byte chunks XOR 2 * (key & 3)): the transposed reads of four
// consecutive keys then hit 128 distinct bytes of banks.
template <int D>
__device__ __forceinline__ int v_swz(int key) {
  return 2 * (key & 3);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// gfx950 transposing LDS read: within each 16-lane group, lane i names a row of 4 consecutive
// 16-bit elements and lane l receives element (l % 4) of rows l/4, l/4 + 4, l/4 + 8, l/4 + 12.
__device__ __forceinline__ s16x4 lds_read_tr16(const unsigned char* addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(addr));
}

// single-stage variants rely on two blocks per CU for latency hiding: ask for 2 waves per SIMD
template <int D, int RT, bool PIPE>
__global__ void __launch_bounds__(kThreads, 2) tree_attn_kernel(AttnParams p) {
  constexpr int KK = D / 32;          // MFMA k-steps over the head dim
  constexpr int DT = D / 16;          // 16-wide head-dim tiles of O^T
  constexpr int ROWS = RT * 16;       // packed rows per block
  constexpr int CPR = D / 8;          // 16-byte chunks per (token, head) row
  constexpr int NL = D / 16;          // per-lane loads per sub-tile, for K and for V each
  constexpr int VSUB = kSubKeys * D * 2;                  // bytes of one V sub-tile
  constexpr int NSTAGE = PIPE ? 2 : 1;                    // V stages per wave (2 = prefetch one sub-tile ahead)
  constexpr int V_BYTES = 4 * NSTAGE * VSUB;
  constexpr int OREG = ROWS * D * 4;                      // one fp32 [ROWS][D] merge region
  constexpr int SM_BYTES = V_BYTES > 2 * OREG ? V_BYTES : 2 * OREG;  // V staging, reused by the wave merge
  constexpr int NREG = (4 * OREG <= SM_BYTES) ? 4 : 2;    // wave-merge regions (2 -> two rounds)
  constexpr int ITEM = ROWS * D + 2 * ROWS;               // floats per partial: O[ROWS][D], m[ROWS], l[ROWS]
  static_assert(kMergeItems * ROWS * 3 * 4 <= SM_BYTES, "merge staging must fit in the shared area");
  __shared__ __attribute__((aligned(16))) unsigned char vsm[SM_BYTES];
  __shared__ __attribute__((aligned(16))) uint16_t q_s[ROWS * D];
  __shared__ float red_m[4][ROWS], red_l[4][ROWS];
  __shared__ float row_m[ROWS], row_l[ROWS];
  __shared__ uint64_t anc_s[65];
  __shared__ int par_s[65];
  __shared__ int pg_s[kMaxPageIds];  // page-table entries covering this item's keys
  __shared__ int flag_s;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.x, rb = blockIdx.y, bg = blockIdx.z;
  const int b = bg / p.Hkv, g = bg - b * p.Hkv;
  const bool is_tree = (s == p.n_splits - 1);
  const int32_t* ptab = p.page_table + size_t(b) * p.max_pages;
  const int row0 = rb * ROWS;

  // ---- round trip 1: everything that does not depend on the sequence's lengths
  const int T_raw = p.T_b ? p.T_b[b] : p.max_T;
  const int L_raw = p.prefix_lens[b];
  const int pg0_spec = (s * p.chunk) >> p.page_shift;  // page ids of this prefix chunk (speculative)
  if (!is_tree) {
    const int npg = ((p.chunk - 1) >> p.page_shift) + 1;
    for (int i = tid; i < npg; i += kThreads) {
      const int pi = pg0_spec + i;
      pg_s[i] = pi < p.max_pages ? ptab[pi] : -1;
    }
  }
  // Q tile -> LDS, row-major [row][d] with 16-byte chunks swizzled by (row & 7); rows up to G * max_T
  // are always inside q, rows past this tree's M are computed and ignored
  for (int idx = tid; idx < ROWS * CPR; idx += kThreads) {
    const int row = idx / CPR, c = idx - row * CPR;
    const int r = row0 + row;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < p.G * p.max_T) {
      const int i = r / p.G, h = g * p.G + (r - i * p.G);
      v = *reinterpret_cast<const uint4*>(p.q + ((size_t(b) * p.max_T + i) * p.Hq + h) * D + 8 * c);
    }
    *reinterpret_cast<uint4*>(q_s + row * D + 8 * (c ^ (row & 7))) = v;
  }
  int par_raw = 0;
  if (is_tree && tid > 0 && tid < p.max_T) par_raw = p.parents[size_t(b) * p.max_T + tid];
  __syncthreads();

  int T = min(max(T_raw, 1), p.max_T);
  int L = L_raw;
  const int cap = p.max_pages << p.page_shift;
  if (L < 0 || L > cap - T) {
    if (p.status && is_tree && rb == 0 && g == 0 && tid == 0) atomicOr(p.status + b, SPEC_STATUS_INVALID_LENGTH);
    L = min(max(L, 0), cap - T);
  }
  const int M = p.G * T;
  if (row0 >= M) return;
  const int nrows = min(ROWS, M - row0);
  const int nsp = (L + p.chunk - 1) / p.chunk;
  if (!is_tree && s >= nsp) return;
  const int n_items = nsp + 1;
  const int key_lo = is_tree ? L : s * p.chunk;
  const int key_hi = is_tree ? L + T : min(L, key_lo + p.chunk);
  const int pg0 = key_lo >> p.page_shift;  // pg_s[i] holds page-table entry pg0 + i

  // ---- tree item: its page ids and the ancestry words (pointer doubling)
  if (is_tree) {
    const int npg = ((key_hi - 1) >> p.page_shift) - pg0 + 1;
    for (int i = tid; i < npg; i += kThreads) pg_s[i] = ptab[pg0 + i];
    if (tid < T) {
      int par = 0;
      uint64_t a = 0;
      if (tid > 0) {
        par = par_raw;
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
  uint64_t row_anc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = row0 + rt * 16 + (lane & 15);
    row_anc[rt] = (is_tree && r < M) ? anc_s[r / p.G] : 0ull;
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

  const int pmask = (1 << p.page_shift) - 1;
  const size_t tok_stride = size_t(p.Hkv) * D;
  const size_t page_stride = tok_stride << p.page_shift;
  const uint16_t* kbase = p.k + size_t(g) * D;
  const uint16_t* vbase = p.v + size_t(g) * D;
  const int g4 = 4 * (lane >> 4);
  bool bad_page = false;
  unsigned char* vwave = vsm + wave * NSTAGE * VSUB;

  // address of the (slot, head g) row in the pool, or of the zero row if the slot is not usable
  // (past the item's range, or an invalid page-table entry); branch-free
  auto row_ptr = [&](const uint16_t* base, int slot, bool& ok) -> const uint16_t* {
    const bool in = slot < key_hi;
    const int phys = pg_s[in ? (slot >> p.page_shift) - pg0 : 0];
    const bool pok = unsigned(phys) < unsigned(p.num_pages);
    bad_page |= in && !pok;
    ok = in && pok;
    const size_t row = size_t(uint32_t(phys) << p.page_shift) + size_t(slot & pmask);
    return ok ? base + row * tok_stride : p.zeros;
  };
  // issue sub-tile st: V straight into LDS stage `stg` (swizzled rows), K into registers
  auto issue = [&](int st, int stg, bf16x8 (&kop)[2][KK], uint32_t (&kvalid)[2]) {
    unsigned char* vdst = vwave + stg * VSUB;
#pragma unroll
    for (int c = 0; c < NL; ++c) {  // 1 KB of LDS per instruction: lane l -> bytes [16 l, 16 l + 16)
      const int key = c * (64 / CPR) + lane / CPR;
      const int pos = lane % CPR;
      bool ok;
      const uint16_t* src = row_ptr(vbase, st + key, ok) + 8 * (pos ^ v_swz<D>(key));
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(vdst + c * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {  // A operand: lane = key (lane & 15), head-dim chunk (lane >> 4) + 4 kk
      bool ok;
      const uint16_t* src = row_ptr(kbase, st + 16 * kt + (lane & 15), ok) + 8 * (lane >> 4);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kop[kt][kk] = load_bf16x8(src + 32 * kk);
      kvalid[kt] = uint32_t(__ballot(ok) & 0xffffull);
    }
  };
  // one sub-tile: S^T = K Q^T, online softmax, O^T += V^T P^T
  auto compute = [&](int st, int stg, const bf16x8 (&kop)[2][KK], const uint32_t (&kvalid)[2]) {
    const unsigned char* vsrc = vwave + stg * VSUB;
    f32x4 sc[2][RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = rt * 16 + (lane & 15);
      bf16x8 qop[KK];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qop[kk] = *reinterpret_cast<const bf16x8*>(q_s + row * D + 8 * ((4 * kk + (lane >> 4)) ^ (row & 7)));
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kt][kk], qop[kk], a, 0, 0, 0);
        sc[kt][rt] = a;
      }
    }
    // visibility of the lane's 8 keys (bit kt*4 + j <-> key 16 kt + 4 (lane>>4) + j)
    const uint32_t kbits = ((kvalid[0] >> g4) & 0xfu) | (((kvalid[1] >> g4) & 0xfu) << 4);
    bf16x8 pop[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      uint32_t vis = kbits;
      if (is_tree) {  // uniform: ancestor test per key (root always visible)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int jn = st + 16 * (e >> 2) + g4 + (e & 3) - L;  // tree node index of this key
          const uint64_t sh = row_anc[rt] >> (jn > 0 ? jn - 1 : 0);
          const bool anc = (jn == 0) || (jn > 0 && (sh & 1ull));
          vis &= anc ? 0xffu : ~(1u << e);
        }
      }
      float sv[8];  // raw scores (masked -> -inf); the scale is folded into the exponent's fma
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[kt * 4 + j] = ((vis >> (kt * 4 + j)) & 1u) ? sc[kt][rt][j] : -INFINITY;
      float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float mnew = fmaxf(m_run[rt], mx * p.scale_log2);  // running max in the scaled (log2) domain
      const bool none = (mnew == -INFINITY);
      const float alpha = none ? 1.f : fast_exp2(m_run[rt] - mnew);
      float pe[8];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pe[e] = none ? 0.f : fast_exp2(__builtin_fmaf(sv[e], p.scale_log2, -mnew));
        psum += pe[e];
      }
      l_run[rt] = l_run[rt] * alpha + psum;
      m_run[rt] = mnew;
      if (__any(alpha != 1.f)) {  // uniform: skip the rescale when no row's max moved
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[rt][dt] *= alpha;
      }
      uint4 pk;
      pk.x = pack2_bf16(pe[0], pe[1]);
      pk.y = pack2_bf16(pe[2], pe[3]);
      pk.z = pack2_bf16(pe[4], pe[5]);
      pk.w = pack2_bf16(pe[6], pe[7]);
      pop[rt] = __builtin_bit_cast(bf16x8, pk);
    }
    // V^T operand for head-dim column dt*16 + (lane & 15): keys 4(lane>>4) + {0..3} and 16 + 4(lane>>4) + {0..3}
    // (the same keys, in the same order, as the lane's P^T column). Two transposing reads: lane i of
    // group g points at key 16 h + 4 g + i/4, columns 16 dt + 4 (i % 4) .. +3.
    const int ig = lane & 15;
    const int q4 = ig >> 2;        // key & 3 of the row this lane points at
    const int cl = (ig & 3) >> 1;  // which 16-byte chunk of the 32-byte column group
    const int e4 = 4 * (ig & 1);   // element offset inside the chunk
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      s16x4 half[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = 16 * h + g4 + q4;
        const int chunk = (2 * dt + cl) ^ v_swz<D>(key);
        half[h] = lds_read_tr16(vsrc + key * (2 * D) + 16 * chunk + 2 * e4);
      }
      const bf16x8 vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[rt], acc[rt][dt], 0, 0, 0);
    }
  };

  // ---- main loop: two register sets for K, two LDS stages for V, one sub-tile in flight ahead.
  // The next sub-tile is always issued (past the end it reads the zero row), so the loop body is
  // straight-line and exactly 2 * NL loads are outstanding at each wait.
  const int first = key_lo + kSubKeys * wave;
  const int nsub = first < key_hi ? (key_hi - first + 4 * kSubKeys - 1) / (4 * kSubKeys) : 0;
  if constexpr (PIPE) {
    bf16x8 kA[2][KK], kB[2][KK];
    uint32_t vA[2], vB[2];
    if (nsub > 0) {
      issue(first, 0, kA, vA);
#pragma unroll 1
      for (int j = 0; j < nsub; j += 2) {
        const int st0 = first + j * 4 * kSubKeys, st1 = st0 + 4 * kSubKeys;
        issue(st1, 1, kB, vB);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NL) : "memory");  // sub-tile j landed; j+1 in flight
        compute(st0, 0, kA, vA);
        if (j + 1 >= nsub) break;
        issue(st1 + 4 * kSubKeys, 0, kA, vA);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NL) : "memory");
        compute(st1, 1, kB, vB);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the prefetch past the end
    }
  } else {  // one stage: other blocks on the SIMD hide the latency
    bf16x8 kA[2][KK];
    uint32_t vA[2];
#pragma unroll 1
    for (int j = 0; j < nsub; ++j) {
      const int st = first + j * 4 * kSubKeys;
      issue(st, 0, kA, vA);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      compute(st, 0, kA, vA);
    }
  }

  if (bad_page && p.status) atomicOr(p.status + b, SPEC_STATUS_INVALID_PAGE);

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    l_run[rt] += __shfl_xor(l_run[rt], 16, kWave);
    l_run[rt] += __shfl_xor(l_run[rt], 32, kWave);
  }

  // ---- merge the 4 waves (fixed order): NREG separate fp32 regions in the V area, summed when read
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
  float* oreg = reinterpret_cast<float*>(vsm);  // [NREG][ROWS][D]
  auto put = [&](bool add) {
    float* o = oreg + (wave % NREG) * (ROWS * D);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int row = rt * 16 + (lane & 15);
        float4* dst = reinterpret_cast<float4*>(o + row * D + dt * 16 + g4);
        const f32x4 v4 = acc[rt][dt] * fac[rt];
        float4 t = make_float4(v4[0], v4[1], v4[2], v4[3]);
        if (add) {
          const float4 x = *dst;
          t = make_float4(x.x + t.x, x.y + t.y, x.z + t.z, x.w + t.w);
        }
        *dst = t;
      }
  };
  if (wave < NREG) put(false);
  __syncthreads();
  if (NREG == 2) {
    if (wave >= 2) put(true);
    __syncthreads();
  }
  auto merged = [&](int row, int d) {
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < NREG; ++r) v += oreg[r * (ROWS * D) + row * D + d];
    return v;
  };

  constexpr float kLn2 = 0.69314718055994530942f;
  if (n_items == 1) {  // no prefix: this item is the whole answer
    for (int idx = tid; idx < nrows * D; idx += kThreads) {
      const int row = idx / D, d = idx - row * D;
      const int r = row0 + row, i = r / p.G, h = g * p.G + (r - i * p.G);
      const float ls = row_l[row];
      const float o = ls > 0.f ? merged(row, d) / ls : 0.f;
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
    const float2 v2 = make_float2(merged(row, 2 * c2), merged(row, 2 * c2 + 1));
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

  // merge in fixed item order. (1) every item's (m, l) -> LDS in one round trip; (2) per-row max,
  // normaliser and item weights; (3) O: each thread owns KP float4 columns and loads them for IB items
  // at a time, so the KP * IB loads of a batch are in flight together.
  constexpr int D4 = D / 4;
  constexpr int KP = (ROWS * D4 + kThreads - 1) / kThreads;  // float4 columns per thread
  constexpr int IB = KP >= 6 ? 4 : (KP >= 4 ? 6 : 12);       // items per batch (bounded registers)
  float* wts = reinterpret_cast<float*>(vsm);                   // [n_items][ROWS] weights
  float* mls = wts + kMergeItems * ROWS;                        // [n_items][2][ROWS] raw (m, l)
  constexpr float kLn2m = 0.69314718055994530942f;
  // n_items <= kMergeItems by construction of the plan
  for (int idx = tid; idx < n_items * 2 * ROWS; idx += kThreads) {
    const int it = idx / (2 * ROWS), r2 = idx - it * 2 * ROWS;
    mls[idx] = (r2 % ROWS) < nrows ? ld_agent(grp + size_t(it < nsp ? it : p.n_splits - 1) * ITEM + ROWS * D + r2) : 0.f;
  }
  __syncthreads();
  if (tid < nrows) {
    float mx = -INFINITY;
    for (int it = 0; it < n_items; ++it) mx = fmaxf(mx, mls[it * 2 * ROWS + tid]);
    float ls = 0.f;
    for (int it = 0; it < n_items; ++it) {
      const float m = mls[it * 2 * ROWS + tid];
      const float f = (m == -INFINITY) ? 0.f : fast_exp2(m - mx);
      ls += mls[it * 2 * ROWS + ROWS + tid] * f;
      wts[it * ROWS + tid] = f;
    }
    row_m[tid] = mx;
    row_l[tid] = ls;
  }
  __syncthreads();
  {
    float4 o[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) o[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int ib = 0; ib < n_items; ib += IB) {
      float4 av[IB][KP];
#pragma unroll
      for (int u = 0; u < IB; ++u)
#pragma unroll
        for (int k = 0; k < KP; ++k) {
          const int idx = tid + k * kThreads;
          const int it = ib + u;
          av[u][k] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (it < n_items && idx < nrows * D4) {
            const int row = idx / D4, c4 = idx - row * D4;
            const uint64_t* q2 = reinterpret_cast<const uint64_t*>(
                grp + size_t(it < nsp ? it : p.n_splits - 1) * ITEM + row * D + 4 * c4);
            const float2 lo2 = __builtin_bit_cast(float2, ld_agent(q2));
            const float2 hi2 = __builtin_bit_cast(float2, ld_agent(q2 + 1));
            av[u][k] = make_float4(lo2.x, lo2.y, hi2.x, hi2.y);
          }
        }
#pragma unroll
      for (int u = 0; u < IB; ++u)
#pragma unroll
        for (int k = 0; k < KP; ++k) {
          const int idx = tid + k * kThreads;
          const int it = ib + u;
          if (it < n_items && idx < nrows * D4) {
            const float wv = wts[it * ROWS + idx / D4];
            o[k].x += av[u][k].x * wv;
            o[k].y += av[u][k].y * wv;
            o[k].z += av[u][k].z * wv;
            o[k].w += av[u][k].w * wv;
          }
        }
    }
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int idx = tid + k * kThreads;
      if (idx >= nrows * D4) continue;
      const int row = idx / D4, c4 = idx - row * D4;
      const float ls = row_l[row];
      const float inv = ls > 0.f ? 1.f / ls : 0.f;
      const int r = row0 + row, i = r / p.G, h = g * p.G + (r - i * p.G);
      uint16_t* dst = p.out + ((size_t(b) * p.max_T + i) * p.Hq + h) * D + 4 * c4;
      *reinterpret_cast<uint2*>(dst) = make_uint2(pack2_bf16(o[k].x * inv, o[k].y * inv), pack2_bf16(o[k].z * inv, o[k].w * inv));
    }
  }
  if (p.lse && tid < nrows) {
    const int r = row0 + tid, i = r / p.G, h = g * p.G + (r - i * p.G);
    const float ls = row_l[tid];
    p.lse[(size_t(b) * p.max_T + i) * p.Hq + h] = ls > 0.f ? (row_m[tid] + __log2f(ls)) * kLn2m : -INFINITY;
  }
}

struct AttnPlan {
  int G, RT, rows, n_rb, chunk, n_splits;
  size_t zero_bytes, part_bytes, ticket_bytes;
};

AttnPlan make_plan(int B, int max_T, int Hq, int Hkv, int d, int page, int max_pages) {
  AttnPlan pl;
  pl.G = Hq / Hkv;
  const int M = pl.G * max_T;
  pl.RT = (M + 15) / 16;
  if (pl.RT > 3) pl.RT = 3;  // 48 rows: the largest tile whose pipelined loop fits the register file without spills
  pl.rows = pl.RT * 16;
  pl.n_rb = (M + pl.rows - 1) / pl.rows;
  const long long slots = (long long)max_pages * page;
  const long long groups = (long long)B * Hkv * pl.n_rb;
  long long chunk = (slots * groups + 4095) / 4096;  // aim at ~4k work items
  if (chunk < 4LL * pl.rows) chunk = 4LL * pl.rows;  // keep partials small next to the KV they summarise
  if (chunk > kMaxChunk) chunk = kMaxChunk;
  if (const char* env = getenv("SPEC_TREE_ATTN_CHUNK")) {
    const long long c = atoll(env);
    if (c >= 128) chunk = c;
  }
  // at most kMergeItems - 1 prefix chunks, so the merge stages every item at once
  const long long min_chunk = (slots + kMergeItems - 2) / (kMergeItems - 1);
  if (chunk < min_chunk) chunk = min_chunk;
  chunk = (chunk + 127) / 128 * 128;
  pl.chunk = int(std::min<long long>(chunk, 1LL << 30));
  pl.n_splits = int((slots + chunk - 1) / chunk) + 1;
  const size_t item = size_t(pl.rows) * d + 2 * size_t(pl.rows);
  pl.zero_bytes = 1024;  // never written: stays as zero-filled as the caller provided it
  pl.part_bytes = align_up(size_t(groups) * pl.n_splits * item * sizeof(float), 256);
  pl.ticket_bytes = align_up(size_t(groups) * sizeof(uint32_t), 256);
  return pl;
}

template <int D, bool PIPE>
void launch_dp(const AttnPlan& pl, const AttnParams& prm, dim3 grid, hipStream_t st) {
  switch (pl.RT) {
    case 1: hipLaunchKernelGGL((tree_attn_kernel<D, 1, PIPE>), grid, dim3(kThreads), 0, st, prm); break;
    case 2: hipLaunchKernelGGL((tree_attn_kernel<D, 2, PIPE>), grid, dim3(kThreads), 0, st, prm); break;
    default: hipLaunchKernelGGL((tree_attn_kernel<D, 3, PIPE>), grid, dim3(kThreads), 0, st, prm); break;
  }
}

// the prefetching loop pays off only when a wave walks more than one sub-tile of its chunk
template <int D>
void launch_d(const AttnPlan& pl, const AttnParams& prm, dim3 grid, hipStream_t st) {
  if (pl.chunk > 4 * kSubKeys)
    launch_dp<D, true>(pl, prm, grid, st);
  else
    launch_dp<D, false>(pl, prm, grid, st);
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
  if (((pl.chunk - 1) >> ilog2(page)) + 1 > kMaxPageIds - 2) return 0;
  return pl.zero_bytes + pl.part_bytes + pl.ticket_bytes;
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
  if (((pl.chunk - 1) >> ilog2(page)) + 1 > kMaxPageIds - 2)
    return fail(SPEC_E_UNSUPPORTED, "spec_tree_attention: prefix of %lld slots needs chunks of %d keys > %d pages",
                (long long)max_pages * page, pl.chunk, kMaxPageIds - 2);
  const size_t need = pl.zero_bytes + pl.part_bytes + pl.ticket_bytes;
  if (!ws || ws_bytes < need) return fail(SPEC_E_WORKSPACE, "spec_tree_attention: workspace %zu bytes < %zu", ws_bytes, need);
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
  prm.zeros = static_cast<const uint16_t*>(ws);
  prm.part = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.zero_bytes);
  prm.tickets = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + pl.zero_bytes + pl.part_bytes);
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
