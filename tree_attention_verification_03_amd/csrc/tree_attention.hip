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
//   The keys of sequence b are its L_b prefix slots followed by its T_b tree
//   slots (stored in the same pages). grid.x = key chunk s, keys
//   [s*chunk, min((s+1)*chunk, L_b + T_b)); grid.y = block of row tiles;
//   grid.z = (b, kv head g).
//   Rows r = i * G + h' pack the G query heads sharing KV head g with the tree
//   nodes, so every K/V tile fetched from HBM serves all G*T rows of (b, g).
//   Rows form 16-row tiles; wave w of a block owns tiles w, w + NW, ... of the
//   block's range and keeps their Q operands in registers.
//   All waves stream the chunk through an NS-stage LDS ring of 32-key tiles (K
//   and V rows loaded straight from HBM into LDS); per tile each wave computes
//   for its rows:
//     S^T = K Q^T  : bf16 MFMA 16x16x32, keys are the A operand (read from LDS);
//     online softmax on S^T columns (each lane owns one query row; the row max
//                    over the 4 lanes sharing it via two xor-shuffles). The
//                    reference max only moves when a score exceeds it by more
//                    than 2^8, so the O rescale is rare; exponentials stay
//                    below 2^8 and exact in the final normalisation;
//     O^T += V^T P^T: P^T is the S^T accumulator re-packed to bf16 in place,
//                    V^T comes from transposing LDS reads.
//   Waves own distinct rows, so nothing is merged inside a block. An item
//   whose sequence needs more than one item writes its partial (O, m, l) to
//   the workspace; a second, small kernel combines the partials of each row
//   in fixed item order and writes out / lse. Deterministic; no atomics.
#include <mutex>

#include "api_common.h"
#include "spec_common.h"

namespace spectree {
namespace {

constexpr int kXcds = 8;  // MI355X: 8 XCDs, each with its own L2

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kTile = 32;         // keys per ring stage
constexpr int kMaxChunk = 1792;   // keys per work item, at most (mixed-length batch: 545 us at 1792, 814 us at 2048)
constexpr float kTau = 8.f;       // log2 headroom of the lazily moved reference max
constexpr int kTargetBlocks = 384;  // ~1.5 blocks per CU: fewer, longer items beat full occupancy (measured)
constexpr int kTargetBlocks8 = 440;  // 8-wave (compute-heavy) plans: 64-node tree 44 us at 440 blocks, 50 us at 400

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
  const uint16_t* zeros;  // a zero-filled (token, head) row in the workspace: source of masked loads
  const float* k_scale;   // FP8-KV variant: per-KV-head scales of the E4M3 codes (else unused)
  const float* v_scale;
  int max_T, Hq, Hkv, G;
  int page_shift, max_pages, num_pages;
  int chunk, n_splits, n_rb, tpb, npg;
  int n_groups;  // B * Hkv * n_splits
  float scale_log2;
};

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// four fp32 -> packed fp16, round-to-nearest-even
__device__ __forceinline__ uint2 pack4_f16(f32x4 v) {
  return __builtin_bit_cast(uint2, __builtin_convertvector(v, f16x4));
}

// two fp32 -> packed bf16 pair, hardware round-to-nearest-even
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// gfx950 transposing LDS read: within each 16-lane group, lane i names a row of 4 consecutive
// 16-bit elements and lane l receives element (l % 4) of rows l/4, l/4 + 4, l/4 + 8, l/4 + 12.
__device__ __forceinline__ s16x4 lds_read_tr16(const unsigned char* addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(addr));
}

// Direct global -> LDS load of 16 bytes per lane (lane l's bytes land at lds_dst + 16 l), written as
// inline asm on purpose: the compiler then keeps these loads out of its wait-count bookkeeping, which
// would otherwise wait for every outstanding direct load before each LDS read of the kernel. The ring
// is synchronised explicitly instead (s_waitcnt vmcnt(n) + barrier), and no load the compiler issues
// is in flight while the ring runs. M0 carries the LDS base (uniform by contract: read from lane 0);
// nothing else in this file uses M0.
__device__ __forceinline__ void load_to_lds16(const void* src, uint32_t lds_off) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_off);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m) : "memory");
}

// LDS byte address of a __shared__ array (taken once: a generic pointer cast back to LDS costs a null
// check per use)
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* shared_array) {
  return uint32_t(reinterpret_cast<uintptr_t>((lds_void*)shared_array));
}

// max over the 4 lanes l, l ^ 16, l ^ 32, l ^ 48 (the lanes holding one query row of an S^T tile), with
// the gfx950 row swaps: swapping the odd 16-lane rows of one copy with the even rows of another puts
// every lane's xor-16 partner in one of the two results (likewise for 32-lane halves)
__device__ __forceinline__ float lanegroup_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(x);
  const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// LDS layout of one ring stage: K rows then V rows, 2*D bytes per key, 16-byte chunks swizzled per key
// (CPR = D / 8 chunks per row):
//   K: chunk c of key j sits at c ^ (j & (CPR - 1)); the A-operand read of 16 keys at one chunk then
//      touches 16 different chunks (d = 128: all 64 banks once);
//   V: chunk c of key j sits at c ^ 2 (j & 3), and at d = 128 also ^ 8 for odd groups of 4 keys: a
//      transposing read of 4 keys hits 4 different 32-byte groups, and the 16-lane groups reading
//      keys 4g..4g+3 and 4(g+1)..4(g+1)+3 use opposite 128-byte halves of the bank row.
template <int D>
__device__ __forceinline__ int k_swz(int key) { return key & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int v_swz(int key) { return 2 * (key & 3) ^ (D == 128 ? 8 * ((key >> 2) & 1) : 0); }

// blocks of this shape that fit one CU's 160 KB of LDS (the ring dominates): 2, or 1 for deep rings
constexpr int blocks_per_cu(int D, int NS) { return NS * 128 * D + 4096 <= 160 * 1024 / 2 ? 2 : 1; }

// SPS ring stages of 32 keys form one softmax step (one barrier, one running-max update per step)

// Split-K merge of one output row, item by item in fixed order against the running maximum
// reference max: out = sum_i w_i l_i o_i / sum_i w_i l_i with w_i = 2^(m_i - max_j m_j) and o_i = O_i / l_i
// the item's normalised output (stored fp16 times a power-of-two row scale). A thread owns 4 columns (o).
struct RowMerge {
  float mx = -INFINITY, ls = 0.f;
  f32x8 o = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // fold the first `navail` of a batch of CB items (the rest are unused loads and may hold anything)
  template <int CB>
  __device__ __forceinline__ void fold(const float (&mi)[CB], const float (&li)[CB], const f32x8 (&ai)[CB], int navail) {
    float mb = mx;
#pragma unroll
    for (int u = 0; u < CB; ++u)
      if (u < navail) mb = fmaxf(mb, mi[u]);
    if (mb == -INFINITY) return;  // nothing visible yet
    const float sc = (mx == -INFINITY) ? 0.f : fast_exp2(mx - mb);
    ls *= sc;
    o *= sc;
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      if (u < navail && mi[u] != -INFINITY) {  // guarded, not weighted
        const float w = fast_exp2(mi[u] - mb) * li[u];
        ls += w;
        o += ai[u] * w;
      }
    }
    mx = mb;
  }
  // out / lse of packed row r (node r / G, head g G + r % G) of sequence b, KV head g; columns 8c..8c+7
  template <int D>
  __device__ __forceinline__ void write(const AttnParams& p, int b, int g, int r, int c) const {
    const int i = r / p.G, h = g * p.G + (r - i * p.G);
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
    const f32x8 v = o * inv;
    *reinterpret_cast<uint4*>(p.out + ((size_t(b) * p.max_T + i) * p.Hq + h) * D + 8 * c) =
        make_uint4(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]), pack2_bf16(v[4], v[5]), pack2_bf16(v[6], v[7]));
    constexpr float kLn2 = 0.69314718055994530942f;
    if (p.lse && c == 0) p.lse[(size_t(b) * p.max_T + i) * p.Hq + h] = ls > 0.f ? (mx + __log2f(ls)) * kLn2 : -INFINITY;
  }
};

template <int D, int NW, int RW, int NS, int SPS>
__global__ void __launch_bounds__(64 * NW, NW / 4 * blocks_per_cu(D, NS)) tree_attn_kernel(AttnParams p) {
  constexpr int KK = D / 32;               // MFMA k-steps over the head dim
  constexpr int DT = D / 16;               // 16-wide head-dim tiles of O^T
  constexpr int CPR = D / 8;               // 16-byte chunks per (token, head) row
  constexpr int ROWB = 2 * D;              // bytes per (token, head) row
  constexpr int TILE_B = kTile * ROWB;     // bytes of K (or V) per ring stage
  constexpr int STAGE_B = 2 * TILE_B;
  constexpr int RPI = 1024 / ROWB;         // key rows per direct-to-LDS instruction (64 lanes x 16 B)
  constexpr int NLD = TILE_B / 1024;       // such instructions per stage and buffer
  constexpr int PW = 2 * NLD / NW;         // ... per wave and stage
  constexpr int NT = 64 * NW;
  static_assert(PW >= 2 && PW * NW == 2 * NLD, "each wave loads whole K/V row pairs");
  static_assert(NS >= 2 * SPS && NS % SPS == 0, "a step's stages are consecutive ring slots");
  constexpr int PH = PW / 2;               // key rows (x 1 KB) per wave and stage, each loaded for K and for V
  // 256-register kernels (at most two waves per SIMD) hold a stage's V operands across the softmax
  constexpr bool kPrefetchV = NW / 4 * blocks_per_cu(D, NS) <= 2;
  static_assert(NT >= 65, "the tree prologue uses one thread per node");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[NS * STAGE_B];
  const uint32_t ring_lds = lds_addr(ring);
  __shared__ uint64_t anc_s[65];
  extern __shared__ int pg_s[];  // page-table entries covering this item's keys (p.npg of them)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform, so everything derived from it is scalar
  // Workgroups are dealt to the 8 XCDs round-robin by flattened id. 8-wave blocks (the only plans
  // with several row blocks per (sequence, KV head, item) group, which stream the same keys) run on
  // a 1-D grid whose ids are re-mapped so a group's row blocks get one residue mod 8 and consecutive
  // slots: they share that XCD's L2, and groups stay balanced over the XCDs (ids past the last group
  // exit). 4-wave blocks have one row block and use the 3-D grid as it is (no division on the way to
  // the first loads).
  int s, rb, bg;
  if constexpr (NW == 8) {
    const int xcd = blockIdx.x & (kXcds - 1), slot = blockIdx.x / kXcds;
    const int grp = (slot / p.n_rb) * kXcds + xcd;
    if (grp >= p.n_groups) return;
    rb = slot - (slot / p.n_rb) * p.n_rb;
    bg = grp / p.n_splits;
    s = grp - bg * p.n_splits;
  } else {
    s = blockIdx.x;
    rb = blockIdx.y;
    bg = blockIdx.z;
  }
  const int b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int32_t* ptab = p.page_table + size_t(b) * p.max_pages;
  const int t0 = rb * p.tpb;  // first row tile of this block
  const int l15 = lane & 15, g4 = 4 * (lane >> 4);

  // ---- round trip 1: everything that does not depend on the sequence's lengths
  const int T_raw = p.T_b ? p.T_b[b] : p.max_T;
  const int L_raw = p.prefix_lens[b];
  const int pg0 = (s * p.chunk) >> p.page_shift;  // pg_s[i] holds page-table entry pg0 + i
  for (int i = tid; i < p.npg; i += NT) {
    const int pi = pg0 + i;
    pg_s[i] = pi < p.max_pages ? ptab[pi] : -1;
  }
  int par_raw = 0;  // wave 0, lane l: the parent of node l + 1
  if (tid < kWave && tid + 1 < p.max_T) par_raw = p.parents[size_t(b) * p.max_T + tid + 1];
  // Q operands of this wave's row tiles: lane = row (lane & 15), head-dim chunk (lane >> 4) + 4 kk.
  // Rows up to G * max_T are inside q; rows past this tree's M are computed and ignored.
  bf16x8 qop[RW][KK];
#pragma unroll
  for (int rw = 0; rw < RW; ++rw) {
    const int lt = wave + NW * rw;
    const int r = 16 * (t0 + lt) + l15;
    const bool ok = lt < p.tpb && r < p.G * p.max_T;
    const int rr = ok ? r : 0;
    const int i = rr / p.G, h = g * p.G + (rr - i * p.G);
    const uint16_t* src = p.q + ((size_t(b) * p.max_T + i) * p.Hq + h) * D + 8 * (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 v = load_bf16x8(src + 32 * kk);
      qop[rw][kk] = ok ? v : bf16x8{};
    }
  }
  __syncthreads();

  int T = min(max(T_raw, 1), p.max_T);
  int L = L_raw;
  const int cap = p.max_pages << p.page_shift;
  if (L < 0 || L > cap - T) {
    if (p.status && s == 0 && rb == 0 && g == 0 && tid == 0) atomicOr(p.status + b, SPEC_STATUS_INVALID_LENGTH);
    L = min(max(L, 0), cap - T);
  }
  const int M = p.G * T;
  const int ntM = (M + 15) >> 4;
  if (t0 >= ntM) return;
  const int n_items = (L + T + p.chunk - 1) / p.chunk;
  if (s >= n_items) return;
  const int key_lo = s * p.chunk;
  const int key_hi = min(L + T, key_lo + p.chunk);
  const bool has_tree = key_hi > L;

  // ---- page-table entries of the chunk must name pages of the pool; tree ancestry words
  bool bad = false;
  {
    const int npg_used = ((key_hi - 1) >> p.page_shift) - pg0 + 1;
    for (int i = tid; i < npg_used; i += NT) bad |= unsigned(pg_s[i]) >= unsigned(p.num_pages);
  }
  // ancestry words of the tree (wave 0; node n in lane n - 1): pointer doubling over lanes, each round
  // doubling the generations covered, then one barrier publishes them
  if (has_tree && tid < kWave) {
    const int n = tid + 1;
    const bool real = n < T;
    int par = 0;
    if (real) {
      par = par_raw;
      if (par < 0 || par >= n) {
        par = 0;
        if (p.status && rb == 0 && g == 0) atomicOr(p.status + b, SPEC_STATUS_INVALID_PARENT);
      }
    }
    uint64_t a = real ? (1ull << tid) : 0ull;
    int jump = par;  // 0 = the root: nothing above
    while (__ballot(jump != 0)) {
      const int src = jump > 0 ? jump - 1 : tid;
      const uint64_t pa = (uint64_t(uint32_t(__shfl(int(a >> 32), src))) << 32) | uint32_t(__shfl(int(a), src));
      const int pj = __shfl(jump, src);
      if (jump != 0) {
        a |= pa;
        jump = pj;
      }
    }
    if (real) anc_s[n] = a;
    if (tid == 0) anc_s[0] = 0;
  }
  const bool pages_ok = !__syncthreads_or(bad);
  if (!pages_ok && p.status && tid == 0) atomicOr(p.status + b, SPEC_STATUS_INVALID_PAGE);
  uint64_t ranc[RW];
#pragma unroll
  for (int rw = 0; rw < RW; ++rw) {
    const int r = 16 * (t0 + wave + NW * rw) + l15;
    ranc[rw] = (has_tree && r < M) ? anc_s[r / p.G] : 0ull;
  }
  // this wave owns at least one row tile of the block that holds rows of this tree
  const bool active = wave < p.tpb && t0 + wave < ntM;

  // per row tile: reference max (log2 domain), O^T accumulator and the row sums of P (from an extra
  // MFMA against an all-ones V^T tile: every lane gets its row's sum, no reduction needed)
  float m_run[RW];
  f32x4 acc[RW][DT], lacc[RW];
#pragma unroll
  for (int rw = 0; rw < RW; ++rw) {
    m_run[rw] = -INFINITY;
    lacc[rw] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[rw][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));

  const int pmask = (1 << p.page_shift) - 1;
  // load addresses in bytes: a page's offset is one 32 x 32 -> 64-bit multiply-add, everything inside a
  // page stays in 32 bits (the host checks that a page spans less than 2^31 bytes)
  const uint32_t tok_b = uint32_t(p.Hkv) * (2 * D);  // bytes between consecutive slots of a page
  const uint32_t page_b = tok_b << p.page_shift;
  const uint64_t kbase = reinterpret_cast<uint64_t>(p.k) + uint64_t(g) * (2 * D);
  const uint64_t vbase = reinterpret_cast<uint64_t>(p.v) + uint64_t(g) * (2 * D);

  // this wave's share of a stage: key rows sub_i * RPI + lane / CPR (sub_i = wave + NW i), one 16-byte chunk
  // per lane, loaded once for K and once for V (swizzled on the global side: LDS gets lane-order bytes)
  int lkey[PH];
  uint32_t koff[PH], voff[PH];  // byte offsets of the lane's chunk inside its (slot, head) row
#pragma unroll
  for (int i = 0; i < PH; ++i) {
    lkey[i] = (wave + NW * i) * RPI + lane / CPR;
    const int pos = lane % CPR;
    koff[i] = 16u * uint32_t(pos ^ k_swz<D>(lkey[i]));
    voff[i] = 16u * uint32_t(pos ^ v_swz<D>(lkey[i]));
  }
  const uint64_t zbase = reinterpret_cast<uint64_t>(p.zeros);
  // issue the direct loads of this wave's share of key tile `tile` into ring stage `slot`; slots past
  // the chunk and slots on invalid pages read the zero row (their keys are masked in compute)
  auto issue = [&](int tile, int slot) {
    const int st = key_lo + tile * kTile;
    const uint32_t sb = ring_lds + slot * STAGE_B;
    const bool full = pages_ok && st + kTile <= key_hi;  // uniform
#pragma unroll
    for (int i = 0; i < PH; ++i) {
      const int slot_k = st + lkey[i];
      uint64_t ks, vs;
      if (full) {
        const uint32_t phys = uint32_t(pg_s[(slot_k >> p.page_shift) - pg0]);
        const uint64_t pgo = uint64_t(phys) * page_b;
        const uint32_t in_pg = uint32_t(slot_k & pmask) * tok_b;
        ks = kbase + pgo + (in_pg + koff[i]);
        vs = vbase + pgo + (in_pg + voff[i]);
      } else {
        const bool in = slot_k < key_hi;
        const uint32_t phys = uint32_t(pg_s[in ? (slot_k >> p.page_shift) - pg0 : 0]);
        const bool ok = in && phys < unsigned(p.num_pages);
        const uint64_t pgo = uint64_t(phys) * page_b;
        const uint32_t in_pg = uint32_t(slot_k & pmask) * tok_b;
        ks = ok ? kbase + pgo + (in_pg + koff[i]) : zbase + koff[i];
        vs = ok ? vbase + pgo + (in_pg + voff[i]) : zbase + voff[i];
      }
      const int sub = wave + NW * i;
      load_to_lds16(reinterpret_cast<const void*>(ks), sb + sub * 1024);
      load_to_lds16(reinterpret_cast<const void*>(vs), sb + TILE_B + sub * 1024);
    }
  };

  // one step = SPS consecutive key tiles (32 SPS keys) for this wave's row tiles: S^T = K Q^T, online
  // softmax over the step's scores, O^T += V^T P^T. Masked steps (the chunk's end, tree slots, invalid
  // pages) test every key; the others skip all masking.
  constexpr int NE = 8 * SPS;  // scores per lane and row tile in one step
  auto compute = [&](int tile, int slot, bool masked) {
    const int st = key_lo + tile * kTile;
    // lane score e <-> key st + 32 (e / 8) + 16 ((e / 4) % 2) + g4 + e % 4
    auto key_of = [&](int e) { return st + 32 * (e >> 3) + 16 * ((e >> 2) & 1) + g4 + (e & 3); };
    f32x4 sc[RW][2 * SPS];
    // K fragments of the step's 2 SPS units of 16 keys (A operand: key l15, head-dim chunk 4 kk + lane / 16),
    // each unit's LDS reads issued before the MFMAs of the unit before it
    auto read_k = [&](int u, bf16x8 (&kop)[KK]) {
      const unsigned char* kr = ring + ((slot + u / 2) % NS) * STAGE_B + (16 * (u & 1) + l15) * ROWB;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kop[kk] = *reinterpret_cast<const bf16x8*>(kr + 16 * ((4 * kk + (lane >> 4)) ^ k_swz<D>(l15)));
    };
    bf16x8 kbuf[2][KK];
    read_k(0, kbuf[0]);
#pragma unroll
    for (int u = 0; u < 2 * SPS; ++u) {
      if (u + 1 < 2 * SPS) read_k(u + 1, kbuf[(u + 1) & 1]);
#pragma unroll
      for (int rw = 0; rw < RW; ++rw) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kbuf[u & 1][kk], qop[rw][kk], a, 0, 0, 0);
        sc[rw][u] = a;
      }
    }
    // V^T operand for head-dim column dt*16 + (lane & 15): keys g4 + {0..3} and 16 + g4 + {0..3} of each
    // stage (the same keys, in the same order, as the lane's P^T column). Two transposing reads: lane i
    // of each 16-lane group points at key 16 h + g4 + i/4, columns 16 dt + 4 (i % 4) .. +3.
    const int q4 = l15 >> 2;        // key & 3 of the row this lane points at
    const int cl = (l15 & 3) >> 1;  // which 16-byte chunk of the 32-byte column group
    const int e4 = 4 * (l15 & 1);   // element offset inside the chunk
    auto read_v = [&](int ss, int dt) {
      const unsigned char* vb = ring + ((slot + ss) % NS) * STAGE_B + TILE_B;
      s16x4 half[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = 16 * h + g4 + q4;
        const int chunk = (2 * dt + cl) ^ v_swz<D>(key);
        half[h] = lds_read_tr16(vb + key * ROWB + 16 * chunk + 2 * e4);
      }
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // kernels with registers to spare read the first stage's V operands now, so the reads run under the
    // softmax arithmetic
    bf16x8 vbuf[DT];
    if constexpr (kPrefetchV) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vbuf[dt] = read_v(0, dt);
    }
    // kernels without them keep one V operand in flight: the first now, each next one before the MFMA
    // that consumes the current one
    bf16x8 vnext;
    if constexpr (!kPrefetchV) vnext = read_v(0, 0);
    // usable keys among the lane's NE (bit e <-> key_of(e))
    uint32_t kvis = (1u << NE) - 1u;
    if (masked) {  // uniform
      kvis = 0;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int key = key_of(e);
        const bool in = key < key_hi;
        const int phys = pg_s[in ? (key >> p.page_shift) - pg0 : 0];
        kvis |= (in && unsigned(phys) < unsigned(p.num_pages)) ? (1u << e) : 0u;
      }
    }
    bf16x8 pop[RW][SPS];
#pragma unroll
    for (int rw = 0; rw < RW; ++rw) {
      float sv[NE];  // raw scores, masked -> -inf; the scale is folded into the exponent's fma
      if (masked) {  // uniform
        uint32_t vis = kvis;
        if (st + SPS * kTile > L) {  // uniform: tree slots in this step; the root is every node's ancestor
#pragma unroll
          for (int e = 0; e < NE; ++e) {
            const int jn = key_of(e) - L;  // tree node index of this key
            const int sh = min(max(jn - 1, 0), 63);
            const bool anc = jn == 0 || (jn > 0 && ((ranc[rw] >> sh) & 1ull));
            vis &= anc || jn < 0 ? 0xffffffffu : ~(1u << e);
          }
        }
        // the empty asm keeps the compiler from merging these selects into the unmasked path (as
        // selects against an all-ones mask)
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          sv[e] = ((vis >> e) & 1u) ? sc[rw][e >> 2][e & 3] : -INFINITY;
          asm volatile("" : "+v"(sv[e]));
        }
      } else {
#pragma unroll
        for (int e = 0; e < NE; ++e) sv[e] = sc[rw][e >> 2][e & 3];
      }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < NE; ++e) mx = fmaxf(mx, sv[e]);
      mx = lanegroup_max(mx);
      const float mxs = mx * p.scale_log2;  // step max in the scaled (log2) domain
      const bool move = mxs > m_run[rw] + kTau;
      if (__any(move)) {  // uniform: some row's reference max moves (always on its first visible key)
        const float mnew = move ? mxs : m_run[rw];
        const float alpha = move ? fast_exp2(m_run[rw] - mnew) : 1.f;
        lacc[rw] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[rw][dt] *= alpha;
        m_run[rw] = mnew;
      }
      const float mref = m_run[rw] == -INFINITY ? 0.f : m_run[rw];  // no visible key yet: every p is 0
#pragma unroll
      for (int ss = 0; ss < SPS; ++ss) {
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(__builtin_fmaf(sv[8 * ss + e], p.scale_log2, -mref));
        uint4 pk;
        pk.x = pack2_bf16(pe[0], pe[1]);
        pk.y = pack2_bf16(pe[2], pe[3]);
        pk.z = pack2_bf16(pe[4], pe[5]);
        pk.w = pack2_bf16(pe[6], pe[7]);
        pop[rw][ss] = __builtin_bit_cast(bf16x8, pk);
        lacc[rw] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pop[rw][ss], lacc[rw], 0, 0, 0);
      }
    }
#pragma unroll
    for (int ss = 0; ss < SPS; ++ss) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        bf16x8 vop;
        if constexpr (kPrefetchV) {
          vop = vbuf[dt];
        } else {
          vop = vnext;
          if (dt + 1 < DT)
            vnext = read_v(ss, dt + 1);
          else if (ss + 1 < SPS)
            vnext = read_v(ss + 1, 0);
        }
#pragma unroll
        for (int rw = 0; rw < RW; ++rw)
          acc[rw][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[rw][ss], acc[rw][dt], 0, 0, 0);
        if constexpr (kPrefetchV) {
          if (ss + 1 < SPS) vbuf[dt] = read_v(ss + 1, dt);  // the next stage's operand, once this one is consumed
        }
      }
    }
  };

  // ---- main loop over the chunk's key tiles, SPS tiles per step. Tile t is requested NS - SPS tiles
  // ahead; every wave issues exactly PW loads per tile (past the end they read the zero row), so once the
  // step's tiles have landed exactly PW * (NS - 2 SPS) of the wave's loads may still be in flight. One
  // barrier per step publishes the tiles just landed and retires the slots about to be refilled (the
  // previous step's: their LDS reads have returned).
  const int ntile = (key_hi - key_lo + kTile - 1) / kTile;
#pragma unroll
  for (int i = 0; i < NS - SPS; ++i) issue(i, i);
#pragma unroll 1
  for (int t = 0; t < ntile; t += SPS) {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(PW * (NS - 2 * SPS)) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < SPS; ++j) {
      const int nt = t + NS - SPS + j;
      issue(nt, nt % NS);
    }
    if (active) {
      const int st = key_lo + t * kTile;
      compute(t, t % NS, !pages_ok || st + SPS * kTile > min(key_hi, L));
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the loads issued past the end

  float l_run[RW];
#pragma unroll
  for (int rw = 0; rw < RW; ++rw) l_run[rw] = lacc[rw][0];

  constexpr float kLn2 = 0.69314718055994530942f;
  // out / lse of one row tile from (m, l, O^T accumulator); lanes hold row (lane & 15), columns dt*16 + g4 + {0..3}
  auto finish = [&](int lt, float m, float ls, const f32x4 (&o)[DT]) {
    const int r = 16 * (t0 + lt) + l15;
    if (r >= M) return;
    const int i = r / p.G, h = g * p.G + (r - i * p.G);
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
    uint16_t* dst = p.out + ((size_t(b) * p.max_T + i) * p.Hq + h) * D + g4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4 v = o[dt] * inv;
      *reinterpret_cast<uint2*>(dst + 16 * dt) = make_uint2(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]));
    }
    if (p.lse && lane < 16)
      p.lse[(size_t(b) * p.max_T + i) * p.Hq + h] = ls > 0.f ? (m + __log2f(ls)) * kLn2 : -INFINITY;
  };

  if (n_items == 1) {  // the whole key range in one item: this is the answer
    if (active) {
#pragma unroll
      for (int rw = 0; rw < RW; ++rw) {
        const int lt = wave + NW * rw;
        if (lt < p.tpb && t0 + lt < ntM) finish(lt, m_run[rw], l_run[rw], acc[rw]);
      }
    }
    return;
  }

  // ---- this item's partial for the combine kernel: o = O / (l sc) in fp16 (the merge weights m and l stay
  // fp32, so its rounding, 2^-12 relative, stays below the bf16 output's own), reference max m, row sum l,
  // and sc, a power of two that keeps the row's |o| below 2^14 (1 unless |O / l| reaches 2^14: fp16 stops at
  // 65504). Layout per (b, g, row block, item): o fp16 [tpb * 16][D], then m, l, sc fp32 [tpb * 16] each.
  if (!active) return;
  const int TR = p.tpb * 16;
  const size_t ITEM = size_t(TR) * (D / 2 + 3);  // in floats
  float* const mine = p.part + ((size_t(bg) * p.n_rb + rb) * size_t(p.n_splits) + s) * ITEM;
#pragma unroll
  for (int rw = 0; rw < RW; ++rw) {
    const int lt = wave + NW * rw;
    if (lt >= p.tpb || t0 + lt >= ntM) continue;
    const int row = lt * 16 + l15;
    if (16 * (t0 + lt) + l15 >= M) continue;  // rows past this tree: never read
    uint16_t* o = reinterpret_cast<uint16_t*>(mine) + size_t(row) * D + g4;
    const float inv = l_run[rw] > 0.f ? 1.f / l_run[rw] : 0.f;
    float amax = 0.f;  // the row's largest |O|: this lane's columns, then the row's four lanes
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int k = 0; k < 4; ++k) amax = fmaxf(amax, fabsf(acc[rw][dt][k]));
    amax = lanegroup_max(amax) * inv;
    int ex = 0;
    (void)frexpf(amax, &ex);  // amax < 2^ex
    const float sc = ex > 14 ? ldexpf(1.f, ex - 14) : 1.f;
    const float mul = inv * (1.f / sc);  // sc is a power of two: exact
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<uint2*>(o + 16 * dt) = pack4_f16(acc[rw][dt] * mul);
    if (lane < 16) {
      mine[size_t(TR) * (D / 2) + row] = m_run[rw];
      mine[size_t(TR) * (D / 2 + 1) + row] = l_run[rw];
      mine[size_t(TR) * (D / 2 + 2) + row] = sc;
    }
  }
}

// ---------------------------------------------------------------- FP8-KV variant (d = 128)
// K and V pages hold OCP E4M3 codes with one fp32 scale per KV head; q is quantized per row to E4M3 with a power of
// two scale 2^e (the smallest e with max|q| <= 448 * 2^e), and both products run on the gfx950 E4M3 MFMA
// 16x16x128, which takes the whole head dim of 16 keys in one instruction:
//   S^T = K8 Q8^T   A = 16 keys x 128 bytes (lane: key l % 16, bytes 32 (l / 16) .. +31), B the same bytes of
//                   the lane's query row; any byte order shared by A and B gives the same dot products;
//   P^T             the 32 scores a lane holds per 128-key step (keys 16 u + 4 (l / 16) + i of its row) become
//                   E4M3 in place: the reference max lags the row max by at most 2^kTau = 256 < 448, so no
//                   scaling; the row sums come from an MFMA against all-ones codes, so l sums the rounded p;
//   O^T += V^T P^T  A = V^T: lane l needs column 16 dt + l % 16 of the same 32 keys, gathered by four
//                   transposing 8-byte LDS reads (in each 16-lane group, lane l receives byte l % 8 of the
//                   rows named by lanes (l / 8) % 2 + 2 m, m = 0..7).
// Scores carry the row's scale 2^e * k_scale[g] into the exponent; O is scaled by v_scale[g] at the end.
constexpr int kTile8 = 64;  // keys per ring stage (64 x 128 B of K, then of V)

// 16-byte chunk swizzles of one 128-byte row (8 chunks), per key:
//   K: c ^ ((key >> 1) & 7): the 16 keys of one A-operand read at one chunk hit 16 distinct 16-byte bank groups;
//   V: c ^ (((key >> 1) & 3) | ((key >> 4) & 1) << 2): the 16 keys each half-wave reads in one transposing read
//      ({0..7, 16..23} or {8..15, 24..31} + 32 t) hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int k8_swz(int key) { return (key >> 1) & 7; }
__device__ __forceinline__ int v8_swz(int key) { return ((key >> 1) & 3) | (((key >> 4) & 1) << 2); }

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

__device__ __forceinline__ f32x4 mfma_e4m3(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);  // E4M3 x E4M3, no block scale
}

// four fp32 -> four E4M3 codes in one dword (round to nearest even)
__device__ __forceinline__ int pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int NW, int NS>
__global__ void __launch_bounds__(64 * NW, NW / 4 * 2) tree_attn_fp8_kernel(AttnParams p) {
  constexpr int D = 128, DT = 8, ROWB = 128, CPR = 8;
  constexpr int TILE_B = kTile8 * ROWB;  // 8 KB of K (or V) per ring stage
  constexpr int STAGE_B = 2 * TILE_B;
  constexpr int NLD = TILE_B / 1024;     // 8 direct loads of 1 KB (8 rows) per stage and buffer
  constexpr int PW = 2 * NLD / NW;       // per wave and stage
  constexpr int PH = PW / 2;
  constexpr int NT = 64 * NW;
  constexpr int SPS = 2;                 // stages per softmax step: 128 keys, one MFMA k-block of P V
  static_assert(PW >= 2 && PW * NW == 2 * NLD, "each wave loads whole K/V row groups");
  static_assert(NS == 2 * SPS, "two steps in the ring");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[NS * STAGE_B];
  const uint32_t ring_lds = lds_addr(ring);
  __shared__ uint64_t anc_s[65];
  extern __shared__ int pg_s[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int s, rb, bg;
  if constexpr (NW == 8) {  // XCD-aware 1-D grid: a group's row blocks share one XCD's L2 (as the bf16 kernel)
    const int xcd = blockIdx.x & (kXcds - 1), slot = blockIdx.x / kXcds;
    const int grp = (slot / p.n_rb) * kXcds + xcd;
    if (grp >= p.n_groups) return;
    rb = slot - (slot / p.n_rb) * p.n_rb;
    bg = grp / p.n_splits;
    s = grp - bg * p.n_splits;
  } else {
    s = blockIdx.x;
    rb = blockIdx.y;
    bg = blockIdx.z;
  }
  const int b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int32_t* ptab = p.page_table + size_t(b) * p.max_pages;
  const int t0 = rb * p.tpb;
  const int l15 = lane & 15, lg = lane >> 4, g4 = 4 * lg;

  const int T_raw = p.T_b ? p.T_b[b] : p.max_T;
  const int L_raw = p.prefix_lens[b];
  const int pg0 = (s * p.chunk) >> p.page_shift;
  for (int i = tid; i < p.npg; i += NT) {
    const int pi = pg0 + i;
    pg_s[i] = pi < p.max_pages ? ptab[pi] : -1;
  }
  int par_raw = 0;
  if (tid < kWave && tid + 1 < p.max_T) par_raw = p.parents[size_t(b) * p.max_T + tid + 1];
  const float ksc = p.k_scale[g], vsc = p.v_scale[g];
  // this wave's row tile: lane = row l % 16, head-dim elements 32 lg .. 32 lg + 31, quantized to E4M3 with the
  // row's exponent (the row's four lanes agree on max|q|)
  const int r_own = 16 * (t0 + wave) + l15;
  i32x8 q8;
  float row_scale;
  {
    const bool ok = wave < p.tpb && r_own < p.G * p.max_T;
    const int rr = ok ? r_own : 0;
    const int i = rr / p.G, h = g * p.G + (rr - i * p.G);
    const uint16_t* src = p.q + ((size_t(b) * p.max_T + i) * p.Hq + h) * D + 32 * lg;
    float x[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 u = reinterpret_cast<const uint4*>(src)[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[8 * c + 2 * k] = ok ? __uint_as_float(w[k] << 16) : 0.f;
        x[8 * c + 2 * k + 1] = ok ? __uint_as_float(w[k] & 0xffff0000u) : 0.f;
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(x[k]));
    amax = lanegroup_max(amax);
    // smallest e with amax <= 448 * 2^e: amax = f 2^x with f in [1/2, 1) and 448 = 0.875 * 2^9
    int ex = 0;
    const float f = frexpf(amax, &ex);
    const int e = amax == 0.f ? 0 : (f <= 0.875f ? ex - 9 : ex - 8);
    row_scale = ldexpf(1.f, e);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      q8[k] = pack4_e4m3(ldexpf(x[4 * k], -e), ldexpf(x[4 * k + 1], -e), ldexpf(x[4 * k + 2], -e), ldexpf(x[4 * k + 3], -e));
  }
  __syncthreads();

  int T = min(max(T_raw, 1), p.max_T);
  int L = L_raw;
  const int cap = p.max_pages << p.page_shift;
  if (L < 0 || L > cap - T) {
    if (p.status && s == 0 && rb == 0 && g == 0 && tid == 0) atomicOr(p.status + b, SPEC_STATUS_INVALID_LENGTH);
    L = min(max(L, 0), cap - T);
  }
  const int M = p.G * T;
  const int ntM = (M + 15) >> 4;
  if (t0 >= ntM) return;
  const int n_items = (L + T + p.chunk - 1) / p.chunk;
  if (s >= n_items) return;
  const int key_lo = s * p.chunk;
  const int key_hi = min(L + T, key_lo + p.chunk);
  const bool has_tree = key_hi > L;

  bool bad = false;
  {
    const int npg_used = ((key_hi - 1) >> p.page_shift) - pg0 + 1;
    for (int i = tid; i < npg_used; i += NT) bad |= unsigned(pg_s[i]) >= unsigned(p.num_pages);
  }
  if (has_tree && tid < kWave) {  // ancestry words by pointer doubling over lanes (node n in lane n - 1)
    const int n = tid + 1;
    const bool real = n < T;
    int par = 0;
    if (real) {
      par = par_raw;
      if (par < 0 || par >= n) {
        par = 0;
        if (p.status && rb == 0 && g == 0) atomicOr(p.status + b, SPEC_STATUS_INVALID_PARENT);
      }
    }
    uint64_t a = real ? (1ull << tid) : 0ull;
    int jump = par;
    while (__ballot(jump != 0)) {
      const int src = jump > 0 ? jump - 1 : tid;
      const uint64_t pa = (uint64_t(uint32_t(__shfl(int(a >> 32), src))) << 32) | uint32_t(__shfl(int(a), src));
      const int pj = __shfl(jump, src);
      if (jump != 0) {
        a |= pa;
        jump = pj;
      }
    }
    if (real) anc_s[n] = a;
    if (tid == 0) anc_s[0] = 0;
  }
  const bool pages_ok = !__syncthreads_or(bad);
  if (!pages_ok && p.status && tid == 0) atomicOr(p.status + b, SPEC_STATUS_INVALID_PAGE);
  // the row's ancestry word stays in LDS (read in masked steps only); rows past the tree see the prefix and root
  const int anc_idx = (has_tree && r_own < M) ? r_own / p.G : 0;
  const bool active = wave < p.tpb && t0 + wave < ntM;
  const float c_row = p.scale_log2 * row_scale * ksc;  // log2-domain factor of this lane's raw scores

  float m_run = -INFINITY;
  f32x4 acc[DT], lacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const i32x8 ones8 = {0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838};

  const int pmask = (1 << p.page_shift) - 1;
  const size_t tok_stride = size_t(p.Hkv) * D;  // bytes between consecutive slots of a page
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k) + size_t(g) * D;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v) + size_t(g) * D;
  const uint8_t* zeros = reinterpret_cast<const uint8_t*>(p.zeros);
  const size_t page_bytes = tok_stride << p.page_shift;
  int lkey[PH], koff[PH], voff[PH];
#pragma unroll
  for (int i = 0; i < PH; ++i) {
    lkey[i] = (wave + NW * i) * 8 + lane / CPR;
    const int pos = lane % CPR;
    koff[i] = 16 * (pos ^ k8_swz(lkey[i]));
    voff[i] = 16 * (pos ^ v8_swz(lkey[i]));
  }
  auto issue = [&](int tile, int slot) {
    const int st = key_lo + tile * kTile8;
    const uint32_t sb = ring_lds + slot * STAGE_B;
    const bool full = pages_ok && st + kTile8 <= key_hi;
#pragma unroll
    for (int i = 0; i < PH; ++i) {
      const int slot_k = st + lkey[i];
      const uint8_t *ks, *vs;
      if (full) {
        const int phys = pg_s[(slot_k >> p.page_shift) - pg0];
        const size_t off = size_t(uint32_t(phys)) * page_bytes + size_t((slot_k & pmask) * tok_stride);
        ks = kbase + off + koff[i];
        vs = vbase + off + voff[i];
      } else {
        const bool in = slot_k < key_hi;
        const int phys = pg_s[in ? (slot_k >> p.page_shift) - pg0 : 0];
        const bool ok = in && unsigned(phys) < unsigned(p.num_pages);
        const size_t off = size_t(uint32_t(phys)) * page_bytes + size_t((slot_k & pmask) * tok_stride);
        ks = ok ? kbase + off + koff[i] : zeros + koff[i];
        vs = ok ? vbase + off + voff[i] : zeros + voff[i];
      }
      const int sub = wave + NW * i;
      load_to_lds16(ks, sb + sub * 1024);
      load_to_lds16(vs, sb + TILE_B + sub * 1024);
    }
  };

  // one 128-key step (ring stages slot, slot + 1)
  auto compute = [&](int tile, int slot, bool masked) {
    const int st = key_lo + tile * kTile8;
    auto key_of = [&](int e) { return st + 16 * (e >> 2) + g4 + (e & 3); };  // lane score e <-> key
    f32x4 sc[8];
    auto read_k = [&](int u) {  // A operand of key tile u (16 keys): key l15, chunks 2 lg and 2 lg + 1
      const int key = 16 * (u & 3) + l15;
      const unsigned char* kr = ring + ((slot + (u >> 2)) % NS) * STAGE_B + key * ROWB;
      const uint4 a = *reinterpret_cast<const uint4*>(kr + 16 * ((2 * lg) ^ k8_swz(key)));
      const uint4 c = *reinterpret_cast<const uint4*>(kr + 16 * ((2 * lg + 1) ^ k8_swz(key)));
      return i32x8{int(a.x), int(a.y), int(a.z), int(a.w), int(c.x), int(c.y), int(c.z), int(c.w)};
    };
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      sc[u] = mfma_e4m3(read_k(u), q8, f32x4{0.f, 0.f, 0.f, 0.f});
      if (u % 2 == 1) __builtin_amdgcn_sched_barrier(0);  // at most two K fragments (16 registers) in flight
    }
    uint32_t vis = 0xffffffffu;
    if (masked) {  // uniform: the chunk's end, tree slots outside the row's ancestry
      // the lane's keys come in 8 groups of 4 consecutive keys (u): tree nodes j0 .. j0 + 3 with j0 = base + 16 u;
      // node <= 0 (prefix, root) is visible, node j >= 1 iff bit j - 1 of the row's ancestry word
      vis = 0;
      const uint64_t ranc = anc_s[anc_idx];
      const int base = st + g4 - L;
      const int lim = key_hi - st - g4;  // keys 16 u + i < lim lie in the chunk
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j0 = base + 16 * u;
        uint32_t a4;
        if (j0 >= 1)
          a4 = j0 <= 64 ? uint32_t(ranc >> (j0 - 1)) & 0xFu : 0u;
        else if (j0 <= -3)
          a4 = 0xFu;
        else
          a4 = ((1u << (1 - j0)) - 1u) | ((uint32_t(ranc) << (1 - j0)) & 0xFu);
        const int cnt = min(max(lim - 16 * u, 0), 4);
        vis |= (a4 & ((1u << cnt) - 1u)) << (4 * u);
      }
      if (!pages_ok) {  // uniform and rare: keys on pages outside the pool, one lookup at a time
#pragma unroll 1
        for (int e = 0; e < 32; ++e) {
          const int key = key_of(e);
          if (key < key_hi && unsigned(pg_s[(key >> p.page_shift) - pg0]) >= unsigned(p.num_pages)) vis &= ~(1u << e);
        }
      }
    }
    if (masked) {  // scores of invisible keys -> -inf, in place
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        float x = ((vis >> e) & 1u) ? sc[e >> 2][e & 3] : -INFINITY;
        asm volatile("" : "+v"(x));
        sc[e >> 2][e & 3] = x;
      }
    }
    float mx = sc[0][0];
#pragma unroll
    for (int e = 1; e < 32; ++e) mx = fmaxf(mx, sc[e >> 2][e & 3]);
    mx = lanegroup_max(mx);
    const float mxs = mx * c_row;
    const bool move = mxs > m_run + kTau;
    if (__any(move)) {
      const float mnew = move ? mxs : m_run;
      const float alpha = move ? fast_exp2(m_run - mnew) : 1.f;
      lacc *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
      m_run = mnew;
    }
    const float mref = m_run == -INFINITY ? 0.f : m_run;
    i32x8 pop;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float pe[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pe[j] = fast_exp2(__builtin_fmaf(sc[k][j], c_row, -mref));
      pop[k] = pack4_e4m3(pe[0], pe[1], pe[2], pe[3]);
    }
    lacc = mfma_e4m3(ones8, pop, lacc);
    // the V reads stay behind the softmax (hoisted above it they would hold 64 registers across it)
    __builtin_amdgcn_sched_barrier(0);
    // V^T operand, column 16 dt + l15: read t covers keys 32 t' + 16 (m >> 2) + g4 + (m & 3) of stage slot + t / 2
    // (t' = t % 2); lane r of each 16-lane group names key (r >> 1) at column half r & 1
    const int mr = l15 >> 1, half = l15 & 1;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      i32x8 vop;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int key = 32 * (t & 1) + 16 * (mr >> 2) + g4 + (mr & 3);
        const unsigned char* vb = ring + ((slot + (t >> 1)) % NS) * STAGE_B + TILE_B + key * ROWB;
        const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vb + 16 * (dt ^ v8_swz(key)) + 8 * half));
        vop[2 * t] = w[0];
        vop[2 * t + 1] = w[1];
      }
      acc[dt] = mfma_e4m3(vop, pop, acc[dt]);
      if (dt % 2 == 1) __builtin_amdgcn_sched_barrier(0);  // at most two columns' V operands in flight
    }
  };

  const int ntile = (key_hi - key_lo + kTile8 - 1) / kTile8;
#pragma unroll
  for (int i = 0; i < NS - SPS; ++i) issue(i, i);
#pragma unroll 1
  for (int t = 0; t < ntile; t += SPS) {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(PW * (NS - 2 * SPS)) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < SPS; ++j) {
      const int nt = t + NS - SPS + j;
      issue(nt, nt % NS);
    }
    if (active) {
      const int st = key_lo + t * kTile8;
      compute(t, t % NS, !pages_ok || st + SPS * kTile8 > min(key_hi, L));
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const float l_run = lacc[0];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] *= vsc;
  constexpr float kLn2 = 0.69314718055994530942f;
  if (!active || r_own >= M) return;
  const int i_node = r_own / p.G, h = g * p.G + (r_own - i_node * p.G);
  if (n_items == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* dst = p.out + ((size_t(b) * p.max_T + i_node) * p.Hq + h) * D + g4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4 v = acc[dt] * inv;
      *reinterpret_cast<uint2*>(dst + 16 * dt) = make_uint2(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]));
    }
    if (p.lse && lane < 16)
      p.lse[(size_t(b) * p.max_T + i_node) * p.Hq + h] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
    return;
  }
  // partial of this item, in the layout the combine kernel reads (o fp16 = O / (l sc), m, l, sc)
  const int TR = p.tpb * 16;
  const size_t ITEM = size_t(TR) * (D / 2 + 3);
  float* const mine = p.part + ((size_t(bg) * p.n_rb + rb) * size_t(p.n_splits) + s) * ITEM;
  const int row = wave * 16 + l15;
  uint16_t* o = reinterpret_cast<uint16_t*>(mine) + size_t(row) * D + g4;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float amax = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int k = 0; k < 4; ++k) amax = fmaxf(amax, fabsf(acc[dt][k]));
  amax = lanegroup_max(amax) * inv;
  int ex = 0;
  (void)frexpf(amax, &ex);
  const float sc = ex > 14 ? ldexpf(1.f, ex - 14) : 1.f;
  const float mul = inv * (1.f / sc);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<uint2*>(o + 16 * dt) = pack4_f16(acc[dt] * mul);
  if (lane < 16) {
    mine[size_t(TR) * (D / 2) + row] = m_run;
    mine[size_t(TR) * (D / 2 + 1) + row] = l_run;
    mine[size_t(TR) * (D / 2 + 2) + row] = sc;
  }
}

// Split-K combine (runs after the main kernel): one wave per block, D / 4 threads per row (4 columns
// each), so a block holds 64 / (D / 4) rows and the grid spreads the partials over many CUs. Rows that
// no tree of the batch can have (r >= G * max_T) exit before any load. The first CB items' partials
// are loaded in the same round trip as the sequence's lengths (loads of items the sequence does not
// have read workspace memory and are never used), so short sequences finish in one round trip. Items
// are combined in fixed order, online against the running maximum reference max:
// out = sum_i w_i O_i / sum_i w_i l_i with w_i = 2^(m_i - max_j m_j). Sequences whose keys fit one
// item were written directly by the main kernel.
// KNOWN: the lengths are loaded first and only the sequence's own items are read (one more round trip,
// used for batches of many sequences, whose lengths may differ: a short sequence then reads its one or
// two items instead of every slot of the longest).
// rows of partials per 64-thread combine block (D / 8 threads per row, 8 columns each)
constexpr int combine_rpb(int D) { return 64 / (D / 8); }

template <int D, bool KNOWN>
__global__ void __launch_bounds__(64) tree_attn_combine(AttnParams p) {
  constexpr int TPR = D / 8;     // threads per row (8 columns each)
  constexpr int RPB = combine_rpb(D);
  constexpr int CB = 16;         // items per batch at most
  const int tid = threadIdx.x;
  const int rsub = tid / TPR, c = tid - rsub * TPR;
  const int rbg = blockIdx.y;
  const int bg = rbg / p.n_rb, rb = rbg - bg * p.n_rb;
  const int b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int TR = p.tpb * 16;
  const int row = blockIdx.x * RPB + rsub;  // row of this row block's partials
  const int r = rb * TR + row;               // packed row (node r / G, head g G + r % G)
  if (row >= TR || r >= p.G * p.max_T) return;
  const int T_raw = p.T_b ? p.T_b[b] : p.max_T;
  const int L_raw = p.prefix_lens[b];
  const size_t ITEM = size_t(TR) * (D / 2 + 3);  // in floats: o fp16 [TR][D], m, l, sc [TR]
  const float* grp = p.part + size_t(rbg) * p.n_splits * ITEM;
  RowMerge mr;
  // n_items: the sequence's item count (KNOWN: loaded before the items), else the first batch's loads go
  // out with the lengths, clamped to the call's split count, and the count is known after them. Slots past
  // the last item repeat a loaded one (never folded), so the batch size CBV follows the count that bounds
  // it (4, 8, 12 or 16): fewer wasted load instructions for sequences with few items
  auto merge = [&](auto cbv, int n_items) {
    constexpr int CBV = decltype(cbv)::value;
#pragma unroll 1
    for (int ib = 0; ib < n_items; ib += CBV) {
      float mi[CBV], li[CBV];
      f32x8 ai[CBV];
#pragma unroll
      for (int u = 0; u < CBV; ++u) {
        const int item = KNOWN ? min(ib + u, n_items - 1) : min(ib + u, p.n_splits - 1);
        const float* base = grp + size_t(item) * ITEM;
        mi[u] = base[size_t(TR) * (D / 2) + row];
        li[u] = base[size_t(TR) * (D / 2 + 1) + row];
        const float scu = base[size_t(TR) * (D / 2 + 2) + row];
        const uint4 h = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + size_t(row) * D + 8 * c);
        ai[u] = __builtin_convertvector(__builtin_bit_cast(f16x8, h), f32x8) * scu;
      }
      if (!KNOWN && ib == 0) {
        const int T = min(max(T_raw, 1), p.max_T);
        const int cap = p.max_pages << p.page_shift;
        const int L = min(max(L_raw, 0), cap - T);  // the main kernel's clamp
        n_items = (L + T + p.chunk - 1) / p.chunk;
        if (n_items == 1 || r >= p.G * T) return false;
      }
      mr.fold<CBV>(mi, li, ai, n_items - ib);
    }
    return true;
  };
  int n_items = p.n_splits;  // an upper bound until the lengths are known
  if constexpr (KNOWN) {
    const int T = min(max(T_raw, 1), p.max_T);
    const int cap = p.max_pages << p.page_shift;
    const int L = min(max(L_raw, 0), cap - T);  // the main kernel's clamp
    n_items = (L + T + p.chunk - 1) / p.chunk;
    if (n_items == 1 || r >= p.G * T) return;
  }
  bool done;
  if (n_items <= 4)
    done = merge(std::integral_constant<int, 4>{}, n_items);
  else if (n_items <= 8)
    done = merge(std::integral_constant<int, 8>{}, n_items);
  else if (n_items <= 12)
    done = merge(std::integral_constant<int, 12>{}, n_items);
  else
    done = merge(std::integral_constant<int, CB>{}, n_items);
  if (!done) return;
  mr.write<D>(p, b, g, r, c);
}

struct AttnShape {
  int NW, RW, NS, SPS;
};

struct AttnPlan {
  AttnShape sh;
  int G, tiles, n_rb, tpb, chunk, n_splits, npg;
  size_t zero_bytes, part_bytes, lds_dyn;
};

// fp8: the FP8-KV kernel's shape (one row tile per wave, 4-stage ring; only the wave count is chosen here)
AttnPlan make_plan(int B, int max_T, int Hq, int Hkv, int d, int page, int max_pages, bool fp8 = false) {
  AttnPlan pl;
  pl.G = Hq / Hkv;
  pl.tiles = (pl.G * max_T + 15) / 16;
  // waves x row tiles per wave (one tile per wave; two only on 4-wave blocks, which have the registers)
  // two 32-key stages per softmax step at d = 128 (the d = 64 kernels take one)
  pl.sh = pl.tiles <= 4 ? AttnShape{4, 1, 4, d == 128 ? 2 : 1} : AttnShape{8, 1, 4, d == 128 ? 2 : 1};
  if (const char* env = getenv("SPEC_TREE_ATTN_SHAPE")) {  // "NW,RW,NS[,SPS]" for sweeps
    int nw = 0, rw = 0, ns = 0, sps = 1;
    const int n = sscanf(env, "%d,%d,%d,%d", &nw, &rw, &ns, &sps);
    const bool single = (nw == 4 || nw == 8) && (rw == 1 || (rw == 2 && nw == 4)) && (ns == 3 || ns == 4) && sps == 1;
    const bool pair = ((rw == 1 && (nw == 4 || nw == 8) && (ns == 4 || ns == 6 || ns == 8)) ||
                       (rw == 2 && ((nw == 4 && ns == 4) || (nw == 8 && (ns == 6 || ns == 8))))) && sps == 2;
    if (n >= 3 && (single || pair)) pl.sh = AttnShape{nw, rw, ns, sps};
  }
  if (d == 64) pl.sh.NW = 4;
  if (fp8) pl.sh = AttnShape{pl.sh.NW, 1, 4, 2};
  const int cap = pl.sh.NW * pl.sh.RW;
  pl.n_rb = (pl.tiles + cap - 1) / cap;
  pl.tpb = (pl.tiles + pl.n_rb - 1) / pl.n_rb;  // row tiles spread evenly over the row blocks
  const long long slots = (long long)max_pages * page;
  const long long groups = (long long)B * Hkv * pl.n_rb;
  const long long target = pl.sh.NW == 8 ? kTargetBlocks8 : kTargetBlocks;
  long long n = (target + groups - 1) / groups;  // items per (b, g, row block)
  long long chunk = (slots + n - 1) / n;
  if (const char* env = getenv("SPEC_TREE_ATTN_CHUNK")) {
    const long long c = atoll(env);
    if (c >= kTile) chunk = c;
  }
  // any chunk length works (every lane looks up its own key's page); an unrounded chunk keeps a
  // sequence's items equal, so no XCD is left with all the short tails
  chunk = std::max<long long>(chunk, 4 * kTile);
  chunk = std::min<long long>(chunk, kMaxChunk);
  pl.chunk = int(chunk);
  pl.n_splits = int((slots + chunk - 1) / chunk);
  pl.npg = int((chunk - 1) / page) + 2;  // a chunk may straddle one page more than it covers
  const size_t item = size_t(pl.tpb) * 16 * (d / 2 + 3);  // floats: o fp16 [rows][d], m, l, sc
  pl.zero_bytes = 1024;  // never written: stays as zero-filled as the caller provided it
  pl.part_bytes = align_up(size_t(groups) * pl.n_splits * item * sizeof(float), 256);
  pl.lds_dyn = size_t(pl.npg) * sizeof(int);
  return pl;
}

template <int D, int NW, int RW>
void launch_ns(const AttnPlan& pl, const AttnParams& prm, dim3 grid, hipStream_t st) {
  if constexpr (D == 128 && RW == 2) {  // two row tiles per wave, two-stage steps
    if (pl.sh.SPS == 2) {
      if constexpr (NW == 8) {  // one block per CU (256 registers per lane)
        if (pl.sh.NS == 8)
          hipLaunchKernelGGL((tree_attn_kernel<D, NW, RW, 8, 2>), grid, dim3(64 * NW), pl.lds_dyn, st, prm);
        else
          hipLaunchKernelGGL((tree_attn_kernel<D, NW, RW, 6, 2>), grid, dim3(64 * NW), pl.lds_dyn, st, prm);
      } else {
        hipLaunchKernelGGL((tree_attn_kernel<D, NW, RW, 4, 2>), grid, dim3(64 * NW), pl.lds_dyn, st, prm);
      }
      return;
    }
  }
  if constexpr (D == 128 && RW == 1) {  // two-stage steps
    if (pl.sh.SPS == 2) {
      if (pl.sh.NS == 8)
        hipLaunchKernelGGL((tree_attn_kernel<D, NW, RW, 8, 2>), grid, dim3(64 * NW), pl.lds_dyn, st, prm);
      else if (pl.sh.NS == 6)
        hipLaunchKernelGGL((tree_attn_kernel<D, NW, RW, 6, 2>), grid, dim3(64 * NW), pl.lds_dyn, st, prm);
      else
        hipLaunchKernelGGL((tree_attn_kernel<D, NW, RW, 4, 2>), grid, dim3(64 * NW), pl.lds_dyn, st, prm);
      return;
    }
  }
  if constexpr (NW == 4 || RW == 1) {  // one-stage steps (8-wave blocks have the registers for one row tile only)
    if (pl.sh.NS == 3)
      hipLaunchKernelGGL((tree_attn_kernel<D, NW, RW, 3, 1>), grid, dim3(64 * NW), pl.lds_dyn, st, prm);
    else
      hipLaunchKernelGGL((tree_attn_kernel<D, NW, RW, 4, 1>), grid, dim3(64 * NW), pl.lds_dyn, st, prm);
  }
}

template <int D>
void launch_d(const AttnPlan& pl, const AttnParams& prm, dim3 grid, hipStream_t st) {
  if constexpr (D == 64) {  // a 32-key stage of d = 64 holds 4 K/V row pairs: at most 4 loading waves
    if (pl.sh.RW == 1)
      launch_ns<D, 4, 1>(pl, prm, grid, st);
    else
      launch_ns<D, 4, 2>(pl, prm, grid, st);
  } else {
    if (pl.sh.NW == 4 && pl.sh.RW == 1)
      launch_ns<D, 4, 1>(pl, prm, grid, st);
    else if (pl.sh.NW == 4)
      launch_ns<D, 4, 2>(pl, prm, grid, st);
    else if (pl.sh.RW == 2)
      launch_ns<D, 8, 2>(pl, prm, grid, st);
    else
      launch_ns<D, 8, 1>(pl, prm, grid, st);
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
  if ((long long)Hkv * d * 2 * page >= (1LL << 31))
    return fail(SPEC_E_UNSUPPORTED, "spec_tree_attention: a page of Hkv=%d heads x %d slots spans 2^31 bytes or more", Hkv, page);
  return SPEC_OK;
}

}  // namespace
}  // namespace spectree

using namespace spectree;

extern "C" size_t spec_tree_attention_workspace_size(int32_t B, int32_t max_T, int32_t Hq, int32_t Hkv, int32_t d,
                                                     int32_t page, int32_t max_pages) {
  if (check_shapes(B, max_T, Hq, Hkv, d, page, max_pages) != SPEC_OK) return 0;
  const AttnPlan pl = make_plan(B, max_T, Hq, Hkv, d, page, max_pages);
  return pl.zero_bytes + pl.part_bytes;
}

// argument checks of both attention entry points (everything but the workspace), and the call's plan
static int32_t attention_validate(const char* who, const void* q, const void* k_pages, const void* v_pages,
                                  const int32_t* page_table, const int32_t* prefix_lens, const int32_t* parents, int32_t B,
                                  int32_t max_T, int32_t Hq, int32_t Hkv, int32_t d, int32_t page, int32_t max_pages,
                                  int32_t num_pages, float sm_scale, void* out, AttnPlan* pl, bool fp8 = false) {
  int32_t rc = check_shapes(B, max_T, Hq, Hkv, d, page, max_pages);
  if (rc != SPEC_OK) return rc;
  if (!q || !k_pages || !v_pages || !page_table || !prefix_lens || !parents || !out)
    return fail(SPEC_E_INVAL, "%s: null tensor pointer", who);
  if (num_pages < 1) return fail(SPEC_E_INVAL, "%s: num_pages=%d", who, num_pages);
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(SPEC_E_INVAL, "%s: sm_scale must be finite and > 0", who);
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pages) | reinterpret_cast<uintptr_t>(v_pages) |
       reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(SPEC_E_INVAL, "%s: q, k_pages, v_pages and out must be 16-byte aligned", who);
  *pl = make_plan(B, max_T, Hq, Hkv, d, page, max_pages, fp8);
  return SPEC_OK;
}

static int32_t attention_launch(const AttnPlan& pl, const void* q, const void* k_pages, const void* v_pages,
                                const int32_t* page_table, const int32_t* prefix_lens, const int32_t* parents,
                                const int32_t* T_b, int32_t B, int32_t max_T, int32_t Hq, int32_t Hkv, int32_t d,
                                int32_t page, int32_t max_pages, int32_t num_pages, float sm_scale, void* out, float* lse,
                                uint32_t* status, void* ws, hipStream_t st, const float* k_scale = nullptr,
                                const float* v_scale = nullptr);

extern "C" int32_t spec_tree_attention(const void* q, const void* k_pages, const void* v_pages, const int32_t* page_table,
                                       const int32_t* prefix_lens, const int32_t* parents, const int32_t* T_b, int32_t B,
                                       int32_t max_T, int32_t Hq, int32_t Hkv, int32_t d, int32_t page, int32_t max_pages,
                                       int32_t num_pages, float sm_scale, void* out, float* lse, uint32_t* status, void* ws,
                                       size_t ws_bytes, void* stream) {
  AttnPlan pl;
  const int32_t rc = attention_validate("spec_tree_attention", q, k_pages, v_pages, page_table, prefix_lens, parents, B,
                                        max_T, Hq, Hkv, d, page, max_pages, num_pages, sm_scale, out, &pl);
  if (rc != SPEC_OK) return rc;
  const size_t need = pl.zero_bytes + pl.part_bytes;
  if (!ws || ws_bytes < need) return fail(SPEC_E_WORKSPACE, "spec_tree_attention: workspace %zu bytes < %zu", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 15) return fail(SPEC_E_INVAL, "spec_tree_attention: ws must be 16-byte aligned");
  return attention_launch(pl, q, k_pages, v_pages, page_table, prefix_lens, parents, T_b, B, max_T, Hq, Hkv, d, page,
                          max_pages, num_pages, sm_scale, out, lse, status, ws, static_cast<hipStream_t>(stream));
}

// k_scale / v_scale non-null: the FP8-KV kernel (E4M3 pages, d = 128)
extern "C" int32_t spec_tree_attention_fp8(const void* q, const void* k_pages, const void* v_pages,
                                           const float* k_scale, const float* v_scale, const int32_t* page_table,
                                           const int32_t* prefix_lens, const int32_t* parents, const int32_t* T_b,
                                           int32_t B, int32_t max_T, int32_t Hq, int32_t Hkv, int32_t d, int32_t page,
                                           int32_t max_pages, int32_t num_pages, float sm_scale, void* out, float* lse,
                                           uint32_t* status, void* ws, size_t ws_bytes, void* stream) {
  if (d != 128) return fail(SPEC_E_UNSUPPORTED, "spec_tree_attention_fp8: head dim %d (only 128)", d);
  AttnPlan pl;
  const int32_t rc = attention_validate("spec_tree_attention_fp8", q, k_pages, v_pages, page_table, prefix_lens, parents,
                                        B, max_T, Hq, Hkv, d, page, max_pages, num_pages, sm_scale, out, &pl, true);
  if (rc != SPEC_OK) return rc;
  if (!k_scale || !v_scale) return fail(SPEC_E_INVAL, "spec_tree_attention_fp8: null scale pointer");
  const size_t need = pl.zero_bytes + pl.part_bytes;
  if (!ws || ws_bytes < need)
    return fail(SPEC_E_WORKSPACE, "spec_tree_attention_fp8: workspace %zu bytes < %zu", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) & 15) return fail(SPEC_E_INVAL, "spec_tree_attention_fp8: ws must be 16-byte aligned");
  return attention_launch(pl, q, k_pages, v_pages, page_table, prefix_lens, parents, T_b, B, max_T, Hq, Hkv, d, page,
                          max_pages, num_pages, sm_scale, out, lse, status, ws, static_cast<hipStream_t>(stream), k_scale,
                          v_scale);
}

static int32_t attention_launch(const AttnPlan& pl, const void* q, const void* k_pages, const void* v_pages,
                                const int32_t* page_table, const int32_t* prefix_lens, const int32_t* parents,
                                const int32_t* T_b, int32_t B, int32_t max_T, int32_t Hq, int32_t Hkv, int32_t d,
                                int32_t page, int32_t max_pages, int32_t num_pages, float sm_scale, void* out, float* lse,
                                uint32_t* status, void* ws, hipStream_t st, const float* k_scale, const float* v_scale) {
  const bool fp8 = k_scale != nullptr;
  AttnParams prm;
  prm.k_scale = k_scale;
  prm.v_scale = v_scale;
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
  prm.tpb = pl.tpb;
  prm.npg = pl.npg;
  prm.scale_log2 = sm_scale * 1.4426950408889634f;
  prm.n_groups = B * Hkv * pl.n_splits;
  const dim3 grid = pl.sh.NW == 8 ? dim3(unsigned((prm.n_groups + kXcds - 1) / kXcds * kXcds * pl.n_rb))
                                  : dim3(pl.n_splits, pl.n_rb, B * Hkv);
  const int rows_used = std::min(pl.tpb * 16, pl.G * max_T);  // rows of a row block any tree can have
  // many sequences with many item slots: read each sequence's own items only (mixed-length batch of 32:
  // the combine read 352 MB for 170 MB of partials)
  const bool known = B >= 8 && pl.n_splits >= 8;
  if (d == 64) {
    launch_d<64>(pl, prm, grid, st);
    const dim3 cgrid(unsigned((rows_used + combine_rpb(64) - 1) / combine_rpb(64)), unsigned(pl.n_rb * B * Hkv));
    if (pl.n_splits > 1) {
      if (known)
        hipLaunchKernelGGL((tree_attn_combine<64, true>), cgrid, dim3(64), 0, st, prm);
      else
        hipLaunchKernelGGL((tree_attn_combine<64, false>), cgrid, dim3(64), 0, st, prm);
    }
  } else {
    if (!fp8)
      launch_d<128>(pl, prm, grid, st);
    else if (pl.sh.NW == 8)
      hipLaunchKernelGGL((tree_attn_fp8_kernel<8, 4>), grid, dim3(512), pl.lds_dyn, st, prm);
    else
      hipLaunchKernelGGL((tree_attn_fp8_kernel<4, 4>), grid, dim3(256), pl.lds_dyn, st, prm);
    const dim3 cgrid(unsigned((rows_used + combine_rpb(128) - 1) / combine_rpb(128)), unsigned(pl.n_rb * B * Hkv));
    if (pl.n_splits > 1) {
      if (known)
        hipLaunchKernelGGL((tree_attn_combine<128, true>), cgrid, dim3(64), 0, st, prm);
      else
        hipLaunchKernelGGL((tree_attn_combine<128, false>), cgrid, dim3(64), 0, st, prm);
    }
  }
  return check_launch("spec_tree_attention");
}

// ---------------------------------------------------------------- no-allocation entry point
// The split-K workspace in a library-held device array: `scratch` (kScratchBytes, zero at load). Host code
// never passes the array's name to a kernel: it takes the array's address on each device once, with that
// device current, through hipGetSymbolAddress, and uses that address.
namespace spectree {
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

__global__ void __launch_bounds__(256) zero_fill_kernel(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}
}  // namespace
}  // namespace spectree

static __device__ __align__(256) unsigned char scratch[spectree::kScratchBytes];

// the current device's address of `scratch` (looked up on the device's first call, then kept)
static int32_t scratch_address(const char* who, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(SPEC_E_DEVICE, "%s: no usable current device (%s)", who, hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(SPEC_E_DEVICE, "%s: hipGetSymbolAddress(scratch): %s", who, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SPEC_OK;
}

extern "C" int32_t spec_tree_attention_noalloc(const void* q, const void* k_pages, const void* v_pages,
                                               const int32_t* page_table, const int32_t* prefix_lens,
                                               const int32_t* parents, const int32_t* T_b, int32_t B, int32_t max_T,
                                               int32_t Hq, int32_t Hkv, int32_t d, int32_t page, int32_t max_pages,
                                               int32_t num_pages, float sm_scale, void* out, float* lse,
                                               uint32_t* status, void* stream) {
  const char* who = "spec_tree_attention_noalloc";
  AttnPlan pl;
  int32_t rc = attention_validate(who, q, k_pages, v_pages, page_table, prefix_lens, parents, B, max_T, Hq, Hkv, d, page,
                                  max_pages, num_pages, sm_scale, out, &pl);
  if (rc != SPEC_OK) return rc;
  const size_t need = pl.zero_bytes + pl.part_bytes;
  if (need > kScratchBytes)
    return fail(SPEC_E_WORKSPACE, "%s: this call needs %zu bytes of split-K scratch; the library holds %zu per device "
                "(use spec_tree_attention with a workspace)", who, need, kScratchBytes);
  void* ws = nullptr;
  rc = scratch_address(who, &ws);
  if (rc != SPEC_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the zero row the kernels read for masked loads: never written, cleared anyway (a kernel, so the call
  // stays capturable)
  hipLaunchKernelGGL(zero_fill_kernel, dim3(1), dim3(256), 0, st, static_cast<uint32_t*>(ws), int(pl.zero_bytes / 4));
  return attention_launch(pl, q, k_pages, v_pages, page_table, prefix_lens, parents, T_b, B, max_T, Hq, Hkv, d, page,
                          max_pages, num_pages, sm_scale, out, lse, status, ws, st);
}
