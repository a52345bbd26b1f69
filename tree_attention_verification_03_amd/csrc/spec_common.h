// Device helpers shared by the libspectree kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spectree {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// round-to-nearest-even fp32 -> bf16 (NaN -> quiet NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// ---------------------------------------------------------------- ordering keys
// Monotone map fp32 -> uint32 (larger float -> larger key) for finite values
// and +-inf; callers canonicalise NaN and -0 first.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Same for fp64.
__device__ __forceinline__ uint64_t f64_order_key(double f) {
  uint64_t u = uint64_t(__double_as_longlong(f));
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// ---------------------------------------------------------------- wave reductions
// All-reduce butterflies on VALU data movement only (no LDS round trips): DPP quad permutes pair lanes
// l ^ 1 and l ^ 2, row_half_mirror pairs the two quads of each 8 lanes, row_mirror the two halves of
// each 16, and the gfx950 row swaps exchange 16-lane rows and 32-lane halves (every lane finds its
// partner's value in one of the two swap results). Associative, commutative ops only.
namespace dpp {
constexpr int kXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kHalfMirror = 0x141; // row_half_mirror
constexpr int kMirror = 0x140;     // row_mirror
}  // namespace dpp

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(v), CTRL, 0xf, 0xf, false));
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return (uint64_t(dpp_u32<CTRL>(uint32_t(v >> 32))) << 32) | dpp_u32<CTRL>(uint32_t(v));
}

// op(value, partner value) over the xor-16 and xor-32 partners via the row swaps
template <typename Op>
__device__ __forceinline__ uint32_t swap_reduce_u32(uint32_t v, Op op) {
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(uint32_t(a[0]), uint32_t(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(uint32_t(c[0]), uint32_t(c[1]));
}

template <typename Op>
__device__ __forceinline__ uint64_t swap_reduce_u64(uint64_t v, Op op) {
  uint32_t lo = uint32_t(v), hi = uint32_t(v >> 32);
  const auto al = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto ah = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  v = op((uint64_t(uint32_t(ah[0])) << 32) | uint32_t(al[0]), (uint64_t(uint32_t(ah[1])) << 32) | uint32_t(al[1]));
  lo = uint32_t(v);
  hi = uint32_t(v >> 32);
  const auto cl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto ch = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  return op((uint64_t(uint32_t(ch[0])) << 32) | uint32_t(cl[0]), (uint64_t(uint32_t(ch[1])) << 32) | uint32_t(cl[1]));
}

template <typename Op>
__device__ __forceinline__ uint64_t wave_reduce_u64(uint64_t v, Op op) {
  v = op(v, dpp_u64<dpp::kXor1>(v));
  v = op(v, dpp_u64<dpp::kXor2>(v));
  v = op(v, dpp_u64<dpp::kHalfMirror>(v));
  v = op(v, dpp_u64<dpp::kMirror>(v));
  return swap_reduce_u64(v, op);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  return wave_reduce_u64(v, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  return wave_reduce_u64(v, [](uint64_t a, uint64_t b) { return a + b; });
}

__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return a | b; };
  v = op(v, dpp_u32<dpp::kXor1>(v));
  v = op(v, dpp_u32<dpp::kXor2>(v));
  v = op(v, dpp_u32<dpp::kHalfMirror>(v));
  v = op(v, dpp_u32<dpp::kMirror>(v));
  return swap_reduce_u32(v, op);
}

// ---------------------------------------------------------------- Philox4x64-10
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11): Philox-4x64 round function, 10 rounds, Weyl key schedule.
struct U64x4 {
  uint64_t w[4];
};

__device__ __forceinline__ U64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                                               uint64_t k1) {
  constexpr uint64_t kMul0 = 0xD2E7470EE14C6C93ull;
  constexpr uint64_t kMul1 = 0xCA5A826395121157ull;
  constexpr uint64_t kWeyl0 = 0x9E3779B97F4A7C15ull;
  constexpr uint64_t kWeyl1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kWeyl0;
      k1 += kWeyl1;
    }
    const uint64_t lo0 = kMul0 * c0, hi0 = __umul64hi(kMul0, c0);
    const uint64_t lo1 = kMul1 * c2, hi1 = __umul64hi(kMul1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  U64x4 o;
  o.w[0] = c0;
  o.w[1] = c1;
  o.w[2] = c2;
  o.w[3] = c3;
  return o;
}

// ---------------------------------------------------------------- wide unsigned integers
typedef unsigned __int128 u128;

struct U192 {
  uint64_t lo, mid, hi;
};

__device__ __forceinline__ U192 mul_u128_u64(u128 a, uint64_t b) {
  const uint64_t a0 = uint64_t(a), a1 = uint64_t(a >> 64);
  const u128 p0 = u128(a0) * b;
  const u128 p1 = u128(a1) * b + (p0 >> 64);
  U192 r;
  r.lo = uint64_t(p0);
  r.mid = uint64_t(p1);
  r.hi = uint64_t(p1 >> 64);
  return r;
}

__device__ __forceinline__ U192 shl_u192(U192 a, int s) {  // 0 < s < 64
  U192 r;
  r.hi = (a.hi << s) | (a.mid >> (64 - s));
  r.mid = (a.mid << s) | (a.lo >> (64 - s));
  r.lo = a.lo << s;
  return r;
}

__device__ __forceinline__ bool le_u192(U192 a, U192 b) {
  if (a.hi != b.hi) return a.hi < b.hi;
  if (a.mid != b.mid) return a.mid < b.mid;
  return a.lo <= b.lo;
}

// floor(a / b) for b != 0 with a quotient known to fit in 64 bits (restoring division).
// floor(a / b) for a quotient below 2^52: an fp64 estimate (relative error ~2^-52, so off by at most
// a few units), corrected to the exact quotient with 128-bit products
__device__ __forceinline__ uint64_t div_u128_u64(u128 a, uint64_t b) {
  const double ad = double(uint64_t(a >> 64)) * 18446744073709551616.0 + double(uint64_t(a));
  uint64_t q = uint64_t(ad / double(b));
  while (u128(q) * b > a) --q;
  while (u128(q + 1) * b <= a) ++q;
  return q;
}

}  // namespace spectree

namespace spectree {

// ---------------------------------------------------------------- cross-block hand-off
// Data one block publishes for another block of the same launch (split-K
// partials, per-slice candidates) is written and read with relaxed atomics at
// agent scope: on CDNA3/CDNA4 these carry the device-scope cache policy, so
// stores write through the XCD's L2 and loads do not hit a stale L2 line of
// another XCD. The writer waits for its stores to complete (vmcnt) before it
// takes a ticket; the block that draws the last ticket reads after it.
// This avoids agent-scope fences, whose L2 writeback serialises the blocks.
// The ordering is the hardware's, not the C++/HIP model's (which leaves
// relaxed accesses unordered): in gfx950 code (the LLVM AMDGPU memory model
// for GFX942/GFX950) a relaxed agent-scope store or load is a global store or
// load with the sc1 bit, served at the device coherence point, and
// s_waitcnt vmcnt(0) returns once the wave's stores are complete there; the
// reader's loads issue only after its ticket's value has returned.
// tests/test_handoff_codegen.py checks the built code for these forms.
template <typename T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until this thread's global stores are complete, and keep the compiler from moving memory ops across
__device__ __forceinline__ void wait_global_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ uint32_t ticket_add(uint32_t* t) {
  return __hip_atomic_fetch_add(t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ticket_add_n(uint32_t* t, uint32_t n) {
  return __hip_atomic_fetch_add(t, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ticket_reset(uint32_t* t) {
  __hip_atomic_store(t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace spectree
