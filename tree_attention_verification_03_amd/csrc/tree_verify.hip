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
// the node's uniforms, so all nodes are evaluated in parallel, in one launch of
// 1024-thread blocks, grid (n_slices + 1, B * max_T):
//   x < n_slices   greedy rows: the block reduces a slice of the row to a packed
//                  64-bit key (order(value) << 32 | ~index) and merges it with
//                  a 64-bit atomicMax - order-free, bit-exact;
//   x = n_slices   sampling rows: the block runs the node's exact integer state
//                  machine (2^-32 fixed point; sums are integers, so reduction
//                  order cannot change them).
// Blocks of the other mode exit at once. Every block then takes a ticket of its
// sequence; the last one walks the tree: longest valid path (greedy) or the
// chain of ACCEPT links (sampling), emits the path, tokens, bonus and status,
// and re-zeroes the workspace.
#include "api_common.h"
#include "spec_common.h"

namespace spectree {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

struct VerifyWs {
  uint64_t* keys;      // [B*max_T] greedy argmax keys (0 = empty)
  uint32_t* rowflag;   // [B*max_T] NaN seen in the greedy row
  int32_t* acc_child;  // [B*max_T] sampling: accepted child node or -1
  int32_t* bonus;      // [B*max_T] sampling: bonus token when the walk stops here
  uint32_t* nflag;     // [B*max_T] sampling node flags
  uint32_t* tickets;   // [B] blocks of the sequence that have finished
};

VerifyWs carve(void* ws, int B, int max_T, size_t* total) {
  const size_t n = size_t(B) * max_T;
  char* c = static_cast<char*>(ws);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = c ? c + off : nullptr;
    off = align_up(off + bytes, 256);
    return r;
  };
  VerifyWs w;
  w.keys = reinterpret_cast<uint64_t*>(take(8 * n));
  w.rowflag = reinterpret_cast<uint32_t*>(take(4 * n));
  w.acc_child = reinterpret_cast<int32_t*>(take(4 * n));
  w.bonus = reinterpret_cast<int32_t*>(take(4 * n));
  w.nflag = reinterpret_cast<uint32_t*>(take(4 * n));
  w.tickets = reinterpret_cast<uint32_t*>(take(4 * size_t(B)));
  *total = off;
  return w;
}

struct VerifyArgs {
  const float* target;
  const float* draft;
  const int32_t* q_row;
  const int32_t* tokens;
  const int32_t* parents;
  const int32_t* T_b;
  const int8_t* mode;
  uint64_t key0, key1, offset;
  int max_T, R, V, n_slices, slice, seg;
  int32_t* accept_len;
  int32_t* accept_nodes;
  int32_t* out_tokens;
  uint32_t* status;
};

__device__ __forceinline__ int seq_T(const int32_t* T_b, int b, int max_T) {
  int T = T_b ? T_b[b] : max_T;
  return T < 1 ? 1 : (T > max_T ? max_T : T);
}

__device__ __forceinline__ uint64_t argmax_key(float x, int v) {
  if (x != x) x = -INFINITY;  // NaN counts as -inf
  if (x == 0.f) x = 0.f;      // -0 == +0
  return (uint64_t(f32_order_key(x)) << 32) | uint64_t(0xffffffffu - uint32_t(v));
}

// ------------------------------------------------------------------ greedy
template <bool VEC>
__device__ void greedy_slice(const VerifyWs& w, const VerifyArgs& a, int row, int lo) {
  __shared__ uint64_t red[kWaves];
  __shared__ uint32_t nanred[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = min(a.V, lo + a.slice);
  const float* r = a.target + size_t(row) * a.V;
  uint64_t best = 0;
  bool nan = false;
  if (VEC) {
#pragma unroll 2
    for (int v = lo + 4 * tid; v < hi; v += 4 * kThreads) {
      const float4 x = *reinterpret_cast<const float4*>(r + v);
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
    atomicMax(reinterpret_cast<unsigned long long*>(w.keys + row), (unsigned long long)m);
    if (f) atomicOr(w.rowflag + row, 1u);
  }
}

// ------------------------------------------------------------------ sampling
__device__ __forceinline__ uint32_t fx(float x) {
  // 2^-32 fixed point: 0 for NaN / x <= 0, 2^32-1 for x >= 1, floor(x * 2^32) otherwise
  if (!(x > 0.f)) return 0u;
  if (x >= 1.f) return 0xffffffffu;
  return uint32_t(x * 4294967296.0f);  // exact power-of-two scaling, truncation = floor
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
__device__ u128 block_exclusive_scan_u128(u128 x, u128* wtot) {
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

template <bool VEC>
__device__ void sample_node(const VerifyWs& w, const VerifyArgs& a, int b, int u, int T) {
  __shared__ int kid_s[64];
  __shared__ int nkid_s;
  __shared__ uint64_t sp_s[kWaves], sq_s[kWaves], am_s[kWaves];
  __shared__ uint32_t nan_s[kWaves];
  __shared__ u128 segsum_s[kWaves];
  __shared__ u128 wtot_s[kWaves];
  __shared__ u128 W_s;
  __shared__ uint64_t gamma_s;
  __shared__ int decide_s;  // -1 keep testing, >= 0 accepted child
  __shared__ int wstar_s;
  __shared__ u128 excl_s;
  __shared__ int bonus_s;

  const int max_T = a.max_T, V = a.V;
  const int node = b * max_T + u;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // children of u in index order (a parent outside [0, c) counts as the root)
  if (wave == 0) {
    int n = 0;
    for (int c0 = 1; c0 < T; c0 += kWave) {
      const int c = c0 + lane;
      bool kid = false;
      if (c < T) {
        int pc = a.parents[size_t(b) * max_T + c];
        if (pc < 0 || pc >= c) pc = 0;
        kid = (pc == u);
      }
      const uint64_t m = __ballot(kid);
      if (kid) kid_s[n + __popcll(m & ((1ull << lane) - 1))] = c;
      n += __popcll(m);
    }
    if (lane == 0) nkid_s = n;
  }
  __syncthreads();
  const int nkid = nkid_s;
  const int qr = a.q_row ? a.q_row[size_t(b) * max_T + u] : -1;
  const bool has_q = nkid > 0 && a.draft != nullptr && qr >= 0 && qr < a.R;
  const float* prow = a.target + size_t(node) * V;
  const float* qrow = has_q ? a.draft + (size_t(b) * a.R + qr) * V : nullptr;
  const int lo = wave * a.seg, hi = min(V, lo + a.seg);

  // pass 0: S_P, S_Q, argmax of P, NaN checks, per-wave sums of P
  uint64_t sp = 0, sq = 0, am = 0;
  bool nan = false;
  seg_for<VEC>(prow, qrow, lo, hi, lane, [&](int v, float x, float y) {
    nan |= (x != x) | (y != y);
    const uint32_t P = fx(x);
    sp += P;
    const uint64_t k = (uint64_t(P) << 32) | uint64_t(0xffffffffu - uint32_t(v));
    am = k > am ? k : am;
    sq += fx(y);
  });
  sp = wave_sum_u64(sp);
  sq = wave_sum_u64(sq);
  am = wave_max_u64(am);
  const uint32_t nw = wave_or_u32(nan ? 1u : 0u);
  if (lane == 0) {
    sp_s[wave] = sp;
    sq_s[wave] = sq;
    am_s[wave] = am;
    nan_s[wave] = nw;
  }
  __syncthreads();
  uint64_t S_P = 0, S_Q = 0, AM = 0;
  uint32_t flags = 0;
  for (int i = 0; i < kWaves; ++i) {
    S_P += sp_s[i];
    S_Q += sq_s[i];
    AM = am_s[i] > AM ? am_s[i] : AM;
    if (nan_s[i]) flags |= SPEC_STATUS_NAN_INPUT;
  }
  const bool test = nkid > 0 && has_q && S_Q > 0;
  if (nkid > 0 && !test) flags |= SPEC_STATUS_ZERO_Q;
  if (tid == 0) {
    W_s = u128(S_P) * S_Q;
    gamma_s = 0;
    decide_s = -1;
  }
  __syncthreads();

  bool tested = false;
  for (int ki = 0; test && ki < nkid; ++ki) {
    const int c = kid_s[ki];
    const int t = a.tokens[size_t(b) * max_T + c];
    if (t < 0 || t >= V) continue;  // invalid draft token: never tested
    tested = true;
    if (tid == 0) {
      const uint32_t Pt = fx(prow[t]), Qt = fx(qrow[t]);
      const u128 Nt = residual(Pt, Qt, S_Q, gamma_s, false);
      const U64x4 r = philox4x64_10(a.offset, uint64_t(b), uint64_t(c), 0, a.key0, a.key1);
      const uint64_t m = (r.w[0] >> 40) + 1;  // r = m / 2^24 in (0, 1]
      bool accept = false;
      if (Nt > 0) {
        const U192 lhs = mul_u128_u64(W_s, m * uint64_t(Qt));  // m Q_t W
        const U192 rhs = shl_u192(mul_u128_u64(Nt, S_Q), 24);   // 2^24 N_t S_Q
        accept = le_u192(lhs, rhs);
      }
      if (accept) {
        decide_s = c;
      } else {
        gamma_s = gamma_s + div_u128_u64(W_s, S_Q);  // residual <- norm(max(0, residual - q))
      }
    }
    __syncthreads();
    if (decide_s >= 0) break;
    // the residual mass W and per-wave sums under the new gamma
    const uint64_t gamma = gamma_s;
    u128 acc = 0;
    seg_for<VEC>(prow, qrow, lo, hi, lane, [&](int, float x, float y) { acc += residual(fx(x), fx(y), S_Q, gamma, false); });
    acc = wave_sum_u128(acc);
    if (lane == 0) segsum_s[wave] = acc;
    __syncthreads();
    if (tid == 0) {
      u128 W = 0;
      for (int i = 0; i < kWaves; ++i) W += segsum_s[i];
      W_s = W;
    }
    __syncthreads();
    if (W_s == 0) flags |= SPEC_STATUS_ZERO_RESIDUAL;
  }

  if (decide_s >= 0) {
    if (tid == 0) {
      st_agent(w.acc_child + node, decide_s);
      st_agent(w.bonus + node, -1);
      st_agent(w.nflag + node, flags);
    }
    return;
  }
  // ---- no draft accepted: resample from the residual (or from P if nothing was tested)
  if (!tested) {
    if (lane == 0) segsum_s[wave] = u128(sp);
    if (tid == 0) W_s = S_P;
  }
  __syncthreads();
  const bool plain = !tested;
  const uint64_t gamma = gamma_s;
  const u128 W = W_s;
  if (W == 0) {
    if (tid == 0) bonus_s = int(0xffffffffu - uint32_t(AM));  // smallest-index argmax of P
  } else {
    // threshold: smallest v with 2^32 * prefix(v) > K W  <=>  prefix(v) > floor(K W / 2^32)
    if (tid == 0) {
      const U64x4 r = philox4x64_10(a.offset, uint64_t(b), uint64_t(u), 0, a.key0, a.key1);
      const uint64_t K = r.w[1] >> 32;
      const U192 kw = mul_u128_u64(W, K);
      const u128 tau = (u128(kw.hi) << 96) | (u128(kw.mid) << 32) | u128(kw.lo >> 32);
      u128 run = 0;
      int ws = kWaves - 1;
      for (int i = 0; i < kWaves; ++i) {
        if (run + segsum_s[i] > tau) {
          ws = i;
          break;
        }
        run += segsum_s[i];
      }
      wstar_s = ws;
      excl_s = tau - run;  // remaining threshold inside the chosen segment
      bonus_s = -1;
    }
    __syncthreads();
    // the whole block searches the chosen segment: each thread sums a contiguous range, a block scan
    // gives every range's prefix, and the one range holding the crossing is walked element by element
    const int wlo = wstar_s * a.seg, whi = min(V, wlo + a.seg);
    const int E = (whi - wlo + kThreads - 1) / kThreads;
    const int e0 = min(whi, wlo + tid * E), e1 = min(whi, e0 + E);
    auto resid = [&](int v) {
      return residual(fx(prow[v]), has_q ? fx(qrow[v]) : 0u, S_Q, gamma, plain);
    };
    u128 tsum = 0;
    for (int v = e0; v < e1; ++v) tsum += resid(v);
    const u128 ex = block_exclusive_scan_u128(tsum, wtot_s);
    const u128 rem = excl_s;
    if (tsum > 0 && ex <= rem && rem < ex + tsum) {
      u128 run = ex;
      for (int v = e0; v < e1; ++v) {
        run += resid(v);
        if (run > rem) {
          bonus_s = v;
          break;
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int bn = bonus_s;
    if (bn < 0) bn = int(0xffffffffu - uint32_t(AM));  // unreachable with exact sums; keeps the output defined
    st_agent(w.acc_child + node, -1);
    st_agent(w.bonus + node, bn);
    st_agent(w.nflag + node, flags);
  }
}

// ------------------------------------------------------------------ walk
// Runs in the last block of sequence b to finish; reads the other blocks' results with agent-scope loads.
__device__ void walk(const VerifyWs& w, const VerifyArgs& a, int b) {
  __shared__ int par_s[65], a_s[65], jmp_s[65], dep_s[65], ok_s[65], path_s[65];
  __shared__ uint32_t st_s, best_s;
  __shared__ int n_s, bonus_s;
  const int tid = threadIdx.x, max_T = a.max_T, V = a.V;
  const int T = seq_T(a.T_b, b, max_T);
  const bool greedy = a.mode[b] != SPEC_MODE_SAMPLE;
  const size_t base = size_t(b) * max_T;
  if (tid == 0) {
    st_s = 0;
    best_s = 0;
  }
  __syncthreads();
  if (tid < T) {
    uint32_t f = 0;
    int par = -1;
    if (tid > 0) {
      par = a.parents[base + tid];
      if (par < 0 || par >= tid) {
        par = 0;
        f |= SPEC_STATUS_INVALID_PARENT;
      }
      const int t = a.tokens[base + tid];
      if (t < 0 || t >= V) f |= SPEC_STATUS_INVALID_TOKEN;
    }
    par_s[tid] = par;
    if (greedy) {
      const uint64_t k = ld_agent(w.keys + base + tid);
      a_s[tid] = int(0xffffffffu - uint32_t(k));
      if (ld_agent(w.rowflag + base + tid)) f |= SPEC_STATUS_NAN_INPUT;
      st_agent(w.keys + base + tid, uint64_t(0));  // leave the workspace zeroed
      st_agent(w.rowflag + base + tid, 0u);
    } else {
      f |= ld_agent(w.nflag + base + tid) & SPEC_STATUS_NAN_INPUT;
    }
    if (f) atomicOr(&st_s, f);
  }
  __syncthreads();

  int e = 0;
  if (greedy) {
    if (tid < T) {
      const int t = tid > 0 ? a.tokens[base + tid] : 0;
      const bool good = tid == 0 || (t >= 0 && t < V && t == a_s[par_s[tid]]);
      ok_s[tid] = good;
      jmp_s[tid] = tid > 0 ? par_s[tid] : 0;
      dep_s[tid] = tid > 0;
    }
    __syncthreads();
    for (int it = 0; it < 7; ++it) {  // pointer doubling: validity = AND, depth = sum along the path
      int no = 0, nd = 0, nj = 0;
      if (tid < T) {
        const int j = jmp_s[tid];
        no = ok_s[tid] & ok_s[j];
        nd = dep_s[tid] + dep_s[j];
        nj = jmp_s[j];
      }
      __syncthreads();
      if (tid < T) {
        ok_s[tid] = no;
        dep_s[tid] = nd;
        jmp_s[tid] = nj;
      }
      __syncthreads();
    }
    // deepest valid node, ties -> smallest index
    if (tid < T && ok_s[tid]) atomicMax(&best_s, (uint32_t(dep_s[tid] + 1) << 8) | uint32_t(255 - tid));
    __syncthreads();
    e = 255 - int(best_s & 255u);
  } else {
    if (tid == 0) {
      int uu = 0, n = 0;
      uint32_t sf = 0;
      path_s[0] = 0;
      while (true) {
        sf |= ld_agent(w.nflag + base + uu) & (SPEC_STATUS_ZERO_Q | SPEC_STATUS_ZERO_RESIDUAL);
        const int c = ld_agent(w.acc_child + base + uu);
        if (c <= uu || c >= T || n >= 64) break;
        uu = c;
        path_s[++n] = uu;
      }
      st_s |= sf;
      dep_s[0] = n;  // reuse as the path length
      a_s[0] = ld_agent(w.bonus + base + uu);
    }
    __syncthreads();
  }
  if (tid == 0) {
    int n;
    int bonus;
    if (greedy) {
      n = dep_s[e];
      int x = e;
      for (int k = n; k >= 0; --k) {
        path_s[k] = x;
        x = par_s[x] < 0 ? 0 : par_s[x];
      }
      bonus = a_s[e];
    } else {
      n = dep_s[0];
      bonus = a_s[0];
    }
    a.accept_len[b] = n;
    a.status[b] = st_s;
    n_s = n;
    bonus_s = bonus;
  }
  __syncthreads();
  const int n = n_s;
  for (int k = tid; k < max_T; k += kThreads) {
    a.accept_nodes[base + k] = k <= n ? path_s[k] : -1;
    a.out_tokens[base + k] = k < n ? a.tokens[base + path_s[k + 1]] : (k == n ? bonus_s : -1);
  }
}

template <bool VEC>
__global__ void __launch_bounds__(kThreads) verify_kernel(VerifyWs w, VerifyArgs a) {
  __shared__ int last_s;
  const int unit = blockIdx.x, row = blockIdx.y;
  const int b = row / a.max_T, u = row - b * a.max_T;
  const int T = seq_T(a.T_b, b, a.max_T);
  const bool greedy = a.mode[b] != SPEC_MODE_SAMPLE;
  if (u < T) {
    if (greedy && unit < a.n_slices) greedy_slice<VEC>(w, a, row, unit * a.slice);
    if (!greedy && unit == a.n_slices) sample_node<VEC>(w, a, b, u, T);
  }
  // every block of the grid counts toward its sequence; the last one to arrive walks the tree
  wait_global_stores();
  __syncthreads();
  if (threadIdx.x == 0) last_s = ticket_add(w.tickets + b) == uint32_t((a.n_slices + 1) * a.max_T - 1);
  __syncthreads();
  if (!last_s) return;
  if (threadIdx.x == 0) ticket_reset(w.tickets + b);  // leave the workspace ready for the next call
  walk(w, a, b);
}

}  // namespace
}  // namespace spectree

using namespace spectree;

extern "C" size_t spec_tree_verify_workspace_size(int32_t B, int32_t max_T, int32_t V) {
  if (B < 1 || max_T < 1 || max_T > 65 || V < 1) return 0;
  size_t total = 0;
  carve(nullptr, B, max_T, &total);
  return total;
}

extern "C" int32_t spec_tree_verify(const float* target, const float* draft_probs, const int32_t* q_row,
                                    const int32_t* tokens, const int32_t* parents, const int32_t* T_b,
                                    const int8_t* mode, uint64_t philox_key0, uint64_t philox_key1,
                                    uint64_t philox_offset, int32_t B, int32_t max_T, int32_t R, int32_t V,
                                    int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens, uint32_t* status,
                                    void* ws, size_t ws_bytes, void* stream) {
  if (B < 1 || max_T < 1) return fail(SPEC_E_INVAL, "spec_tree_verify: B=%d max_T=%d", B, max_T);
  if (max_T > 65) return fail(SPEC_E_UNSUPPORTED, "spec_tree_verify: max_T=%d > 65", max_T);
  if (V < 1 || V >= (1 << 24)) return fail(SPEC_E_UNSUPPORTED, "spec_tree_verify: V=%d not in [1, 2^24)", V);
  if (draft_probs && (R < 1 || !q_row)) return fail(SPEC_E_INVAL, "spec_tree_verify: draft_probs needs R >= 1 and q_row");
  if (!target || !tokens || !parents || !mode || !accept_len || !accept_nodes || !out_tokens || !status)
    return fail(SPEC_E_INVAL, "spec_tree_verify: null pointer");
  if ((long long)B * max_T > 65535LL) return fail(SPEC_E_UNSUPPORTED, "spec_tree_verify: B*max_T=%lld > 65535",
                                                  (long long)B * max_T);
  size_t need = 0;
  VerifyWs w = carve(ws, B, max_T, &need);
  if (!ws || ws_bytes < need) return fail(SPEC_E_WORKSPACE, "spec_tree_verify: workspace %zu < %zu bytes", ws_bytes, need);
  const int rows = B * max_T;
  // greedy slices: whole multiples of one block pass (4 K elements), about 512 slice blocks per launch
  long long sl = ((long long)V * rows + 511) / 512;
  sl = (sl + 4095) / 4096 * 4096;
  if (sl > 65536) sl = 65536;
  VerifyArgs a;
  a.target = target;
  a.draft = draft_probs;
  a.q_row = q_row;
  a.tokens = tokens;
  a.parents = parents;
  a.T_b = T_b;
  a.mode = mode;
  a.key0 = philox_key0;
  a.key1 = philox_key1;
  a.offset = philox_offset;
  a.max_T = max_T;
  a.R = draft_probs ? R : 0;
  a.V = V;
  a.slice = int(sl);
  a.n_slices = int((V + sl - 1) / sl);
  a.seg = (V + kWaves - 1) / kWaves;
  a.seg = (a.seg + 3) / 4 * 4;  // segment bounds on 16-byte boundaries for the vector path
  a.accept_len = accept_len;
  a.accept_nodes = accept_nodes;
  a.out_tokens = out_tokens;
  a.status = status;
  const bool vec = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(target) | reinterpret_cast<uintptr_t>(draft_probs)) & 15) == 0;
  const dim3 grid(a.n_slices + 1, rows);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (vec)
    hipLaunchKernelGGL(verify_kernel<true>, grid, dim3(kThreads), 0, st, w, a);
  else
    hipLaunchKernelGGL(verify_kernel<false>, grid, dim3(kThreads), 0, st, w, a);
  return check_launch("spec_tree_verify");
}
