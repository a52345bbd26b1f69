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
// the node's uniforms, so all nodes are evaluated in parallel:
//   verify_greedy_scan   greedy rows: (row, slice) blocks reduce a packed
//                        64-bit key (order(value) << 32 | ~index) and merge it
//                        with a 64-bit atomicMax - order-free, bit-exact.
//   verify_sample_node   sampling rows: one block per node runs the exact
//                        integer state machine (2^-32 fixed point; sums are
//                        integers, so reduction order cannot change them).
//   verify_walk          one block per sequence: longest valid path (greedy) or
//                        the chain of ACCEPT links (sampling), emits the path,
//                        tokens, bonus and status, and re-zeroes the workspace.
#include "api_common.h"
#include "spec_common.h"

namespace spectree {
namespace {

constexpr int kScanThreads = 256;
constexpr int kNodeThreads = 1024;
constexpr int kNodeWaves = kNodeThreads / kWave;
constexpr int kWalkThreads = 128;

struct VerifyWs {
  uint64_t* keys;      // [B*max_T] greedy argmax keys (0 = empty)
  uint32_t* rowflag;   // [B*max_T] NaN seen in the greedy row
  int32_t* acc_child;  // [B*max_T] sampling: accepted child node or -1
  int32_t* bonus;      // [B*max_T] sampling: bonus token when the walk stops here
  uint32_t* nflag;     // [B*max_T] sampling node flags
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
  *total = off;
  return w;
}

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
__global__ void __launch_bounds__(kScanThreads) verify_greedy_scan(VerifyWs w, const float* target, const int32_t* T_b,
                                                                    const int8_t* mode, int max_T, int V, int slice) {
  __shared__ uint64_t red[kScanThreads / kWave];
  __shared__ uint32_t nanred[kScanThreads / kWave];
  const int row = blockIdx.y;
  const int b = row / max_T, u = row - b * max_T;
  if (mode[b] == SPEC_MODE_SAMPLE || u >= seq_T(T_b, b, max_T)) return;
  const int lo = blockIdx.x * slice;
  const int hi = min(V, lo + slice);
  const float* r = target + size_t(row) * V;
  uint64_t best = 0;
  bool nan = false;
  if (VEC) {
    for (int v = lo + 4 * threadIdx.x; v < hi; v += 4 * kScanThreads) {
      const float4 x = *reinterpret_cast<const float4*>(r + v);
      nan |= (x.x != x.x) | (x.y != x.y) | (x.z != x.z) | (x.w != x.w);
      uint64_t k0 = argmax_key(x.x, v), k1 = argmax_key(x.y, v + 1), k2 = argmax_key(x.z, v + 2), k3 = argmax_key(x.w, v + 3);
      k0 = k0 > k1 ? k0 : k1;
      k2 = k2 > k3 ? k2 : k3;
      k0 = k0 > k2 ? k0 : k2;
      best = k0 > best ? k0 : best;
    }
  } else {
    for (int v = lo + threadIdx.x; v < hi; v += kScanThreads) {
      const float x = r[v];
      nan |= (x != x);
      const uint64_t k = argmax_key(x, v);
      best = k > best ? k : best;
    }
  }
  best = wave_max_u64(best);
  const uint32_t nw = wave_or_u32(nan ? 1u : 0u);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[wave] = best;
    nanred[wave] = nw;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t m = red[0];
    uint32_t f = nanred[0];
    for (int i = 1; i < kScanThreads / kWave; ++i) {
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

__device__ __forceinline__ u128 wave_sum_u128(u128 x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += shfl_xor_u128(x, o);
  return x;
}

__global__ void __launch_bounds__(kNodeThreads) verify_sample_node(VerifyWs w, const float* target, const float* draft,
                                                                    const int32_t* q_row, const int32_t* tokens,
                                                                    const int32_t* parents, const int32_t* T_b,
                                                                    const int8_t* mode, uint64_t key0, uint64_t key1,
                                                                    uint64_t offset, int max_T, int R, int V, int seg) {
  __shared__ int kid_s[64];
  __shared__ int nkid_s;
  __shared__ uint64_t sp_s[kNodeWaves], sq_s[kNodeWaves], am_s[kNodeWaves];
  __shared__ uint32_t nanp_s[kNodeWaves], nanq_s[kNodeWaves];
  __shared__ u128 segsum_s[kNodeWaves];
  __shared__ u128 W_s;
  __shared__ uint64_t gamma_s;
  __shared__ int decide_s;  // -1 keep testing, -2 stop (resample), >= 0 accepted child
  __shared__ int wstar_s;
  __shared__ u128 excl_s;
  __shared__ int bonus_s;

  const int node = blockIdx.x;
  const int b = node / max_T, u = node - b * max_T;
  const int T = seq_T(T_b, b, max_T);
  if (mode[b] != SPEC_MODE_SAMPLE || u >= T) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // children of u in index order (a parent outside [0, c) counts as the root)
  if (wave == 0) {
    int n = 0;
    for (int c0 = 1; c0 < T; c0 += kWave) {
      const int c = c0 + lane;
      bool kid = false;
      if (c < T) {
        int pc = parents[size_t(b) * max_T + c];
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
  const int qr = q_row ? q_row[size_t(b) * max_T + u] : -1;
  const bool has_q = nkid > 0 && draft != nullptr && qr >= 0 && qr < R;
  const float* prow = target + size_t(node) * V;
  const float* qrow = has_q ? draft + (size_t(b) * R + qr) * V : nullptr;
  const int lo = wave * seg, hi = min(V, lo + seg);

  // pass 0: S_P, S_Q, argmax of P, NaN checks, per-wave sums of P
  uint64_t sp = 0, sq = 0, am = 0;
  bool nanp = false, nanq = false;
  for (int v = lo + lane; v < hi; v += kWave) {
    const float x = prow[v];
    nanp |= (x != x);
    const uint32_t P = fx(x);
    sp += P;
    const uint64_t k = (uint64_t(P) << 32) | uint64_t(0xffffffffu - uint32_t(v));
    am = k > am ? k : am;
    if (has_q) {
      const float y = qrow[v];
      nanq |= (y != y);
      sq += fx(y);
    }
  }
  sp = wave_sum_u64(sp);
  sq = wave_sum_u64(sq);
  am = wave_max_u64(am);
  const uint32_t np = wave_or_u32(nanp), nq = wave_or_u32(nanq);
  if (lane == 0) {
    sp_s[wave] = sp;
    sq_s[wave] = sq;
    am_s[wave] = am;
    nanp_s[wave] = np;
    nanq_s[wave] = nq;
  }
  __syncthreads();
  uint64_t S_P = 0, S_Q = 0, AM = 0;
  uint32_t flags = 0;
  for (int i = 0; i < kNodeWaves; ++i) {
    S_P += sp_s[i];
    S_Q += sq_s[i];
    AM = am_s[i] > AM ? am_s[i] : AM;
    if (nanp_s[i] || nanq_s[i]) flags |= SPEC_STATUS_NAN_INPUT;
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
    const int t = tokens[size_t(b) * max_T + c];
    if (t < 0 || t >= V) continue;  // invalid draft token: never tested
    tested = true;
    if (tid == 0) {
      const uint32_t Pt = fx(prow[t]), Qt = fx(qrow[t]);
      const u128 Nt = residual(Pt, Qt, S_Q, gamma_s, false);
      const U64x4 r = philox4x64_10(offset, uint64_t(b), uint64_t(c), 0, key0, key1);
      const uint64_t m = (r.w[0] >> 40) + 1;  // r = m / 2^24 in (0, 1]
      bool accept = false;
      if (Nt > 0) {
        const U192 lhs = mul_u128_u64(W_s, m * uint64_t(Qt));          // m Q_t W
        const U192 rhs = shl_u192(mul_u128_u64(Nt, S_Q), 24);           // 2^24 N_t S_Q
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
    // recompute the residual mass W and per-wave sums under the new gamma
    const uint64_t gamma = gamma_s;
    u128 acc = 0;
    for (int v = lo + lane; v < hi; v += kWave) acc += residual(fx(prow[v]), fx(qrow[v]), S_Q, gamma, false);
    acc = wave_sum_u128(acc);
    if (lane == 0) segsum_s[wave] = acc;
    __syncthreads();
    if (tid == 0) {
      u128 W = 0;
      for (int i = 0; i < kNodeWaves; ++i) W += segsum_s[i];
      W_s = W;
    }
    __syncthreads();
    if (W_s == 0) flags |= SPEC_STATUS_ZERO_RESIDUAL;
  }

  if (decide_s >= 0) {
    if (tid == 0) {
      w.acc_child[node] = decide_s;
      w.bonus[node] = -1;
      w.nflag[node] = flags;
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
      const U64x4 r = philox4x64_10(offset, uint64_t(b), uint64_t(u), 0, key0, key1);
      const uint64_t K = r.w[1] >> 32;
      const U192 kw = mul_u128_u64(W, K);
      const u128 tau = (u128(kw.hi) << 96) | (u128(kw.mid) << 32) | u128(kw.lo >> 32);
      u128 run = 0;
      int ws = kNodeWaves - 1;
      for (int i = 0; i < kNodeWaves; ++i) {
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
    if (wave == wstar_s) {
      const u128 rem = excl_s;  // find first v in this segment with prefix_in_segment(v) > rem
      u128 run = 0;
      const int wlo = wstar_s * seg, whi = min(V, wlo + seg);
      for (int c0 = wlo; c0 < whi; c0 += kWave) {
        const int v = c0 + lane;
        const u128 n = v < whi ? residual(fx(prow[v]), has_q ? fx(qrow[v]) : 0u, S_Q, gamma, plain) : u128(0);
        // inclusive wave scan
        u128 incl = n;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const u128 t = shfl_up_u128(incl, o);
          if (lane >= o) incl += t;
        }
        const bool hit = run + incl > rem;
        const uint64_t hm = __ballot(hit);
        if (hm) {
          if (lane == __ffsll((long long)hm) - 1) bonus_s = v;
          break;
        }
        const uint64_t tot_lo = __shfl(uint64_t(incl), kWave - 1, kWave);
        const uint64_t tot_hi = __shfl(uint64_t(incl >> 64), kWave - 1, kWave);
        run += (u128(tot_hi) << 64) | tot_lo;  // this chunk's total (lane 63's inclusive sum)
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int bn = bonus_s;
    if (bn < 0) bn = int(0xffffffffu - uint32_t(AM));  // unreachable with exact sums; keeps the output defined
    w.acc_child[node] = -1;
    w.bonus[node] = bn;
    w.nflag[node] = flags;
  }
}

// ------------------------------------------------------------------ walk
__global__ void __launch_bounds__(kWalkThreads) verify_walk(VerifyWs w, const int32_t* tokens, const int32_t* parents,
                                                             const int32_t* T_b, const int8_t* mode, int max_T, int V,
                                                             int32_t* accept_len, int32_t* accept_nodes,
                                                             int32_t* out_tokens, uint32_t* status) {
  __shared__ int par_s[65], a_s[65], jmp_s[65], dep_s[65], ok_s[65];
  __shared__ uint32_t flag_red[kWalkThreads / kWave];
  __shared__ uint32_t best_red[kWalkThreads / kWave];
  __shared__ int path_s[65];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = seq_T(T_b, b, max_T);
  const bool greedy = mode[b] != SPEC_MODE_SAMPLE;
  const size_t base = size_t(b) * max_T;
  uint32_t f = 0;
  if (tid < T) {
    int par = -1;
    if (tid > 0) {
      par = parents[base + tid];
      if (par < 0 || par >= tid) {
        par = 0;
        f |= SPEC_STATUS_INVALID_PARENT;
      }
      const int t = tokens[base + tid];
      if (t < 0 || t >= V) f |= SPEC_STATUS_INVALID_TOKEN;
    }
    par_s[tid] = par;
    if (greedy) {
      const uint64_t k = w.keys[base + tid];
      a_s[tid] = int(0xffffffffu - uint32_t(k));
      if (w.rowflag[base + tid]) f |= SPEC_STATUS_NAN_INPUT;
      w.keys[base + tid] = 0;  // leave the workspace zeroed
      w.rowflag[base + tid] = 0;
    } else {
      f |= w.nflag[base + tid] & SPEC_STATUS_NAN_INPUT;
    }
  }
  f = wave_or_u32(f);
  if (lane == 0) flag_red[wave] = f;
  __syncthreads();
  uint32_t st = flag_red[0] | flag_red[1];

  int e = 0;
  if (greedy) {
    if (tid < T) {
      const int t = tid > 0 ? tokens[base + tid] : 0;
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
    uint32_t key = 0;
    if (tid < T && ok_s[tid]) key = (uint32_t(dep_s[tid] + 1) << 8) | uint32_t(255 - tid);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint32_t x = __shfl_xor(key, o, kWave);
      key = x > key ? x : key;
    }
    if (lane == 0) best_red[wave] = key;
    __syncthreads();
    const uint32_t kb = best_red[0] > best_red[1] ? best_red[0] : best_red[1];
    e = 255 - int(kb & 255u);
  } else {
    if (tid == 0) {
      int uu = 0, n = 0;
      path_s[0] = 0;
      while (true) {
        st |= w.nflag[base + uu] & (SPEC_STATUS_ZERO_Q | SPEC_STATUS_ZERO_RESIDUAL);
        const int c = w.acc_child[base + uu];
        if (c <= uu || c >= T || n >= 64) break;
        uu = c;
        path_s[++n] = uu;
      }
      dep_s[0] = n;  // reuse as the path length
      a_s[0] = w.bonus[base + uu];
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
    accept_len[b] = n;
    status[b] = st;
    for (int k = 0; k < max_T; ++k) {
      accept_nodes[base + k] = k <= n ? path_s[k] : -1;
      out_tokens[base + k] = k < n ? tokens[base + path_s[k + 1]] : (k == n ? bonus : -1);
    }
  }
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
  if ((long long)B * max_T > 65535LL * 64) return fail(SPEC_E_UNSUPPORTED, "spec_tree_verify: B*max_T too large");
  size_t need = 0;
  VerifyWs w = carve(ws, B, max_T, &need);
  if (!ws || ws_bytes < need) return fail(SPEC_E_WORKSPACE, "spec_tree_verify: workspace %zu < %zu bytes", ws_bytes, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int rows = B * max_T;
  // greedy scan: slices sized so that the launch has >= ~1k blocks
  long long sl = ((long long)V * rows + 1023) / 1024;
  sl = (sl + 1023) / 1024 * 1024;
  if (sl < 1024) sl = 1024;
  if (sl > 16384) sl = 16384;
  const int slice = int(sl);
  const dim3 sgrid((V + slice - 1) / slice, rows);
  const bool vec = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(target) & 15) == 0);
  if (vec)
    hipLaunchKernelGGL(verify_greedy_scan<true>, sgrid, dim3(kScanThreads), 0, st, w, target, T_b, mode, max_T, V, slice);
  else
    hipLaunchKernelGGL(verify_greedy_scan<false>, sgrid, dim3(kScanThreads), 0, st, w, target, T_b, mode, max_T, V, slice);
  const int seg = (V + kNodeWaves - 1) / kNodeWaves;
  hipLaunchKernelGGL(verify_sample_node, dim3(rows), dim3(kNodeThreads), 0, st, w, target, draft_probs, q_row, tokens,
                     parents, T_b, mode, philox_key0, philox_key1, philox_offset, max_T, draft_probs ? R : 0, V, seg);
  hipLaunchKernelGGL(verify_walk, dim3(B), dim3(kWalkThreads), 0, st, w, tokens, parents, T_b, mode, max_T, V,
                     accept_len, accept_nodes, out_tokens, status);
  return check_launch("spec_tree_verify");
}
