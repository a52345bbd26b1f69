"""Seeded synthetic inputs shaped like the pages' workloads.

Recipe (every draw comes from ``numpy.random.Generator(PCG64)`` streams spawned
from one ``SeedSequence(seed)``, one stream per purpose, so changing one input
does not shift the others):

* prefix lengths, topk, depth: fixed, or uniform integers in the stated range;
* KV pool: pages of ``page`` tokens, shape ``[num_pages, page, Hkv, d]``; the
  physical page order is a random permutation (or the identity for a
  "contiguous" workload); K and V ~ N(0, 1) in fp32, rounded to bf16 (RNE);
  the tree slots ``L_b .. L_b + T - 1`` (node i at slot ``L_b + i``) are drawn
  the same way, since the target's forward pass writes them there;
* Q ~ N(0, 1), rounded to bf16, shape ``[B, T_max, Hq, d]``;
* draft rows: fp32 logits ~ N(0, 2) (sigma = 2), one row per (sequence, step,
  frontier slot); log-probs (fp64 log-softmax, stored fp32) feed the tree
  builder and probabilities (fp64 softmax, stored fp32) feed verification;
  row 0 is the root row (step 1), row ``1 + (d - 2) * max_topk + f`` is step
  d's row for frontier slot f;
* target rows ``[B, T_max, V]``: fp32 logits ~ N(0, 3) for greedy sequences;
  for sampling sequences fp64 softmax(logits / temperature), stored fp32 (the
  logits themselves are kept as ``target_logits`` for every row);
* root tokens uniform in [0, V); Philox key = (seed, 0x5EED), offset 0;
* truncated draft vocabulary (``draft_vocab`` = V_d < V): a token map of V_d
  distinct token ids drawn without replacement from [0, V) in random order
  (a frequency ranking has no relation to token ids); the draft rows hold V_d
  entries (logits ~ N(0, 2) over the subset) and the draft probabilities are
  scattered to the full vocabulary (zero outside the subset).
* FP8 KV pools (``fp8_kv_pools``): per KV head a scale 2^U(-7, -5); values
  ~ N(0, 1) / scale in fp32, clipped to +-448 and converted to OCP E4M3 codes
  by torch's float8_e4m3fn cast (input data only: the attention consumes the
  codes as they are).

Nothing here builds trees, masks, attends or verifies.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from .configs import WorkloadSpec

MODE_GREEDY = 0
MODE_SAMPLE = 1


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 with round-to-nearest-even; returns uint16 bit patterns.

    Inputs here are finite normal draws, so no NaN handling is needed.
    """
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    lsb = u >> np.uint32(16)
    lsb &= np.uint32(1)
    u += np.uint32(0x7FFF)  # finite inputs: no uint32 overflow
    u += lsb
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def _bf16_normals(rng: np.random.Generator, shape, chunk: int = 1 << 22) -> np.ndarray:
    """N(0, 1) fp32 draws rounded to bf16 bits, drawn in order chunk by chunk."""
    out = np.empty(int(np.prod(shape)), dtype=np.uint16)
    for lo in range(0, out.size, chunk):
        hi = min(out.size, lo + chunk)
        out[lo:hi] = f32_to_bf16_bits(rng.standard_normal(hi - lo, dtype=np.float32))
    return out.reshape(shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _fp64_log_softmax(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float64)
    m = z.max(axis=-1, keepdims=True)
    s = np.log(np.exp(z - m).sum(axis=-1, keepdims=True))
    return z - m - s


@dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    page: int
    V: int
    max_topk: int
    max_depth: int
    max_T: int
    prefix_lens: np.ndarray  # int32 [B]
    topk: np.ndarray  # int32 [B]
    depth: np.ndarray  # int32 [B]
    num_draft: np.ndarray  # int32 [B]
    T_b: np.ndarray  # int32 [B]
    modes: np.ndarray  # int8 [B], 0 greedy / 1 sample
    temperature: np.ndarray  # float32 [B]
    page_table: np.ndarray  # int32 [B, max_pages]
    num_pages: int
    k_pages: np.ndarray  # uint16 (bf16 bits) [num_pages, page, Hkv, d]
    v_pages: np.ndarray  # uint16 (bf16 bits) [num_pages, page, Hkv, d]
    q: np.ndarray  # uint16 (bf16 bits) [B, max_T, Hq, d]
    root_tokens: np.ndarray  # int32 [B]
    draft_logprobs: np.ndarray  # float32 [B, R, V]
    draft_probs: np.ndarray  # float32 [B, R, V]
    target: np.ndarray  # float32 [B, max_T, V]
    philox_key: tuple
    philox_offset: int
    sm_scale: float
    compact: bool = False
    extra: dict = field(default_factory=dict)
    target_logits: np.ndarray = None  # float32 [B, max_T, V]: the logits every target row was formed from
    token_map: Optional[np.ndarray] = None  # int32 [V_d]: draft row entry i stands for token token_map[i]

    @property
    def R(self) -> int:
        return self.draft_probs.shape[1]

    @property
    def max_pages(self) -> int:
        return self.page_table.shape[1]

    def step_rows(self, step: int) -> np.ndarray:
        """Draft log-prob rows consumed by tree-build step ``step`` (1-based): [B, F, V]."""
        lo, hi = step_row_range(step, self.max_topk)
        return self.draft_logprobs[:, lo:hi, :]


def step_row_range(step: int, max_topk: int):
    """Rows of the draft-row array that hold step ``step``'s frontier rows."""
    if step == 1:
        return 0, 1
    lo = 1 + (step - 2) * max_topk
    return lo, lo + max_topk


def _draw_int(rng, spec, B):
    if isinstance(spec, int):
        return np.full(B, spec, dtype=np.int32)
    lo, hi = spec
    return rng.integers(lo, hi + 1, size=B).astype(np.int32)


def make_workload(
    *,
    name: str = "custom",
    B: int,
    Hq: int,
    Hkv: int,
    d: int,
    prefix,
    topk,
    depth,
    num_draft,
    V: int,
    verify: str = "greedy",
    temperature: float = 1.0,
    page: int = 16,
    contiguous_pages: bool = False,
    compact: bool = False,
    seed: int = 0,
    max_topk: Optional[int] = None,
    max_depth: Optional[int] = None,
    extra_pages: int = 0,
    draft_vocab: Optional[int] = None,
) -> Workload:
    """Draw one workload. ``prefix``/``topk``/``depth``/``num_draft`` are an int,
    an inclusive (lo, hi) tuple range, or an explicit per-sequence list."""
    ss = np.random.SeedSequence(seed)
    (s_len, s_kv, s_q, s_draft, s_target, s_root, s_pages) = ss.spawn(7)
    r_len = np.random.Generator(np.random.PCG64(s_len))

    def per_seq(spec):
        # a list / array gives explicit per-sequence values; a tuple is a range
        if isinstance(spec, (list, np.ndarray)):
            arr = np.asarray(spec, dtype=np.int32)
            if arr.shape != (B,):
                raise ValueError(f"per-sequence list must have length {B}")
            return arr
        return _draw_int(r_len, spec, B)

    prefix_lens = per_seq(prefix)
    topk_b = per_seq(topk)
    depth_b = per_seq(depth)
    nd_b = per_seq(num_draft)
    max_topk = int(max_topk if max_topk is not None else topk_b.max())
    max_depth = int(max_depth if max_depth is not None else depth_b.max())
    T_b = (nd_b + 1).astype(np.int32)
    max_T = int(T_b.max())

    if verify == "greedy":
        modes = np.zeros(B, dtype=np.int8)
    elif verify == "sample":
        modes = np.ones(B, dtype=np.int8)
    elif verify == "alternate":
        modes = (np.arange(B) % 2).astype(np.int8)
    else:
        raise ValueError(verify)
    temps = np.where(modes == MODE_SAMPLE, np.float32(temperature), np.float32(0.0)).astype(np.float32)

    # ---- paged KV pool -------------------------------------------------
    pages_per_seq = [int(-(-(int(L) + max_T) // page)) for L in prefix_lens]
    max_pages = max(pages_per_seq)
    num_pages = sum(pages_per_seq) + extra_pages
    r_pages = np.random.Generator(np.random.PCG64(s_pages))
    phys = np.arange(num_pages, dtype=np.int32) if contiguous_pages else r_pages.permutation(num_pages).astype(np.int32)
    page_table = np.full((B, max_pages), -1, dtype=np.int32)
    cursor = 0
    for b in range(B):
        n = pages_per_seq[b]
        page_table[b, :n] = phys[cursor:cursor + n]
        cursor += n
    r_kv = np.random.Generator(np.random.PCG64(s_kv))
    kv_shape = (num_pages, page, Hkv, d)
    k_pages = _bf16_normals(r_kv, kv_shape)
    v_pages = _bf16_normals(r_kv, kv_shape)

    r_q = np.random.Generator(np.random.PCG64(s_q))
    q = _bf16_normals(r_q, (B, max_T, Hq, d))

    # ---- draft rows ----------------------------------------------------
    R = 1 + (max_depth - 1) * max_topk
    r_draft = np.random.Generator(np.random.PCG64(s_draft))
    token_map = None
    Vd = V
    if draft_vocab is not None and int(draft_vocab) != V:
        Vd = int(draft_vocab)
        if not (max_topk <= Vd < V):
            raise ValueError("draft_vocab must be in [max_topk, V)")
        r_map = np.random.Generator(np.random.PCG64(ss.spawn(1)[0]))
        token_map = r_map.choice(V, size=Vd, replace=False).astype(np.int32)
    draft_logprobs = np.empty((B, R, Vd), dtype=np.float32)
    draft_probs = np.zeros((B, R, V), dtype=np.float32)
    for b in range(B):
        z = r_draft.standard_normal((R, Vd), dtype=np.float32) * np.float32(2.0)
        lp = _fp64_log_softmax(z)
        draft_logprobs[b] = lp.astype(np.float32)
        if token_map is None:
            draft_probs[b] = np.exp(lp).astype(np.float32)
        else:
            draft_probs[b][:, token_map] = np.exp(lp).astype(np.float32)

    # ---- target rows ---------------------------------------------------
    r_t = np.random.Generator(np.random.PCG64(s_target))
    target = np.empty((B, max_T, V), dtype=np.float32)
    target_logits = np.empty((B, max_T, V), dtype=np.float32)
    for b in range(B):
        z = r_t.standard_normal((max_T, V), dtype=np.float32) * np.float32(3.0)
        target_logits[b] = z
        if modes[b] == MODE_SAMPLE:
            target[b] = np.exp(_fp64_log_softmax(z.astype(np.float64) / float(temperature))).astype(np.float32)
        else:
            target[b] = z

    r_root = np.random.Generator(np.random.PCG64(s_root))
    root_tokens = r_root.integers(0, V, size=B).astype(np.int32)

    return Workload(
        name=name, B=B, Hq=Hq, Hkv=Hkv, d=d, page=page, V=V,
        max_topk=max_topk, max_depth=max_depth, max_T=max_T,
        prefix_lens=prefix_lens, topk=topk_b, depth=depth_b, num_draft=nd_b, T_b=T_b,
        modes=modes, temperature=temps, page_table=page_table, num_pages=num_pages,
        k_pages=k_pages, v_pages=v_pages, q=q, root_tokens=root_tokens,
        draft_logprobs=draft_logprobs, draft_probs=draft_probs, target=target, target_logits=target_logits,
        philox_key=(int(seed) & 0xFFFFFFFFFFFFFFFF, 0x5EED), philox_offset=0,
        sm_scale=float(1.0 / np.sqrt(d)), compact=compact, token_map=token_map,
    )


def from_spec(spec: WorkloadSpec, seed: Optional[int] = None, draft_vocab: Optional[int] = None) -> Workload:
    """Draw the named workload at full size (optionally with a truncated draft vocabulary)."""
    return make_workload(
        draft_vocab=draft_vocab,
        name=spec.name, B=spec.batch, Hq=spec.q_heads, Hkv=spec.kv_heads, d=spec.head_dim,
        prefix=spec.prefix, topk=spec.topk, depth=spec.depth, num_draft=spec.num_draft,
        V=spec.vocab, verify=spec.verify, temperature=spec.temperature if spec.verify != "greedy" else 1.0,
        page=spec.page, contiguous_pages=spec.contiguous_pages, compact=spec.compact,
        seed=spec.seed if seed is None else seed,
        max_topk=spec.max_topk, max_depth=spec.max_depth,
    )


def random_parents(rng: np.random.Generator, T: int, kind: str = "random") -> np.ndarray:
    """Parent-pointer arrays for attention-only cases (inputs, not a built tree).

    ``random``: parents[i] uniform in [0, i); ``chain``: parents[i] = i - 1;
    ``star``: every draft hangs off the root.
    """
    p = np.full(T, -1, dtype=np.int32)
    for i in range(1, T):
        if kind == "chain":
            p[i] = i - 1
        elif kind == "star":
            p[i] = 0
        else:
            p[i] = rng.integers(0, i)
    return p


def fp8_kv_pools(shape, seed: int, chunk: int = 1 << 22):
    """E4M3 code pools of ``shape`` = [P, page, Hkv, d] for K and V, and fp32 per-KV-head scales.

    Returns (k8, v8, k_scale, v_scale): uint8 arrays and float32 [Hkv] arrays.
    """
    import torch

    rng = np.random.default_rng([seed, 0xF8])
    Hkv = shape[2]
    scales = [(2.0 ** rng.uniform(-7, -5, size=Hkv)).astype(np.float32) for _ in range(2)]
    pools = []
    for sc in scales:
        inv = (1.0 / sc.astype(np.float64)).astype(np.float32)
        out = np.empty(shape, dtype=np.uint8)
        flat = out.reshape(-1, Hkv, shape[3])
        for lo in range(0, flat.shape[0], max(1, chunk // (Hkv * shape[3]))):
            hi = min(flat.shape[0], lo + max(1, chunk // (Hkv * shape[3])))
            x = rng.standard_normal((hi - lo, Hkv, shape[3]), dtype=np.float32) * inv[None, :, None]
            np.clip(x, -448.0, 448.0, out=x)
            flat[lo:hi] = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        pools.append(out)
    return pools[0], pools[1], scales[0], scales[1]
