"""One verification step on the GPU: tree build -> tree attention -> verify -> KV compaction.

``DeviceWorkload`` moves a host workload (numpy arrays) into device tensors
once; ``SpecTreeStep`` preallocates every output and zeroed workspace so a step
only enqueues library calls on the current stream (no allocation, no host
synchronisation), which also makes it capturable in a HIP graph.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import ops


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> device bf16 tensor (bit-exact)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def step_row_range(step: int, max_topk: int):
    if step == 1:
        return 0, 1
    lo = 1 + (step - 2) * max_topk
    return lo, lo + max_topk


class DeviceWorkload:
    """Device copies of a ``workloads.Workload``."""

    def __init__(self, w, device="cuda", logits: bool = False):
        """``logits``: also upload the target logits and temperatures (verification from logits)."""
        self.w = w
        dev = torch.device(device)
        self.device = dev
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
        self.prefix_lens = i32(w.prefix_lens)
        self.topk = i32(w.topk)
        self.depth = i32(w.depth)
        self.num_draft = i32(w.num_draft)
        self.T_b = i32(w.T_b)
        self.modes = torch.from_numpy(np.ascontiguousarray(w.modes, dtype=np.int8)).to(dev)
        self.page_table = i32(w.page_table)
        self.root_tokens = i32(w.root_tokens)
        self.k_pages = bf16_tensor(w.k_pages, dev)
        self.v_pages = bf16_tensor(w.v_pages, dev)
        self.q = bf16_tensor(w.q, dev)
        self.draft_logprobs = torch.from_numpy(w.draft_logprobs).to(dev)
        self.draft_probs = torch.from_numpy(w.draft_probs).to(dev)
        self.target = torch.from_numpy(w.target).to(dev)
        self.token_map = None if w.token_map is None else i32(w.token_map)  # truncated draft vocabulary
        if logits:
            self.target_logits = torch.from_numpy(w.target_logits).to(dev)
            self.temperature = torch.from_numpy(np.ascontiguousarray(w.temperature, dtype=np.float32)).to(dev)


@dataclass
class StepOutputs:
    frontier: torch.Tensor
    tokens: torch.Tensor
    parents: torch.Tensor
    depth: torch.Tensor
    anc: torch.Tensor
    q_row: torch.Tensor
    attn_out: torch.Tensor
    lse: torch.Tensor
    attn_status: torch.Tensor
    accept_len: torch.Tensor
    accept_nodes: torch.Tensor
    out_tokens: torch.Tensor
    status: torch.Tensor
    new_prefix_lens: torch.Tensor


class SpecTreeStep:
    def __init__(self, dw: DeviceWorkload, attn_status: bool = True, fused_finish: bool = True,
                 verify_from_logits: bool = False):
        """``verify_from_logits``: verify with spec_tree_verify_logits on the target logits and temperatures
        (the DeviceWorkload must have been made with ``logits=True``)."""
        w = dw.w
        self.dw = dw
        self.from_logits = verify_from_logits
        self.fused_finish = fused_finish
        dev = dw.device
        B, T = w.B, w.max_T
        z = lambda *s, dt=torch.int32: torch.zeros(*s, dtype=dt, device=dev)
        self.o = StepOutputs(
            frontier=z(B, w.max_topk), tokens=z(B, T), parents=z(B, T), depth=z(B, T), anc=z(B, T, dt=torch.int64),
            q_row=z(B, T), attn_out=torch.zeros(B, T, w.Hq, w.d, dtype=torch.bfloat16, device=dev),
            lse=torch.zeros(B, T, w.Hq, dtype=torch.float32, device=dev), attn_status=z(B), accept_len=z(B),
            accept_nodes=z(B, T), out_tokens=z(B, T), status=z(B), new_prefix_lens=z(B))
        self.ws_build = ops.zeroed_workspace(ops.spec_tree_build_workspace_size(B, w.max_topk, w.max_depth), dev)
        self.ws_attn = ops.zeroed_workspace(
            ops.spec_tree_attention_workspace_size(B, T, w.Hq, w.Hkv, w.d, w.page, w.max_pages), dev)
        self.ws_verify = ops.zeroed_workspace(
            (ops.spec_tree_verify_logits_workspace_size if verify_from_logits else ops.spec_tree_verify_workspace_size)(
                B, T, w.V), dev)
        self.sampling = bool((w.modes == ops.MODE_SAMPLE).any())
        # the attention status word is OR-ed into, so collecting it costs a fill per step
        self.attn_status = attn_status

    # -- the four stages --------------------------------------------------
    def build(self):
        """Every step; a sequence is reranked at its own last step (fused launches), or, with
        ``fused_finish=False``, by a separate finish launch after the last step."""
        w, dw, o = self.dw.w, self.dw, self.o
        for step in range(1, w.max_depth + 1):
            lo, hi = step_row_range(step, w.max_topk)
            rows = dw.draft_logprobs[:, lo:hi, :]
            if self.fused_finish and dw.token_map is not None:
                ops.spec_tree_build_step_finish_map(self.ws_build, step, rows, dw.token_map, dw.topk, dw.depth,
                                                    w.max_topk, w.max_depth, o.frontier, dw.root_tokens,
                                                    dw.num_draft, w.max_T, o.tokens, o.parents, o.depth, o.anc,
                                                    o.q_row)
            elif self.fused_finish:
                ops.spec_tree_build_step_finish(self.ws_build, step, rows, dw.topk, dw.depth, w.max_topk,
                                                w.max_depth, o.frontier, dw.root_tokens, dw.num_draft, w.max_T,
                                                o.tokens, o.parents, o.depth, o.anc, o.q_row)
            elif dw.token_map is not None:
                ops.spec_tree_build_step_map(self.ws_build, step, rows, dw.token_map, dw.topk, dw.depth, w.max_topk,
                                             w.max_depth, o.frontier)
            else:
                ops.spec_tree_build_step(self.ws_build, step, rows, dw.topk, dw.depth, w.max_topk, w.max_depth,
                                         o.frontier)
        if not self.fused_finish:
            ops.spec_tree_build_finish(self.ws_build, dw.root_tokens, dw.topk, dw.depth, dw.num_draft, w.max_topk,
                                       w.max_depth, w.max_T, o.tokens, o.parents, o.depth, o.anc, o.q_row)

    def attention(self):
        w, dw, o = self.dw.w, self.dw, self.o
        if self.attn_status:
            o.attn_status.zero_()
        ops.spec_tree_attention(dw.q, dw.k_pages, dw.v_pages, dw.page_table, dw.prefix_lens, o.parents, dw.T_b,
                                w.sm_scale, o.attn_out, o.lse, o.attn_status if self.attn_status else None,
                                self.ws_attn)

    def verify(self):
        w, dw, o = self.dw.w, self.dw, self.o
        if self.from_logits:
            ops.spec_tree_verify_logits(dw.target_logits, dw.temperature, dw.draft_probs if self.sampling else None,
                                        o.q_row, o.tokens, o.parents, dw.T_b, dw.modes, w.philox_key,
                                        w.philox_offset, o.accept_len, o.accept_nodes, o.out_tokens, o.status,
                                        self.ws_verify)
            return
        ops.spec_tree_verify(dw.target, dw.draft_probs if self.sampling else None, o.q_row, o.tokens, o.parents,
                             dw.T_b, dw.modes, w.philox_key, w.philox_offset, o.accept_len, o.accept_nodes,
                             o.out_tokens, o.status, self.ws_verify)

    def compact(self):
        dw, o = self.dw, self.o
        ops.spec_kv_compact(dw.k_pages, dw.v_pages, dw.page_table, dw.prefix_lens, o.accept_nodes, o.accept_len,
                            o.new_prefix_lens)

    def run(self, compact: bool = None):
        self.build()
        self.attention()
        self.verify()
        if compact if compact is not None else self.dw.w.compact:
            self.compact()
        return self.o
