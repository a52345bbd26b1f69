"""Torch-facing binding of libspectree: argument checks and marshalling only.

Every function has the name of the C entry point it calls (include/spec_tree.h)
and takes device tensors; all computation happens in the HIP kernels. PyTorch
provides device memory and the current stream, nothing else.
"""
from __future__ import annotations

from typing import Optional

import torch

from ._lib import check, load

MODE_GREEDY = 0
MODE_SAMPLE = 1
STATUS_INVALID_PARENT = 1
STATUS_INVALID_TOKEN = 2
STATUS_NAN_INPUT = 4
STATUS_ZERO_Q = 8
STATUS_ZERO_RESIDUAL = 16
STATUS_INVALID_PAGE = 32
STATUS_INVALID_LENGTH = 64


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, dtype, name: str, contiguous: bool = True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def spec_abi_version() -> int:
    return int(load().spec_abi_version())


def spec_last_error() -> str:
    return load().spec_last_error().decode(errors="replace")


# ------------------------------------------------------------------ workspaces
def spec_tree_build_workspace_size(B: int, max_topk: int, max_depth: int) -> int:
    return int(load().spec_tree_build_workspace_size(B, max_topk, max_depth))


def spec_tree_attention_workspace_size(B, max_T, Hq, Hkv, d, page, max_pages) -> int:
    return int(load().spec_tree_attention_workspace_size(B, max_T, Hq, Hkv, d, page, max_pages))


def spec_tree_verify_workspace_size(B: int, max_T: int, V: int) -> int:
    return int(load().spec_tree_verify_workspace_size(B, max_T, V))


def zeroed_workspace(nbytes: int, device) -> torch.Tensor:
    """Workspaces must be zero-filled before first use (the library keeps them that way)."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ tree build
def _draft_rows(draft_logprobs, step, max_topk):
    _dev(draft_logprobs, torch.float32, "draft_logprobs", contiguous=False)
    B, F, V = draft_logprobs.shape
    if draft_logprobs.stride(2) != 1 or (F > 1 and draft_logprobs.stride(1) != V):
        raise ValueError("draft_logprobs rows must be contiguous [.., F, V]")
    if F < (1 if step == 1 else max_topk):
        raise ValueError(f"step {step} needs {1 if step == 1 else max_topk} draft rows per sequence, got {F}")
    return B, V


def _token_map(token_map, V):
    _dev(token_map, torch.int32, "token_map")
    if token_map.numel() != V:
        raise ValueError(f"token_map has {token_map.numel()} entries, the draft rows {V}")


def spec_tree_build_step(ws: torch.Tensor, step: int, draft_logprobs: torch.Tensor, topk: torch.Tensor,
                         depth: torch.Tensor, max_topk: int, max_depth: int, frontier_tokens: torch.Tensor):
    """draft_logprobs: fp32 [B, F, V] view (rows contiguous; any batch stride)."""
    B, V = _draft_rows(draft_logprobs, step, max_topk)
    _dev(topk, torch.int32, "topk")
    _dev(depth, torch.int32, "depth")
    _dev(frontier_tokens, torch.int32, "frontier_tokens")
    _dev(ws, torch.uint8, "ws")
    rc = load().spec_tree_build_step(_ptr(ws), ws.numel(), step, _ptr(draft_logprobs), draft_logprobs.stride(0),
                                     _ptr(topk), _ptr(depth), B, max_topk, max_depth, V, _ptr(frontier_tokens),
                                     _stream(ws))
    check(rc, "spec_tree_build_step")


def spec_tree_build_step_map(ws: torch.Tensor, step: int, draft_logprobs: torch.Tensor, token_map: torch.Tensor,
                             topk: torch.Tensor, depth: torch.Tensor, max_topk: int, max_depth: int,
                             frontier_tokens: torch.Tensor):
    """spec_tree_build_step over a truncated draft vocabulary: draft_logprobs fp32 [B, F, V_d], token_map
    int32 [V_d] (row entry i stands for token token_map[i])."""
    B, V = _draft_rows(draft_logprobs, step, max_topk)
    _token_map(token_map, V)
    _dev(topk, torch.int32, "topk")
    _dev(depth, torch.int32, "depth")
    _dev(frontier_tokens, torch.int32, "frontier_tokens")
    _dev(ws, torch.uint8, "ws")
    rc = load().spec_tree_build_step_map(_ptr(ws), ws.numel(), step, _ptr(draft_logprobs), _ptr(token_map),
                                         draft_logprobs.stride(0), _ptr(topk), _ptr(depth), B, max_topk, max_depth,
                                         V, _ptr(frontier_tokens), _stream(ws))
    check(rc, "spec_tree_build_step_map")


def _finish_outputs(topk, depth, frontier_tokens, root_tokens, num_draft, tokens, parents, depth_out, anc_mask, q_row,
                    ws):
    for n, t in (("topk", topk), ("depth", depth), ("frontier_tokens", frontier_tokens), ("root_tokens", root_tokens),
                 ("num_draft", num_draft), ("tokens", tokens), ("parents", parents), ("depth_out", depth_out),
                 ("q_row", q_row)):
        _dev(t, torch.int32, n)
    _dev(anc_mask, torch.int64, "anc_mask")  # uint64 bit patterns
    _dev(ws, torch.uint8, "ws")


def spec_tree_build_step_finish(ws: torch.Tensor, step: int, draft_logprobs: torch.Tensor, topk: torch.Tensor,
                                depth: torch.Tensor, max_topk: int, max_depth: int, frontier_tokens: torch.Tensor,
                                root_tokens, num_draft, max_T, tokens, parents, depth_out, anc_mask, q_row):
    """Step ``step`` plus the finish of the sequences whose depth is ``step`` (one launch)."""
    B, V = _draft_rows(draft_logprobs, step, max_topk)
    _finish_outputs(topk, depth, frontier_tokens, root_tokens, num_draft, tokens, parents, depth_out, anc_mask, q_row,
                    ws)
    rc = load().spec_tree_build_step_finish(
        _ptr(ws), ws.numel(), step, _ptr(draft_logprobs), draft_logprobs.stride(0), _ptr(topk), _ptr(depth), B,
        max_topk, max_depth, V, _ptr(frontier_tokens), _ptr(root_tokens), _ptr(num_draft), max_T, _ptr(tokens),
        _ptr(parents), _ptr(depth_out), _ptr(anc_mask), _ptr(q_row), _stream(ws))
    check(rc, "spec_tree_build_step_finish")


def spec_tree_build_step_finish_map(ws: torch.Tensor, step: int, draft_logprobs: torch.Tensor,
                                    token_map: torch.Tensor, topk: torch.Tensor, depth: torch.Tensor, max_topk: int,
                                    max_depth: int, frontier_tokens: torch.Tensor, root_tokens, num_draft, max_T,
                                    tokens, parents, depth_out, anc_mask, q_row):
    """spec_tree_build_step_finish over a truncated draft vocabulary (token_map int32 [V_d])."""
    B, V = _draft_rows(draft_logprobs, step, max_topk)
    _token_map(token_map, V)
    _finish_outputs(topk, depth, frontier_tokens, root_tokens, num_draft, tokens, parents, depth_out, anc_mask, q_row,
                    ws)
    rc = load().spec_tree_build_step_finish_map(
        _ptr(ws), ws.numel(), step, _ptr(draft_logprobs), _ptr(token_map), draft_logprobs.stride(0), _ptr(topk),
        _ptr(depth), B, max_topk, max_depth, V, _ptr(frontier_tokens), _ptr(root_tokens), _ptr(num_draft), max_T,
        _ptr(tokens), _ptr(parents), _ptr(depth_out), _ptr(anc_mask), _ptr(q_row), _stream(ws))
    check(rc, "spec_tree_build_step_finish_map")


def spec_tree_build_finish(ws, root_tokens, topk, depth, num_draft, max_topk, max_depth, max_T, tokens, parents,
                           depth_out, anc_mask, q_row):
    for n, t in (("root_tokens", root_tokens), ("topk", topk), ("depth", depth), ("num_draft", num_draft),
                 ("tokens", tokens), ("parents", parents), ("depth_out", depth_out), ("q_row", q_row)):
        _dev(t, torch.int32, n)
    _dev(anc_mask, torch.int64, "anc_mask")  # uint64 bit patterns
    B = root_tokens.shape[0]
    rc = load().spec_tree_build_finish(_ptr(ws), ws.numel(), _ptr(root_tokens), _ptr(topk), _ptr(depth),
                                       _ptr(num_draft), B, max_topk, max_depth, max_T, _ptr(tokens), _ptr(parents),
                                       _ptr(depth_out), _ptr(anc_mask), _ptr(q_row), _stream(ws))
    check(rc, "spec_tree_build_finish")


def spec_tree_mask(parents, T_b, anc_mask, depth=None, status=None):
    _dev(parents, torch.int32, "parents")
    _dev(anc_mask, torch.int64, "anc_mask")
    B, max_T = parents.shape
    rc = load().spec_tree_mask(_ptr(parents), _ptr(T_b), B, max_T, _ptr(anc_mask), _ptr(depth), _ptr(status),
                               _stream(parents))
    check(rc, "spec_tree_mask")


# ------------------------------------------------------------------ attention
def spec_tree_attention(q, k_pages, v_pages, page_table, prefix_lens, parents, T_b, sm_scale, out, lse=None,
                        status=None, ws=None):
    """q: bf16 [B, max_T, Hq, d]; k/v_pages: bf16 [P, page, Hkv, d]; page_table int32 [B, max_pages]."""
    _dev(q, torch.bfloat16, "q")
    _dev(k_pages, torch.bfloat16, "k_pages")
    _dev(v_pages, torch.bfloat16, "v_pages")
    _dev(page_table, torch.int32, "page_table")
    _dev(prefix_lens, torch.int32, "prefix_lens")
    _dev(parents, torch.int32, "parents")
    _dev(out, torch.bfloat16, "out")
    if T_b is not None:
        _dev(T_b, torch.int32, "T_b")
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    if status is not None:
        _dev(status, torch.int32, "status")
    B, max_T, Hq, d = q.shape
    P, page, Hkv, d2 = k_pages.shape
    if d2 != d or v_pages.shape != k_pages.shape or out.shape != q.shape or parents.shape != (B, max_T):
        raise ValueError("inconsistent attention shapes")
    max_pages = page_table.shape[1]
    if ws is None:
        ws = zeroed_workspace(spec_tree_attention_workspace_size(B, max_T, Hq, Hkv, d, page, max_pages), q.device)
    rc = load().spec_tree_attention(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_table), _ptr(prefix_lens),
                                    _ptr(parents), _ptr(T_b), B, max_T, Hq, Hkv, d, page, max_pages, P,
                                    float(sm_scale), _ptr(out), _ptr(lse), _ptr(status), _ptr(ws), ws.numel(),
                                    _stream(q))
    check(rc, "spec_tree_attention")
    return ws


# ------------------------------------------------------------------ verify
def spec_tree_verify(target, draft_probs, q_row, tokens, parents, T_b, mode, philox_key, philox_offset, accept_len,
                     accept_nodes, out_tokens, status, ws=None):
    _dev(target, torch.float32, "target")
    B, max_T, V = target.shape
    R = 0
    if draft_probs is not None:
        _dev(draft_probs, torch.float32, "draft_probs")
        R = draft_probs.shape[1]
        _dev(q_row, torch.int32, "q_row")
    for n, t in (("tokens", tokens), ("parents", parents), ("accept_len", accept_len),
                 ("accept_nodes", accept_nodes), ("out_tokens", out_tokens), ("status", status)):
        _dev(t, torch.int32, n)
    _dev(mode, torch.int8, "mode")
    if ws is None:
        ws = zeroed_workspace(spec_tree_verify_workspace_size(B, max_T, V), target.device)
    k0, k1 = (int(x) & 0xFFFFFFFFFFFFFFFF for x in philox_key)
    rc = load().spec_tree_verify(_ptr(target), _ptr(draft_probs), _ptr(q_row), _ptr(tokens), _ptr(parents), _ptr(T_b),
                                 _ptr(mode), k0, k1, int(philox_offset) & 0xFFFFFFFFFFFFFFFF, B, max_T, R, V,
                                 _ptr(accept_len), _ptr(accept_nodes), _ptr(out_tokens), _ptr(status), _ptr(ws),
                                 ws.numel(), _stream(target))
    check(rc, "spec_tree_verify")
    return ws


def spec_tree_verify_logits_workspace_size(B: int, max_T: int, V: int) -> int:
    return int(load().spec_tree_verify_logits_workspace_size(B, max_T, V))


def spec_tree_verify_logits(logits, temperature, draft_probs, q_row, tokens, parents, T_b, mode, philox_key,
                            philox_offset, accept_len, accept_nodes, out_tokens, status, ws=None):
    """spec_tree_verify with the sampling sequences' target distributions formed from ``logits`` (fp32
    [B, max_T, V]) and ``temperature`` (fp32 [B] or None = 1) inside the library."""
    _dev(logits, torch.float32, "logits")
    B, max_T, V = logits.shape
    if temperature is not None:
        _dev(temperature, torch.float32, "temperature")
        if temperature.numel() < B:
            raise ValueError(f"temperature holds {temperature.numel()} values for {B} sequences")
    R = 0
    if draft_probs is not None:
        _dev(draft_probs, torch.float32, "draft_probs")
        R = draft_probs.shape[1]
        _dev(q_row, torch.int32, "q_row")
    for n, t in (("tokens", tokens), ("parents", parents), ("accept_len", accept_len),
                 ("accept_nodes", accept_nodes), ("out_tokens", out_tokens), ("status", status)):
        _dev(t, torch.int32, n)
    _dev(mode, torch.int8, "mode")
    if ws is None:
        ws = zeroed_workspace(spec_tree_verify_logits_workspace_size(B, max_T, V), logits.device)
    k0, k1 = (int(x) & 0xFFFFFFFFFFFFFFFF for x in philox_key)
    rc = load().spec_tree_verify_logits(_ptr(logits), _ptr(temperature), _ptr(draft_probs), _ptr(q_row), _ptr(tokens),
                                        _ptr(parents), _ptr(T_b), _ptr(mode), k0, k1,
                                        int(philox_offset) & 0xFFFFFFFFFFFFFFFF, B, max_T, R, V, _ptr(accept_len),
                                        _ptr(accept_nodes), _ptr(out_tokens), _ptr(status), _ptr(ws), ws.numel(),
                                        _stream(logits))
    check(rc, "spec_tree_verify_logits")
    return ws


# ------------------------------------------------------------------ compaction
def spec_kv_compact(k_pages, v_pages, page_table, prefix_lens, accept_nodes, accept_len, new_prefix_lens,
                    num_layers: int = 1, layer_stride_elems: int = 0):
    """k_pages / v_pages: bf16 [P, page, Hkv, d] (layer 0 of ``num_layers`` pools ``layer_stride_elems`` apart)."""
    _dev(k_pages, torch.bfloat16, "k_pages", contiguous=False)
    _dev(v_pages, torch.bfloat16, "v_pages", contiguous=False)
    P, page, Hkv, d = k_pages.shape
    B, max_T = accept_nodes.shape
    rc = load().spec_kv_compact(_ptr(k_pages), _ptr(v_pages), _ptr(page_table), _ptr(prefix_lens), _ptr(accept_nodes),
                                _ptr(accept_len), B, max_T, Hkv, d, page, page_table.shape[1], P, num_layers,
                                layer_stride_elems, _ptr(new_prefix_lens), _stream(k_pages))
    check(rc, "spec_kv_compact")
