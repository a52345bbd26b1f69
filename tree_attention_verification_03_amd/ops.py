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


def _check(*specs):
    """Validate tensor arguments before any launch: specs are (name, tensor, dtype, shape, contiguous);
    a shape entry of None matches any size. Every argument's type, dtype, shape and layout is checked
    first, then that all of them sit on one GPU, so a mistake in any argument raises here on the host
    instead of reaching a kernel that indexes by the declared sizes."""
    _check_layout(*specs)
    _check_device(*specs)


def _check_layout(*specs):
    for name, t, dtype, shape, contiguous in specs:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor (got {type(t).__name__})")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
        if shape is not None and (t.dim() != len(shape)
                                  or any(w is not None and int(g) != int(w) for g, w in zip(t.shape, shape))):
            want = tuple("*" if w is None else int(w) for w in shape)
            raise ValueError(f"{name} must have shape {want} (got {tuple(t.shape)})")
        if contiguous and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _check_device(*specs):
    dev = None
    for name, t, _, _, _ in specs:
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU (got {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other arguments on {dev}")


def _spec(name, t, dtype, shape=None, contiguous=True):
    return (name, t, dtype, shape, contiguous)


def _opt(name, t, dtype, shape=None, contiguous=True):
    """An optional argument: no spec when it is None."""
    return () if t is None else ((name, t, dtype, shape, contiguous),)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _overlap(a: torch.Tensor, b: torch.Tensor) -> bool:
    a0, b0 = a.data_ptr(), b.data_ptr()
    return a0 < b0 + b.numel() * b.element_size() and b0 < a0 + a.numel() * a.element_size()


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
    """Shape of a step's draft rows: fp32 [B, F, V] view whose rows are contiguous (any batch stride)."""
    if not isinstance(draft_logprobs, torch.Tensor) or draft_logprobs.dim() != 3:
        raise ValueError("draft_logprobs must be a 3-D tensor [B, F, V]")
    B, F, V = draft_logprobs.shape
    if draft_logprobs.stride(2) != 1 or (F > 1 and draft_logprobs.stride(1) != V):
        raise ValueError("draft_logprobs rows must be contiguous [.., F, V]")
    if F < (1 if step == 1 else max_topk):
        raise ValueError(f"step {step} needs {1 if step == 1 else max_topk} draft rows per sequence, got {F}")
    return B, V


def _step_specs(ws, draft_logprobs, topk, depth, frontier_tokens, B, max_topk):
    return (_spec("draft_logprobs", draft_logprobs, torch.float32, contiguous=False),
            _spec("topk", topk, torch.int32, (B,)), _spec("depth", depth, torch.int32, (B,)),
            _spec("frontier_tokens", frontier_tokens, torch.int32, (B, max_topk)),
            _spec("ws", ws, torch.uint8, (None,)))


def _finish_specs(root_tokens, num_draft, tokens, parents, depth_out, anc_mask, q_row, B, max_T):
    return (_spec("root_tokens", root_tokens, torch.int32, (B,)), _spec("num_draft", num_draft, torch.int32, (B,)),
            _spec("tokens", tokens, torch.int32, (B, max_T)), _spec("parents", parents, torch.int32, (B, max_T)),
            _spec("depth_out", depth_out, torch.int32, (B, max_T)),
            _spec("anc_mask", anc_mask, torch.int64, (B, max_T)),  # uint64 bit patterns
            _spec("q_row", q_row, torch.int32, (B, max_T)))


def spec_tree_build_step(ws: torch.Tensor, step: int, draft_logprobs: torch.Tensor, topk: torch.Tensor,
                         depth: torch.Tensor, max_topk: int, max_depth: int, frontier_tokens: torch.Tensor):
    """draft_logprobs: fp32 [B, F, V] view (rows contiguous; any batch stride)."""
    B, V = _draft_rows(draft_logprobs, step, max_topk)
    _check(*_step_specs(ws, draft_logprobs, topk, depth, frontier_tokens, B, max_topk))
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
    _check(*_step_specs(ws, draft_logprobs, topk, depth, frontier_tokens, B, max_topk),
           _spec("token_map", token_map, torch.int32, (V,)))
    rc = load().spec_tree_build_step_map(_ptr(ws), ws.numel(), step, _ptr(draft_logprobs), _ptr(token_map),
                                         draft_logprobs.stride(0), _ptr(topk), _ptr(depth), B, max_topk, max_depth,
                                         V, _ptr(frontier_tokens), _stream(ws))
    check(rc, "spec_tree_build_step_map")


def spec_tree_build_step_finish(ws: torch.Tensor, step: int, draft_logprobs: torch.Tensor, topk: torch.Tensor,
                                depth: torch.Tensor, max_topk: int, max_depth: int, frontier_tokens: torch.Tensor,
                                root_tokens, num_draft, max_T, tokens, parents, depth_out, anc_mask, q_row):
    """Step ``step`` plus the finish of the sequences whose depth is ``step`` (one launch)."""
    B, V = _draft_rows(draft_logprobs, step, max_topk)
    _check(*_step_specs(ws, draft_logprobs, topk, depth, frontier_tokens, B, max_topk),
           *_finish_specs(root_tokens, num_draft, tokens, parents, depth_out, anc_mask, q_row, B, max_T))
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
    _check(*_step_specs(ws, draft_logprobs, topk, depth, frontier_tokens, B, max_topk),
           _spec("token_map", token_map, torch.int32, (V,)),
           *_finish_specs(root_tokens, num_draft, tokens, parents, depth_out, anc_mask, q_row, B, max_T))
    rc = load().spec_tree_build_step_finish_map(
        _ptr(ws), ws.numel(), step, _ptr(draft_logprobs), _ptr(token_map), draft_logprobs.stride(0), _ptr(topk),
        _ptr(depth), B, max_topk, max_depth, V, _ptr(frontier_tokens), _ptr(root_tokens), _ptr(num_draft), max_T,
        _ptr(tokens), _ptr(parents), _ptr(depth_out), _ptr(anc_mask), _ptr(q_row), _stream(ws))
    check(rc, "spec_tree_build_step_finish_map")


def spec_tree_build_finish(ws, root_tokens, topk, depth, num_draft, max_topk, max_depth, max_T, tokens, parents,
                           depth_out, anc_mask, q_row):
    if not isinstance(root_tokens, torch.Tensor) or root_tokens.dim() != 1:
        raise ValueError("root_tokens must be a 1-D tensor [B]")
    B = root_tokens.shape[0]
    _check(_spec("topk", topk, torch.int32, (B,)), _spec("depth", depth, torch.int32, (B,)),
           _spec("ws", ws, torch.uint8, (None,)),
           *_finish_specs(root_tokens, num_draft, tokens, parents, depth_out, anc_mask, q_row, B, max_T))
    rc = load().spec_tree_build_finish(_ptr(ws), ws.numel(), _ptr(root_tokens), _ptr(topk), _ptr(depth),
                                       _ptr(num_draft), B, max_topk, max_depth, max_T, _ptr(tokens), _ptr(parents),
                                       _ptr(depth_out), _ptr(anc_mask), _ptr(q_row), _stream(ws))
    check(rc, "spec_tree_build_finish")


def spec_tree_mask(parents, T_b, anc_mask, depth=None, status=None):
    """parents int32 [B, max_T]; T_b int32 [B] or None; anc_mask int64 [B, max_T] (uint64 bits); depth int32
    [B, max_T] or None; status int32 [B] or None (uint32 bits)."""
    if not isinstance(parents, torch.Tensor) or parents.dim() != 2:
        raise ValueError("parents must be a 2-D tensor [B, max_T]")
    B, max_T = parents.shape
    _check(_spec("parents", parents, torch.int32, (B, max_T)), *_opt("T_b", T_b, torch.int32, (B,)),
           _spec("anc_mask", anc_mask, torch.int64, (B, max_T)), *_opt("depth", depth, torch.int32, (B, max_T)),
           *_opt("status", status, torch.int32, (B,)))
    rc = load().spec_tree_mask(_ptr(parents), _ptr(T_b), B, max_T, _ptr(anc_mask), _ptr(depth), _ptr(status),
                               _stream(parents))
    check(rc, "spec_tree_mask")


# ------------------------------------------------------------------ attention
def spec_tree_attention(q, k_pages, v_pages, page_table, prefix_lens, parents, T_b, sm_scale, out, lse=None,
                        status=None, ws=None):
    """q: bf16 [B, max_T, Hq, d]; k/v_pages: bf16 [P, page, Hkv, d]; page_table int32 [B, max_pages]."""
    for name, t, nd in (("q", q, 4), ("k_pages", k_pages, 4), ("page_table", page_table, 2)):
        if not isinstance(t, torch.Tensor) or t.dim() != nd:
            raise ValueError(f"{name} must be a {nd}-D tensor")
    B, max_T, Hq, d = q.shape
    P, page, Hkv = k_pages.shape[:3]
    max_pages = page_table.shape[1]
    _check(_spec("q", q, torch.bfloat16), _spec("k_pages", k_pages, torch.bfloat16, (P, page, Hkv, d)),
           _spec("v_pages", v_pages, torch.bfloat16, (P, page, Hkv, d)),
           _spec("page_table", page_table, torch.int32, (B, max_pages)),
           _spec("prefix_lens", prefix_lens, torch.int32, (B,)), _spec("parents", parents, torch.int32, (B, max_T)),
           *_opt("T_b", T_b, torch.int32, (B,)), _spec("out", out, torch.bfloat16, (B, max_T, Hq, d)),
           *_opt("lse", lse, torch.float32, (B, max_T, Hq)), *_opt("status", status, torch.int32, (B,)),
           *_opt("ws", ws, torch.uint8, (None,)))
    if ws is None:
        ws = zeroed_workspace(spec_tree_attention_workspace_size(B, max_T, Hq, Hkv, d, page, max_pages), q.device)
    rc = load().spec_tree_attention(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_table), _ptr(prefix_lens),
                                    _ptr(parents), _ptr(T_b), B, max_T, Hq, Hkv, d, page, max_pages, P,
                                    float(sm_scale), _ptr(out), _ptr(lse), _ptr(status), _ptr(ws), ws.numel(),
                                    _stream(q))
    check(rc, "spec_tree_attention")
    return ws


def spec_tree_attention_fp8(q, k_pages, v_pages, k_scale, v_scale, page_table, prefix_lens, parents, T_b, sm_scale,
                            out, lse=None, status=None, ws=None):
    """FP8-KV variant (d = 128): k/v_pages uint8 (or float8_e4m3fn) [P, page, Hkv, 128] E4M3 codes, k_scale /
    v_scale fp32 [Hkv]; q bf16 [B, max_T, Hq, 128]; other arguments as spec_tree_attention."""
    for name, t, nd in (("q", q, 4), ("k_pages", k_pages, 4), ("page_table", page_table, 2)):
        if not isinstance(t, torch.Tensor) or t.dim() != nd:
            raise ValueError(f"{name} must be a {nd}-D tensor")
    k_pages, v_pages = (t.view(torch.uint8) if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn else t
                        for t in (k_pages, v_pages))
    B, max_T, Hq, d = q.shape
    P, page, Hkv = k_pages.shape[:3]
    max_pages = page_table.shape[1]
    _check(_spec("q", q, torch.bfloat16), _spec("k_pages", k_pages, torch.uint8, (P, page, Hkv, d)),
           _spec("v_pages", v_pages, torch.uint8, (P, page, Hkv, d)), _spec("k_scale", k_scale, torch.float32, (Hkv,)),
           _spec("v_scale", v_scale, torch.float32, (Hkv,)),
           _spec("page_table", page_table, torch.int32, (B, max_pages)),
           _spec("prefix_lens", prefix_lens, torch.int32, (B,)), _spec("parents", parents, torch.int32, (B, max_T)),
           *_opt("T_b", T_b, torch.int32, (B,)), _spec("out", out, torch.bfloat16, (B, max_T, Hq, d)),
           *_opt("lse", lse, torch.float32, (B, max_T, Hq)), *_opt("status", status, torch.int32, (B,)),
           *_opt("ws", ws, torch.uint8, (None,)))
    if ws is None:
        ws = zeroed_workspace(spec_tree_attention_workspace_size(B, max_T, Hq, Hkv, d, page, max_pages), q.device)
    rc = load().spec_tree_attention_fp8(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale), _ptr(v_scale),
                                        _ptr(page_table), _ptr(prefix_lens), _ptr(parents), _ptr(T_b), B, max_T, Hq,
                                        Hkv, d, page, max_pages, P, float(sm_scale), _ptr(out), _ptr(lse),
                                        _ptr(status), _ptr(ws), ws.numel(), _stream(q))
    check(rc, "spec_tree_attention_fp8")
    return ws


def spec_tree_attention_noalloc(q, k_pages, v_pages, page_table, prefix_lens, parents, T_b, sm_scale, out, lse=None,
                                status=None):
    """spec_tree_attention with its split-K workspace in the library's own device scratch (64 MiB per GPU): no
    allocation, for callers that cannot allocate (graph capture, serving loops). Calls on one GPU must not overlap."""
    for name, t, nd in (("q", q, 4), ("k_pages", k_pages, 4), ("page_table", page_table, 2)):
        if not isinstance(t, torch.Tensor) or t.dim() != nd:
            raise ValueError(f"{name} must be a {nd}-D tensor")
    B, max_T, Hq, d = q.shape
    P, page, Hkv = k_pages.shape[:3]
    max_pages = page_table.shape[1]
    _check(_spec("q", q, torch.bfloat16), _spec("k_pages", k_pages, torch.bfloat16, (P, page, Hkv, d)),
           _spec("v_pages", v_pages, torch.bfloat16, (P, page, Hkv, d)),
           _spec("page_table", page_table, torch.int32, (B, max_pages)),
           _spec("prefix_lens", prefix_lens, torch.int32, (B,)), _spec("parents", parents, torch.int32, (B, max_T)),
           *_opt("T_b", T_b, torch.int32, (B,)), _spec("out", out, torch.bfloat16, (B, max_T, Hq, d)),
           *_opt("lse", lse, torch.float32, (B, max_T, Hq)), *_opt("status", status, torch.int32, (B,)))
    rc = load().spec_tree_attention_noalloc(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_table), _ptr(prefix_lens),
                                            _ptr(parents), _ptr(T_b), B, max_T, Hq, Hkv, d, page, max_pages, P,
                                            float(sm_scale), _ptr(out), _ptr(lse), _ptr(status), _stream(q))
    check(rc, "spec_tree_attention_noalloc")


# ------------------------------------------------------------------ verify
def _verify_specs(rows, rows_name, draft_probs, q_row, tokens, parents, T_b, mode, accept_len, accept_nodes,
                  out_tokens, status, ws):
    if not isinstance(rows, torch.Tensor) or rows.dim() != 3:
        raise ValueError(f"{rows_name} must be a 3-D tensor [B, max_T, V]")
    B, max_T, V = rows.shape
    R = 0
    if draft_probs is not None:
        if not isinstance(draft_probs, torch.Tensor) or draft_probs.dim() != 3:
            raise ValueError("draft_probs must be a 3-D tensor [B, R, V]")
        R = draft_probs.shape[1]
        if q_row is None:
            raise ValueError("draft_probs needs q_row")
    specs = (_spec(rows_name, rows, torch.float32), *_opt("draft_probs", draft_probs, torch.float32, (B, None, V)),
             *_opt("q_row", q_row, torch.int32, (B, max_T)), _spec("tokens", tokens, torch.int32, (B, max_T)),
             _spec("parents", parents, torch.int32, (B, max_T)), *_opt("T_b", T_b, torch.int32, (B,)),
             _spec("mode", mode, torch.int8, (B,)), _spec("accept_len", accept_len, torch.int32, (B,)),
             _spec("accept_nodes", accept_nodes, torch.int32, (B, max_T)),
             _spec("out_tokens", out_tokens, torch.int32, (B, max_T)), _spec("status", status, torch.int32, (B,)),
             *_opt("ws", ws, torch.uint8, (None,)))
    return B, max_T, V, R, specs


def spec_tree_verify(target, draft_probs, q_row, tokens, parents, T_b, mode, philox_key, philox_offset, accept_len,
                     accept_nodes, out_tokens, status, ws=None):
    B, max_T, V, R, specs = _verify_specs(target, "target", draft_probs, q_row, tokens, parents, T_b, mode,
                                          accept_len, accept_nodes, out_tokens, status, ws)
    _check(*specs)
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
    B, max_T, V, R, specs = _verify_specs(logits, "logits", draft_probs, q_row, tokens, parents, T_b, mode,
                                          accept_len, accept_nodes, out_tokens, status, ws)
    _check(*specs, *_opt("temperature", temperature, torch.float32, (B,)))
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
    """k_pages / v_pages: bf16 [P, page, Hkv, d], dense; layer l's pool starts ``l * layer_stride_elems`` elements
    after layer 0's (a contiguous [num_layers, P, page, Hkv, d] tensor passes its layer-0 view and
    P * page * Hkv * d). ``new_prefix_lens`` must not overlap ``prefix_lens``."""
    for name, t, nd in (("k_pages", k_pages, 4), ("accept_nodes", accept_nodes, 2), ("page_table", page_table, 2)):
        if not isinstance(t, torch.Tensor) or t.dim() != nd:
            raise ValueError(f"{name} must be a {nd}-D tensor")
    P, page, Hkv, d = k_pages.shape
    B, max_T = accept_nodes.shape
    specs = (_spec("k_pages", k_pages, torch.bfloat16, (P, page, Hkv, d)),
             _spec("v_pages", v_pages, torch.bfloat16, (P, page, Hkv, d)),
             _spec("page_table", page_table, torch.int32, (B, None)),
             _spec("prefix_lens", prefix_lens, torch.int32, (B,)),
             _spec("accept_nodes", accept_nodes, torch.int32, (B, max_T)),
             _spec("accept_len", accept_len, torch.int32, (B,)),
             _spec("new_prefix_lens", new_prefix_lens, torch.int32, (B,)))
    _check_layout(*specs)
    if _overlap(new_prefix_lens, prefix_lens):
        raise ValueError("new_prefix_lens must not overlap prefix_lens (blocks still read L_b while it is written)")
    if num_layers < 1:
        raise ValueError("num_layers must be >= 1")
    for name, t in (("k_pages", k_pages), ("v_pages", v_pages)):
        need = t.storage_offset() + (num_layers - 1) * int(layer_stride_elems) + t.numel()
        if t.untyped_storage().nbytes() // t.element_size() < need:
            raise ValueError(f"{name}: {num_layers} layers {layer_stride_elems} elements apart exceed its storage")
    _check_device(*specs)
    rc = load().spec_kv_compact(_ptr(k_pages), _ptr(v_pages), _ptr(page_table), _ptr(prefix_lens), _ptr(accept_nodes),
                                _ptr(accept_len), B, max_T, Hkv, d, page, page_table.shape[1], P, num_layers,
                                layer_stride_elems, _ptr(new_prefix_lens), _stream(k_pages))
    check(rc, "spec_kv_compact")


PRUNE_TAIL = 0  # after spec_kv_compact: release the pages past the new length that the tree touched
PRUNE_REMAP = 1  # page == 1: zero-copy remap of the accepted path, release the rejected nodes' slots


def spec_kv_prune(page_table, prefix_lens, T_b, accept_nodes, accept_len, page: int, num_pages: int, mode: int,
                  freed, freed_count, new_prefix_lens, status=None):
    """page_table int32 [B, max_pages] (rewritten in place); prefix_lens, T_b, accept_len int32 [B]; accept_nodes
    int32 [B, max_T]; outputs freed int32 [B, max_T], freed_count int32 [B], new_prefix_lens int32 [B] (may be
    prefix_lens itself), status int32 [B] or None (uint32 bits)."""
    for name, t in (("accept_nodes", accept_nodes), ("page_table", page_table)):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError(f"{name} must be a 2-D tensor")
    B, max_T = accept_nodes.shape
    specs = (_spec("page_table", page_table, torch.int32, (B, None)),
             _spec("prefix_lens", prefix_lens, torch.int32, (B,)), _spec("T_b", T_b, torch.int32, (B,)),
             _spec("accept_nodes", accept_nodes, torch.int32, (B, max_T)),
             _spec("accept_len", accept_len, torch.int32, (B,)), _spec("freed", freed, torch.int32, (B, max_T)),
             _spec("freed_count", freed_count, torch.int32, (B,)),
             _spec("new_prefix_lens", new_prefix_lens, torch.int32, (B,)), *_opt("status", status, torch.int32, (B,)))
    _check_layout(*specs)
    outs = [("page_table", page_table), ("freed", freed), ("freed_count", freed_count),
            ("new_prefix_lens", new_prefix_lens)] + ([("status", status)] if status is not None else [])
    ins = [("prefix_lens", prefix_lens), ("T_b", T_b), ("accept_nodes", accept_nodes), ("accept_len", accept_len)]
    for i, (na, a) in enumerate(outs):
        for nb, b in outs[i + 1:] + ins:
            if _overlap(a, b) and not (na == "new_prefix_lens" and b.data_ptr() == a.data_ptr() and nb == "prefix_lens"):
                raise ValueError(f"{na} must not overlap {nb}")
    _check_device(*specs)
    rc = load().spec_kv_prune(_ptr(page_table), _ptr(prefix_lens), _ptr(T_b), _ptr(accept_nodes), _ptr(accept_len), B,
                              max_T, page, page_table.shape[1], num_pages, mode, _ptr(freed), _ptr(freed_count),
                              _ptr(new_prefix_lens), _ptr(status), _stream(page_table))
    check(rc, "spec_kv_prune")
