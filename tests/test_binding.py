"""Host-side argument checks of the torch binding (no GPU, no launch).

Every entry point of ``tree_attention_verification_03_amd.ops`` validates the
type, dtype, shape and layout of every tensor argument against the sizes it
passes to the library (B, max_T, Hq, Hkv, d, V, R, max_topk) before it loads
the library or launches anything, so a caller's mistake is a host-side error
and never an out-of-bounds device access. These tests hand it CPU tensors with
one mistake each and check the specific error; the library loader is replaced
by one that fails the test if it is reached.
"""
import pytest
import torch

from tree_attention_verification_03_amd import ops


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def forbidden():
        raise AssertionError("the library was reached before the arguments were checked")

    monkeypatch.setattr(ops, "load", forbidden)


i32 = lambda *s: torch.zeros(*s, dtype=torch.int32)
i64 = lambda *s: torch.zeros(*s, dtype=torch.int64)
f32 = lambda *s: torch.zeros(*s, dtype=torch.float32)
bf16 = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
i8 = lambda *s: torch.zeros(*s, dtype=torch.int8)
u8 = lambda *s: torch.zeros(*s, dtype=torch.uint8)

B, T, Hq, Hkv, d, P, PG, MP, V, R = 3, 9, 8, 2, 64, 40, 16, 6, 100, 5


def _attn(**kw):
    a = dict(q=bf16(B, T, Hq, d), k_pages=bf16(P, PG, Hkv, d), v_pages=bf16(P, PG, Hkv, d), page_table=i32(B, MP),
             prefix_lens=i32(B), parents=i32(B, T), T_b=i32(B), sm_scale=0.125, out=bf16(B, T, Hq, d),
             lse=f32(B, T, Hq), status=i32(B), ws=u8(64))
    a.update(kw)
    return ops.spec_tree_attention(**a)


@pytest.mark.parametrize("bad,msg", [
    (dict(v_pages=bf16(P, PG, Hkv, d + 64)), "v_pages must have shape"),
    (dict(page_table=i32(B + 1, MP)), "page_table must have shape"),
    (dict(prefix_lens=i32(B - 1)), "prefix_lens must have shape"),
    (dict(parents=i32(B, T - 1)), "parents must have shape"),
    (dict(T_b=i32(B + 2)), "T_b must have shape"),
    (dict(out=bf16(B, T, Hq, d)[:, :, :, :32]), "out must have shape"),
    (dict(lse=f32(B, T, Hq + 1)), "lse must have shape"),
    (dict(status=i32(1)), "status must have shape"),
    (dict(out=bf16(B, T, d, Hq).transpose(2, 3)), "out must be contiguous"),
    (dict(page_table=i64(B, MP)), "page_table must be torch.int32"),
    (dict(q=torch.zeros(B, T, Hq, d)), "q must be torch.bfloat16"),
])
def test_attention_rejects(bad, msg):
    with pytest.raises((ValueError, TypeError), match=msg):
        _attn(**bad)


def test_attention_checks_shapes_before_the_device():
    # every shape is right: the only complaint left is that the tensors are not on the GPU
    with pytest.raises(ValueError, match="must be on the GPU"):
        _attn()


def _verify(logits=False, **kw):
    a = dict(draft_probs=f32(B, R, V), q_row=i32(B, T), tokens=i32(B, T), parents=i32(B, T), T_b=i32(B),
             mode=i8(B), philox_key=(1, 2), philox_offset=0, accept_len=i32(B), accept_nodes=i32(B, T),
             out_tokens=i32(B, T), status=i32(B), ws=u8(64))
    if logits:
        a.update(logits=f32(B, T, V), temperature=f32(B))
    else:
        a.update(target=f32(B, T, V))
    a.update(kw)
    return (ops.spec_tree_verify_logits if logits else ops.spec_tree_verify)(**a)


@pytest.mark.parametrize("logits", [False, True], ids=["probs", "logits"])
@pytest.mark.parametrize("bad,msg", [
    (dict(draft_probs=f32(B, R, V - 1)), "draft_probs must have shape"),
    (dict(draft_probs=f32(B + 1, R, V)), "draft_probs must have shape"),
    (dict(q_row=None), "draft_probs needs q_row"),
    (dict(q_row=i32(B, T + 1)), "q_row must have shape"),
    (dict(tokens=i32(B, T - 2)), "tokens must have shape"),
    (dict(parents=i32(B - 1, T)), "parents must have shape"),
    (dict(mode=i8(B + 1)), "mode must have shape"),
    (dict(mode=i32(B)), "mode must be torch.int8"),
    (dict(accept_nodes=i32(B, 2)), "accept_nodes must have shape"),
    (dict(out_tokens=i32(B, T)[:, ::1].t().contiguous().t()), "out_tokens must be contiguous"),
    (dict(accept_len=i32(2 * B)), "accept_len must have shape"),
])
def test_verify_rejects(logits, bad, msg):
    with pytest.raises((ValueError, TypeError), match=msg):
        _verify(logits=logits, **bad)


def test_verify_logits_temperature_shape():
    with pytest.raises(ValueError, match="temperature must have shape"):
        _verify(logits=True, temperature=f32(B - 1))
    with pytest.raises(ValueError, match="must be on the GPU"):
        _verify(logits=True)


def test_build_rejects():
    K, D = 4, 3
    rows = f32(B, K, V)
    good = dict(ws=u8(64), step=2, draft_logprobs=rows, topk=i32(B), depth=i32(B), max_topk=K, max_depth=D,
                frontier_tokens=i32(B, K), root_tokens=i32(B), num_draft=i32(B), max_T=T, tokens=i32(B, T),
                parents=i32(B, T), depth_out=i32(B, T), anc_mask=i64(B, T), q_row=i32(B, T))
    for bad, msg in ((dict(frontier_tokens=i32(B, K - 1)), "frontier_tokens must have shape"),
                     (dict(topk=i32(B + 1)), "topk must have shape"),
                     (dict(anc_mask=i64(B, T + 1)), "anc_mask must have shape"),
                     (dict(q_row=i32(B, T - 1)), "q_row must have shape"),
                     (dict(draft_logprobs=f32(B, K - 1, V)), "needs 4 draft rows"),
                     (dict(draft_logprobs=f32(B, V, K).transpose(1, 2)), "rows must be contiguous")):
        with pytest.raises((ValueError, TypeError), match=msg):
            ops.spec_tree_build_step_finish(**{**good, **bad})
    with pytest.raises(ValueError, match="token_map must have shape"):
        ops.spec_tree_build_step_map(u8(64), 1, f32(B, 1, V), i32(V + 1), i32(B), i32(B), K, D, i32(B, K))
    with pytest.raises(ValueError, match="num_draft must have shape"):
        ops.spec_tree_build_finish(u8(64), i32(B), i32(B), i32(B), i32(B + 1), K, D, T, i32(B, T), i32(B, T),
                                   i32(B, T), i64(B, T), i32(B, T))


def test_mask_rejects():
    with pytest.raises(ValueError, match="anc_mask must have shape"):
        ops.spec_tree_mask(i32(B, T), None, i64(B, T - 1))
    with pytest.raises(ValueError, match="depth must have shape"):
        ops.spec_tree_mask(i32(B, T), i32(B), i64(B, T), depth=i32(B, T + 1))
    with pytest.raises(ValueError, match="must be on the GPU"):
        ops.spec_tree_mask(i32(B, T), i32(B), i64(B, T), depth=i32(B, T), status=i32(B))


def test_kv_compact_rejects():
    pool = bf16(3, P, PG, Hkv, d)
    good = dict(k_pages=pool[0], v_pages=bf16(3, P, PG, Hkv, d)[0], page_table=i32(B, MP), prefix_lens=i32(B),
                accept_nodes=i32(B, T), accept_len=i32(B), new_prefix_lens=i32(B), num_layers=3,
                layer_stride_elems=P * PG * Hkv * d)
    for bad, msg in ((dict(page_table=i64(B, MP)), "page_table must be torch.int32"),
                     (dict(prefix_lens=i32(B + 1)), "prefix_lens must have shape"),
                     (dict(accept_len=torch.zeros(B)), "accept_len must be torch.int32"),
                     (dict(new_prefix_lens=i32(B - 1)), "new_prefix_lens must have shape"),
                     (dict(v_pages=bf16(P, PG, Hkv, 2 * d)[:, :, :, ::2]), "v_pages must be contiguous"),
                     (dict(num_layers=4), "exceed its storage")):
        with pytest.raises((ValueError, TypeError), match=msg):
            ops.spec_kv_compact(**{**good, **bad})
    lens = i32(2 * B)
    with pytest.raises(ValueError, match="must not overlap"):
        ops.spec_kv_compact(**{**good, "prefix_lens": lens[:B], "new_prefix_lens": lens[1:B + 1]})
    with pytest.raises(ValueError, match="must be on the GPU"):
        ops.spec_kv_compact(**good)


def test_kv_prune_rejects():
    good = dict(page_table=i32(B, MP), prefix_lens=i32(B), T_b=i32(B), accept_nodes=i32(B, T), accept_len=i32(B),
                page=PG, num_pages=P, mode=ops.PRUNE_TAIL, freed=i32(B, T), freed_count=i32(B),
                new_prefix_lens=i32(B), status=i32(B))
    for bad, msg in ((dict(page_table=i64(B, MP)), "page_table must be torch.int32"),
                     (dict(T_b=i32(B + 1)), "T_b must have shape"),
                     (dict(freed=i32(B, T - 1)), "freed must have shape"),
                     (dict(freed_count=f32(B)), "freed_count must be torch.int32"),
                     (dict(status=i32(B, 2)), "status must have shape"),
                     (dict(accept_nodes=i32(B, 2 * T)[:, ::2]), "accept_nodes must be contiguous")):
        with pytest.raises((ValueError, TypeError), match=msg):
            ops.spec_kv_prune(**{**good, **bad})
    buf = i32(B * (T + 1))
    with pytest.raises(ValueError, match="freed must not overlap freed_count"):
        ops.spec_kv_prune(**{**good, "freed": buf[:B * T].view(B, T), "freed_count": buf[B * T - 1:B * T - 1 + B]})
    with pytest.raises(ValueError, match="page_table must not overlap accept_nodes"):
        ops.spec_kv_prune(**{**good, "page_table": buf[:B * MP].view(B, MP), "accept_nodes": buf[:B * T].view(B, T)})
    # new_prefix_lens may be prefix_lens itself (in place), but not a shifted view of it
    lens = i32(2 * B)
    with pytest.raises(ValueError, match="new_prefix_lens must not overlap prefix_lens"):
        ops.spec_kv_prune(**{**good, "prefix_lens": lens[:B], "new_prefix_lens": lens[1:B + 1]})
    with pytest.raises(ValueError, match="must be on the GPU"):
        ops.spec_kv_prune(**{**good, "new_prefix_lens": good["prefix_lens"]})


def test_attention_fp8_rejects():
    u8 = lambda *s: torch.zeros(*s, dtype=torch.uint8)
    good = dict(q=bf16(B, T, Hq, 128), k_pages=u8(P, PG, Hkv, 128), v_pages=u8(P, PG, Hkv, 128), k_scale=f32(Hkv),
                v_scale=f32(Hkv), page_table=i32(B, MP), prefix_lens=i32(B), parents=i32(B, T), T_b=i32(B),
                sm_scale=0.125, out=bf16(B, T, Hq, 128), lse=f32(B, T, Hq), status=i32(B), ws=u8(64))
    for bad, msg in ((dict(k_pages=bf16(P, PG, Hkv, 128)), "k_pages must be torch.uint8"),
                     (dict(v_pages=u8(P, PG, Hkv, 64)), "v_pages must have shape"),
                     (dict(k_scale=f32(Hkv + 1)), "k_scale must have shape"),
                     (dict(v_scale=torch.zeros(Hkv, dtype=torch.float64)), "v_scale must be torch.float32")):
        with pytest.raises((ValueError, TypeError), match=msg):
            ops.spec_tree_attention_fp8(**{**good, **bad})
    with pytest.raises(ValueError, match="must be on the GPU"):  # float8 pages are taken as their codes
        ops.spec_tree_attention_fp8(**{**good, "k_pages": good["k_pages"].view(torch.float8_e4m3fn)})
