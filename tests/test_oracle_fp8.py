"""Pins for the oracle's FP8 E4M3 values, its query quantization and the FP8-KV attention variant.

The E4M3 decoder and encoder are checked against torch's float8_e4m3fn conversions (a library routine for the same
OCP format) over every code and over ties, subnormals and random values; the row exponent at its boundaries; the
attention variant against closed forms that fix which scale multiplies which head.
"""
import numpy as np
import pytest
import torch

from oracle.attention import tree_attention_fp8
from oracle.fp8 import E4M3_MAX, e4m3_decode, e4m3_encode, q_row_exponent, quantize_q_rows


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got).sum() == 2
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert e4m3_decode(0x7E) == E4M3_MAX and e4m3_decode(0x01) == 2.0**-9 and e4m3_decode(0x38) == 1.0


def test_encode_matches_torch_on_ties_subnormals_and_random_values():
    vals = e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2  # every tie between neighbours (exact in fp32)
    rng = np.random.default_rng(0)
    xs = np.concatenate([vals, mids, -mids, rng.uniform(-448, 448, 5000), 2.0 ** rng.uniform(-12, 8.8, 5000),
                         rng.uniform(0, 2.0**-6, 2000)]).astype(np.float32)
    xs = xs[np.abs(xs) <= 448]
    assert np.array_equal(e4m3_encode(xs), _torch_encode(xs))
    # hand cases: ties go to the even code
    assert e4m3_encode(1.0625) == 0x38 and e4m3_encode(1.1875) == 0x3A and e4m3_encode(-2.0) == 0xC0
    assert e4m3_encode(3 * 2.0**-10) == 0x02 and e4m3_encode(2.0**-10) == 0x00 and e4m3_encode(3 * 2.0**-11) == 0x01
    with pytest.raises(ValueError):
        e4m3_encode(449.0)


def test_row_exponent_boundaries():
    assert q_row_exponent(0.0) == 0
    assert q_row_exponent(448.0) == 0 and q_row_exponent(448.0 * (1 + 2.0**-20)) == 1
    assert q_row_exponent(224.0) == -1 and q_row_exponent(224.5) == 0
    assert q_row_exponent(1.0) == -8 and q_row_exponent(1.75) == -8 and q_row_exponent(1.76) == -7
    for amax in np.random.default_rng(1).uniform(1e-3, 1e3, 200):
        e = q_row_exponent(float(amax))
        assert amax <= 448 * 2.0**e and amax > 448 * 2.0 ** (e - 1)


def test_quantize_rows():
    rng = np.random.default_rng(2)
    q = rng.normal(size=(3, 5, 128)) * rng.uniform(0.01, 10, size=(3, 5, 1))
    qq = quantize_q_rows(q)
    # scaling a row by a power of two scales its quantization by the same power
    np.testing.assert_array_equal(quantize_q_rows(q * 8.0), qq * 8.0)
    # relative error at most 2^-4 where the scaled element is a normal E4M3 value, absolute 2^-10 * 2^e elsewhere
    for r in np.ndindex(q.shape[:-1]):
        e = q_row_exponent(float(np.abs(q[r]).max()))
        big = np.abs(q[r]) * 2.0**-e >= 2.0**-6
        assert (np.abs(qq[r] - q[r])[big] <= 2.0**-4 * np.abs(q[r])[big]).all()
        assert (np.abs(qq[r] - q[r])[~big] <= 2.0**-10 * 2.0**e).all()
        assert np.abs(qq[r]).max() == pytest.approx(np.abs(q[r]).max(), rel=2.0**-4)
    # rows already on the grid come back unchanged
    grid = e4m3_decode(rng.integers(0, 126, size=(2, 64)).astype(np.uint8)) * 2.0**-3
    grid[:, 0] = 448 * 2.0**-3
    np.testing.assert_array_equal(quantize_q_rows(grid), grid)


def test_fp8_attention_single_key_returns_the_scaled_value_of_its_head():
    """One visible key (empty prefix, root-only tree): every head's output is its KV head's V row times that
    head's v_scale; lse is the scaled score with k_scale applied."""
    rng = np.random.default_rng(3)
    Hq, Hkv, d = 4, 2, 128
    k8 = rng.integers(0, 120, size=(1, 1, Hkv, d)).astype(np.uint8) | (rng.integers(0, 2, size=(1, 1, Hkv, d)) * 128).astype(np.uint8)
    v8 = rng.integers(0, 120, size=(1, 1, Hkv, d)).astype(np.uint8)
    ks, vs = np.array([0.5, 3.0]), np.array([2.0, 0.25])
    q = e4m3_decode(rng.integers(0, 100, size=(1, 1, Hq, d)).astype(np.uint8)) * 2.0**-4
    q[..., 0] = 448 * 2.0**-4  # rows already quantized: q is used as it is
    out, lse = tree_attention_fp8(q, k8, v8, ks, vs, np.zeros((1, 1), int), [0], [[-1]], [1], 0.125)
    for h in range(Hq):
        g = h // 2
        np.testing.assert_array_equal(out[0, 0, h], e4m3_decode(v8[0, 0, g]) * vs[g])
        assert lse[0, 0, h] == pytest.approx(0.125 * float(q[0, 0, h] @ (e4m3_decode(k8[0, 0, g]) * ks[g])), rel=1e-12)


def test_fp8_attention_equal_keys_average_the_values():
    """All keys equal: softmax is uniform, so the output is the mean of the visible dequantized values
    (prefix of 5 + the root for a root-only tree)."""
    rng = np.random.default_rng(4)
    d, L = 128, 5
    k8 = np.tile(rng.integers(0, 100, size=(1, 1, 1, d)).astype(np.uint8), (1, 8, 1, 1))
    v8 = rng.integers(0, 126, size=(1, 8, 1, d)).astype(np.uint8)
    q = rng.normal(size=(1, 1, 1, d))
    out, _ = tree_attention_fp8(q, k8, v8, [1.5], [0.75], np.zeros((1, 1), int), [L], [[-1]], [1], 0.1)
    np.testing.assert_allclose(out[0, 0, 0], e4m3_decode(v8[0, : L + 1, 0]).mean(axis=0) * 0.75, rtol=1e-12)
