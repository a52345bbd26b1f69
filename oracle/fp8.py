"""FP8 E4M3 values and the FP8-KV variant's query quantization (test infrastructure: part of the CPU oracle; only
tests, the smoke check and the bench's CPU baseline use it).

Sources: tanhdev "Tech Radar: SGLang EAGLE-2", section 3 "Quantitative Hardware Benchmarks on NVIDIA H100" (FP8
targets); n1n.ai "Speculative Decoding in Production: EAGLE-3 Dynamic Trees", FAQ "Can speculative decoding be
combined with FP8 or AWQ quantization?" (FP8 target execution alongside speculative decoding). The pages fix no
format; the readings below are this variant's definition.

Format (the OCP 8-bit floating point E4M3 encoding, "fn": no infinities): bit 7 sign, bits 6..3 exponent e
(bias 7), bits 2..0 mantissa m. e = 0: value m * 2^-9 (subnormal); 1 <= e <= 15: (1 + m / 8) * 2^(e - 7), except
e = 15, m = 7, which is NaN. Largest finite magnitude 448.

Query quantization (reading): every (sequence, node, query head) row of q is scaled by 2^-e with e the smallest
integer such that max|q| <= 448 * 2^e (e = 0 for an all-zero row), and each element is rounded to the nearest
E4M3 value, ties to the even code. The row then stands for code value * 2^e.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0**-9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & (c & 7 == 7), np.nan, val)
    return sign * val


_FINITE = np.array([c for c in range(127)], dtype=np.int64)  # non-negative finite codes, increasing in value
_FINITE_VAL = e4m3_decode(_FINITE)


def e4m3_encode(x) -> np.ndarray:
    """float values with |x| <= 448 -> uint8 codes, round to nearest, ties to the even code."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or (np.abs(x) > E4M3_MAX).any():
        raise ValueError("e4m3_encode: |x| must be finite and <= 448")
    a = np.abs(x)
    hi = np.searchsorted(_FINITE_VAL, a, side="left")  # first finite value >= a
    hi = np.minimum(hi, len(_FINITE) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - _FINITE_VAL[lo], _FINITE_VAL[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_FINITE[hi] % 2 == 0))
    code = np.where(a == _FINITE_VAL[hi], _FINITE[hi], np.where(pick_hi, _FINITE[hi], _FINITE[lo]))
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def q_row_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e (0 for amax == 0)."""
    if amax == 0.0:
        return 0
    e = int(np.ceil(np.log2(amax / E4M3_MAX)))
    while amax > E4M3_MAX * 2.0**e:  # exact comparisons fix the log2 estimate
        e += 1
    while amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return e


def quantize_q_rows(q) -> np.ndarray:
    """q [..., d] (float) -> the values the quantized rows stand for (float64, same shape)."""
    q = np.asarray(q, dtype=np.float64)
    out = np.empty_like(q)
    flat_q, flat_o = q.reshape(-1, q.shape[-1]), out.reshape(-1, q.shape[-1])
    for r in range(flat_q.shape[0]):
        e = q_row_exponent(float(np.abs(flat_q[r]).max()))
        flat_o[r] = e4m3_decode(e4m3_encode(flat_q[r] * 2.0**-e)) * 2.0**e
    return out
