"""Oracle: fp8 (OCP e4m3fn) cast of q/k with one per-tensor scale -- test infrastructure.

The pages send fp8 payloads through the exchange with a separate scale
tensor beside them (LightX2V "Add optimized Ulysses attention path": the FP8
communication records carry ``payload`` and ``scale`` and ``attn_post_fp8``
dequantises with them).  They print neither the encoding nor the scale
formula.  Readings adopted here:

* encoding: OCP 8-bit floating point E4M3 ("e4m3fn"): 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits, subnormals at exponent 0, no infinities,
  0x7f / 0xff are NaN, largest finite magnitude 448;
* scale: one per tensor (q, k separately) over all P shards:
  ``amax = max |x|``, ``scale = amax / 448``, ``inv_scale = 448 / amax``,
  both in float32 (``amax == 0`` gives ``scale = inv_scale = 1``);
* cast: ``y = float32(x) * inv_scale`` (one float32 multiply), clamped to
  ``[-448, 448]``, then rounded to the nearest e4m3fn value, ties to the
  even code (round-to-nearest-even);
* dequantised value = ``decode(code) * scale``; attention folds the two
  scales into the score scale.

Everything below is the definition written out: a table of the 127
non-negative finite e4m3fn values and a nearest-value search.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _positive_table() -> np.ndarray:
    """Values of codes 0x00..0x7e (all finite non-negative e4m3fn values), float64."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        if e == 0:
            vals[code] = (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = _positive_table()


def decode(codes: np.ndarray) -> np.ndarray:
    """e4m3fn code bytes -> float64 values (NaN codes -> nan)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    out = np.where(mag == 0x7F, np.nan, _TABLE[np.minimum(mag, 126)])
    return np.where(c & 0x80, -out, out)


def encode(x: np.ndarray) -> np.ndarray:
    """Round float values (already within [-448, 448]) to e4m3fn codes, RNE.

    Nearest of the two neighbouring table values; on a tie the even code
    (mantissa LSB 0) wins.  The sign bit follows the sign of ``x``
    (so -0.0 and negative values that round to zero give 0x80).
    """
    xv = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(xv)) or np.any(np.abs(xv) > E4M3_MAX):
        raise ValueError("encode expects finite values within [-448, 448]")
    a = np.abs(xv)
    lo = np.searchsorted(_TABLE, a, side="right") - 1          # table[lo] <= a
    lo = np.clip(lo, 0, 126)
    hi = np.minimum(lo + 1, 126)
    d_lo = a - _TABLE[lo]
    d_hi = _TABLE[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(xv)
    return (mag | np.where(neg, 0x80, 0).astype(np.uint8)).astype(np.uint8)


def scales_from_amax(amax: float) -> tuple[np.float32, np.float32]:
    """(scale, inv_scale) in float32 for a tensor whose max |x| is ``amax``."""
    a = np.float32(amax)
    if a == 0:
        return np.float32(1.0), np.float32(1.0)
    return np.float32(a / np.float32(E4M3_MAX)), np.float32(np.float32(E4M3_MAX) / a)


def amax(arrays: list[np.ndarray]) -> np.float32:
    """max |x| over every element of every array (exact for bf16 inputs)."""
    return np.float32(max(float(np.max(np.abs(np.asarray(a, dtype=np.float64)))) if a.size else 0.0
                          for a in arrays))


def quantize(x: np.ndarray, inv_scale: np.float32) -> np.ndarray:
    """Codes of ``clamp(float32(x) * inv_scale, -448, 448)`` (float32 multiply)."""
    with np.errstate(over="ignore"):      # overflow to +-inf is clamped to +-448 below
        y = np.asarray(x, dtype=np.float32) * np.float32(inv_scale)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return encode(y)


def score_scale(softmax_scale: float, q_scale: np.float32, k_scale: np.float32) -> np.float32:
    """Score multiplier for fp8 q/k: float32 (softmax_scale * q_scale) * k_scale."""
    return np.float32(np.float32(np.float32(softmax_scale) * np.float32(q_scale)) * np.float32(k_scale))
