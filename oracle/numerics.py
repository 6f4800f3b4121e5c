"""Rounding of real values to the storage formats the codec uses.

* fp16 with a chosen direction (nearest-even, toward -inf, toward +inf) for the
  per-group zero-point and scale.  The TempoKV page (section 3.1, Eq. 1) defines
  the scale and zero-point of the affine quantizer but not their storage
  format; the reading taken here stores both as fp16, the zero-point rounded
  down and the scale rounded up, so that the quantization grid still covers the
  group's range after rounding.
* bf16 and fp32 with round-to-nearest-even from fp64, for the centre means of
  the k-means update (NanoKV, Table 4: BF16 centres).

Everything is vectorized numpy.  The tests pin these functions against an
exact, table-driven definition over every finite value of the target format.
"""
from __future__ import annotations

import numpy as np

F16_MAX = 65504.0
BF16_MAX = float.fromhex("0x1.fep127")
F32_MAX = float(np.finfo(np.float32).max)


def fp16_round(v, mode: str) -> np.ndarray:
    """Round fp32 values to fp16: mode 'nearest' (ties to even), 'down' or 'up'.

    Raises ValueError for non-finite input or |v| > 65504 (outside the fp16
    range, which the codec treats as out of contract).
    """
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite value given to fp16 rounding")
    if np.any(np.abs(v) > F16_MAX):
        raise ValueError("value outside the fp16 range")
    h = v.astype(np.float16)  # round to nearest, ties to even
    if mode == "nearest":
        return h
    back = h.astype(np.float32)
    if mode == "down":
        fix = back > v
        h[fix] = np.nextafter(h[fix], np.float16(-np.inf))
    elif mode == "up":
        fix = back < v
        h[fix] = np.nextafter(h[fix], np.float16(np.inf))
    else:
        raise ValueError(f"unknown rounding mode {mode!r}")
    return h


def f16_bits(h: np.ndarray) -> np.ndarray:
    return np.asarray(h, dtype=np.float16).view(np.uint16)


def f16_from_bits(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16)


def _round_binary(x, p: int, emin: int, vmax: float) -> np.ndarray:
    """Round fp64 values to a binary format with p significand bits (implicit bit
    included) and smallest normal 2^emin, ties to even; gradual underflow."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value given to rounding")
    _, e = np.frexp(x)                      # |x| in [2^(e-1), 2^e)
    qexp = np.maximum(e - p, emin - p + 1)  # exponent of one unit in the last place
    y = np.rint(np.ldexp(x, -qexp))         # scaling by 2^k is exact; rint is ties-to-even
    out = np.ldexp(y, qexp)
    if np.any(np.abs(out) > vmax):
        raise ValueError("value outside the target range")
    return out


def round_to_bf16(x) -> np.ndarray:
    """fp64 -> bf16 (round to nearest even), returned as the float32 values."""
    return _round_binary(x, 8, -126, BF16_MAX).astype(np.float32)


def round_to_f32(x) -> np.ndarray:
    """fp64 -> fp32 (round to nearest even)."""
    return _round_binary(x, 24, -126, F32_MAX).astype(np.float32)


def round_to_storage(x, storage: str) -> np.ndarray:
    if storage == "bf16":
        return round_to_bf16(x)
    if storage == "f32":
        return round_to_f32(x)
    raise ValueError(f"unknown storage dtype {storage!r}")
