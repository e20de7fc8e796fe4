"""Exact decoders for the two storage formats of the path (fp64).

The KV cache is FP8 throughout ("PageWeaver: KV-Guided Query Unions for Sparse
Attention", Abstract, on the H200 Union8 measurements).  The pages do not name
the FP8 variant; the reading taken is OCP e4m3fn, the format gfx950 supports
natively (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
field 0 is subnormal; the all-ones pattern S.1111.111 is NaN; there is no
infinity; the largest finite magnitude is 448).
"""
from __future__ import annotations

import numpy as np


def e4m3fn_value(code: int) -> float:
    """Value of one e4m3fn byte, written out from the format's definition."""
    code &= 0xFF
    sign = -1.0 if (code >> 7) else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """uint8 codes (any shape) -> fp64 values."""
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> fp64 values (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):        # NaN payloads stay NaN
        return b.view(np.float32).astype(np.float64)
