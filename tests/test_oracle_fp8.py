"""Pins of the oracle's exact decoders (CPU only)."""
import math
import os

import numpy as np
import torch

from oracle.fp8 import E4M3FN_TABLE, decode_bf16, decode_e4m3fn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_points.txt")


def test_e4m3fn_all_codes_match_torch():
    # independent route: torch's own float8_e4m3fn -> float32 conversion
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().double().numpy()
    ours = decode_e4m3fn(np.arange(256, dtype=np.uint8))
    nan_ref, nan_ours = np.isnan(ref), np.isnan(ours)
    assert np.array_equal(nan_ref, nan_ours)
    assert np.array_equal(ref[~nan_ref], ours[~nan_ours])
    assert np.array_equal(np.signbit(ref[~nan_ref]), np.signbit(ours[~nan_ours]))


def test_e4m3fn_spec_points():
    n = 0
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, value = line.split()[:2]
        want = float(value)
        got = E4M3FN_TABLE[int(code, 16)]
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code
        n += 1
    assert n >= 12


def test_e4m3fn_structure():
    finite = E4M3FN_TABLE[~np.isnan(E4M3FN_TABLE)]
    assert np.isnan(E4M3FN_TABLE).sum() == 2
    assert finite.max() == 448.0 and finite.min() == -448.0
    pos = E4M3FN_TABLE[:127]
    assert np.all(np.diff(pos) > 0)                       # monotone in the code
    assert np.array_equal(E4M3FN_TABLE[128:255], -E4M3FN_TABLE[:127])


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=100000, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    ours = decode_bf16(bits)
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(t[~nan], ours[~nan])
