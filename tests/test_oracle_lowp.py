"""Pins of the low-precision variant's fp64 model (CPU only): e4m3fn rounding
against torch's converter and hand-worked ties, the variant equal to the exact
attention when every rounding is exact, hand-worked two-key rows, and a
rigorous per-element bound on its distance from the exact attention."""
import math

import numpy as np
import pytest
import torch

from oracle.attention import Problem, attention_query
from oracle.fp8 import E4M3FN_TABLE, decode_bf16, decode_e4m3fn
from oracle.lowp import (TAU, attention_query_lowp, e4m3_rne, quantize_q_row, row_exponent,
                         split_scale)
from tests.oracle_helpers import tiny_problem

LOG2E = math.log2(math.e)


def _pb(inp):
    return Problem(inp["q_bits"], inp["k_codes"], inp["v_codes"], inp["scales"], inp["sel_pages"])


def _bf16_bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _e4m3_codes(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


# ---------------------------------------------------------------- rounding

def test_e4m3_rne_matches_torch():
    # independent route: torch's float32 -> float8_e4m3fn conversion (round to nearest even)
    vals = E4M3FN_TABLE[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(3)
    x = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        rng.uniform(0, 448, 50000), 2.0 ** rng.uniform(-14, 8.7, 50000)])
    x = x.astype(np.float32).astype(np.float64)
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
    got = e4m3_rne(x)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got[got == 0]), np.signbit(ref[ref == 0]))


@pytest.mark.parametrize("x,want", [
    (1.0625, 1.0),        # halfway between 0x38 (1.0) and 0x39 (1.125): even code 0x38
    (1.1875, 1.25),       # halfway between 0x39 and 0x3A (1.25): even code 0x3A
    (2.0 ** -0.5, 0.6875),  # 0.7071 lies below the midpoint 0.71875 of 0x33 (0.6875) and 0x34
    (1.2, 1.25),          # above the midpoint 1.1875
    (2.0 ** -0.5 * 1.2, 0.875),  # 0.8485 lies above the midpoint 0.84375 of 0x35 and 0x36
    (2.0 ** -10, 0.0),    # halfway between 0 and the smallest subnormal 2^-9: even code 0x00
    (3 * 2.0 ** -10, 2.0 ** -8),  # halfway between 0x01 (2^-9) and 0x02 (2^-8): code 0x02
    (248.0, 256.0),       # halfway between 0x77 (240) and 0x78 (256): code 0x78
    (-38.5, -40.0),       # between 36 and 40, above the midpoint 38
])
def test_e4m3_rne_by_hand(x, want):
    assert e4m3_rne(np.array([x]))[0] == want


def test_e4m3_rne_rejects_out_of_range():
    with pytest.raises(ValueError):
        e4m3_rne(np.array([449.0]))


def test_q_row_scaling_by_hand():
    # max |q| = 1 = (1/2) 2^1, so e = 7 and the row is scaled by 128 into [128, 256)
    q = decode_bf16(_bf16_bits([1.0, 0.3, -0.00390625, 0.0]))   # bf16(0.3) = 0.30078125
    assert row_exponent(q) == 7
    # 0.30078125 * 128 = 38.5 -> 40; -2^-8 * 128 = -0.5 exactly
    np.testing.assert_array_equal(quantize_q_row(q), [1.0, 40 / 128, -0.00390625, 0.0])
    assert row_exponent(np.zeros(4)) == 0
    assert row_exponent(np.array([3.0])) == 6                   # 3 * 64 = 192


def test_split_scale():
    for v in [1.0, 1.25, 0.3, 7.5, 2.0 ** 40 * 1.7, 2.0 ** -30]:
        phi, k = split_scale(v)
        assert 1.0 <= phi < 2.0 and phi * 2.0 ** k == v and k == math.floor(math.log2(v))


# --------------------------------------------------- exact roundings: = exact attention

def _exact_case(seed):
    """Inputs on which every rounding of the variant is exact, so that it must equal the exact
    attention: q rows with two entries +-1 (the row times 1 or 2), K codes in {0, +-1}, a
    k_scale that makes the log2 scores integers, and V scales phi 2^k with phi in {1, 1.5}.
    A score then lies at most 8 below its row's reference and at most tau above it, where
    2^(s - m) phi is an e4m3fn value (down to 3 * 2^-9).  Rows of tokens 48..63 put 2 on the
    first four dimensions, which only the last page's keys use (score 8 +- 2 there, +-2
    elsewhere): those rows move their reference on the last page."""
    rng = np.random.default_rng(seed)
    T, Hq, Hkv, D, P = 64, 4, 2, 32, 8
    N, S = T // P, 5
    q = np.zeros((T, Hq, D), dtype=np.float32)
    for t in range(T):
        for hq in range(Hq):
            idx = 4 + rng.choice(D - 4, size=2, replace=False)
            q[t, hq, idx] = rng.choice([-1.0, 1.0], size=2) * (1.0 if t >= 48 else rng.choice([1.0, 2.0]))
            if t >= 48:
                q[t, hq, :4] = 2.0
    k = rng.choice([-1.0, 0.0, 1.0], size=(N, Hkv, P, D), p=[0.1, 0.8, 0.1]).astype(np.float32)
    k[:, :, :, :4] = 0.0
    k[-1, :, :, :4] = 1.0
    v = rng.standard_normal((N, Hkv, P, D)).astype(np.float32)
    scales = np.empty((2, N, Hkv), dtype=np.float64)
    scales[0] = math.sqrt(D) / LOG2E                 # s_j = <q, k> in log2 units
    scales[1] = rng.choice([1.0, 1.5], size=(N, Hkv)) * 2.0 ** rng.integers(-4, 5, size=(N, Hkv))
    sel = np.full((Hkv, T, S), -1, dtype=np.int32)
    for h in range(Hkv):
        for t in range(T):
            p = t // P
            cand = list(rng.permutation(p + 1)[: min(S - 2, p + 1)])
            if t >= 56 and (N - 1) not in cand:
                cand.append(N - 1)
            row = cand + [int(cand[0])]                # a repeated page
            sel[h, t, : len(row)] = row
    return {"q_bits": _bf16_bits(q), "k_codes": _e4m3_codes(k), "v_codes": _e4m3_codes(v),
            "scales": scales.astype(np.float32), "sel_pages": sel}


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_lowp_equals_exact_when_rounding_is_exact(seed):
    inp = _exact_case(seed)
    pb = _pb(inp)
    # k_scale is stored in fp32, so a log2 score is n (1 + d) with |n| <= 16, |d| <= 2^-24: the
    # exact attention sees 2^(n d) - 1 <= 16 2^-24 ln 2 of relative weight error that the
    # variant's rounding removes, i.e. at most 2 * 6.7e-7 * max |V| on the output
    vmax = max(float(np.abs(pb.v_hat(h)).max()) for h in range(pb.H_kv))
    tol = 2 * 16 * 2.0 ** -24 * math.log(2) * vmax / (1 - 1e-5)
    c = LOG2E / math.sqrt(pb.D)
    moved = 0
    for h in range(pb.H_kv):
        kc = decode_e4m3fn(pb.k_codes[:, h])
        for t in range(pb.T):
            a = attention_query_lowp(pb, h, t)
            b = attention_query(pb, h, t)
            np.testing.assert_allclose(a, b, rtol=0, atol=tol, err_msg=f"h={h} t={t}")
            # a row whose last page's largest score passes its first page's by more than tau
            # has moved its reference at least once
            sup = [int(u) for u in pb.support(h, t) if int(u) * pb.P <= t]
            if len(sup) > 1:
                for r in range(pb.G):
                    q = pb.q_rows(t, h)[r]
                    mx = [float(max(kc[u, j] @ q for j in range(pb.P) if u * pb.P + j <= t))
                          * pb.scales[0, u, h] * c for u in (sup[0], sup[-1])]
                    moved += int(mx[1] > mx[0] + TAU)
    assert moved > 0


def test_lowp_single_visible_key_is_that_value():
    # token 0 sees exactly key 0 of page 0: weight 1 whatever the rounding
    inp = tiny_problem(T=32, Hq=4, Hkv=2, D=16, P=16, S=2, seed=4)
    pb = _pb(inp)
    for h in range(pb.H_kv):
        want = decode_e4m3fn(pb.v_codes[0, h, 0]) * pb.scales[1, 0, h]
        got = attention_query_lowp(pb, h, 0)
        for r in range(pb.G):
            np.testing.assert_allclose(got[r], want, rtol=1e-15, atol=0)


@pytest.mark.parametrize("v_scale,p1,p2", [
    (1.0, 1.0, 0.6875),    # p = rne(2^0) and rne(2^-0.5) = 0.6875
    (1.2, 1.25, 0.875),    # phi = 1.2: rne(1.2) = 1.25, rne(0.8485) = 0.875
])
def test_lowp_two_keys_by_hand(v_scale, p1, p2):
    # one query at token 1 on page 0 (P = 2) sees keys 0 and 1, with log2 scores 1 and 0.5
    D = 16
    q = np.zeros((2, 1, D), dtype=np.float32)
    q[:, 0, 0] = 1.0
    k = np.zeros((1, 1, 2, D), dtype=np.float32)
    k[0, 0, 0, 0], k[0, 0, 1, 0] = 2.0, 1.0
    v = np.zeros((1, 1, 2, D), dtype=np.float32)
    v[0, 0, 0, :2], v[0, 0, 1, :2] = [1.0, -2.0], [3.0, 0.5]
    scales = np.array([[[0.5 * math.sqrt(D) / LOG2E]], [[v_scale]]], dtype=np.float64)
    sel = np.array([[[0], [0]]], dtype=np.int32)
    inp = {"q_bits": _bf16_bits(q), "k_codes": _e4m3_codes(k), "v_codes": _e4m3_codes(v),
           "scales": scales.astype(np.float32), "sel_pages": sel}
    pb = _pb(inp)
    vs = float(np.float32(v_scale))
    want = vs * (p1 * np.array([1.0, -2.0]) + p2 * np.array([3.0, 0.5])) / (p1 + p2)
    got = attention_query_lowp(pb, 0, 1)[0, :2]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)
    exact = attention_query(pb, 0, 1)[0, :2]
    assert np.abs(got - exact).max() > 1e-3          # the variant does differ from the method


# --------------------------------------------------- bound on the distance to the exact result

def _row_bound(pb, h, t, r):
    """Per-element bound on |O_lowp - O_exact| of one row from the rounding model: the weight of
    key j is multiplied by (1 + eta_j) with |eta_j| <= E_j = 2^Delta_j (1 + rho_j) - 1, Delta_j
    bounding the score change from rounding q and rho_j the relative rounding error of p_j."""
    sup = pb.support(h, t)
    keys = [(int(u), j) for u in sup for j in range(pb.P) if int(u) * pb.P + j <= t]
    if not keys:
        return np.zeros(pb.D)
    q = pb.q_rows(t, h)[r]
    qt = quantize_q_row(q)
    c = LOG2E / math.sqrt(pb.D)
    kc = np.stack([decode_e4m3fn(pb.k_codes[u, h, j]) for u, j in keys])
    ks = np.array([pb.scales[0, u, h] for u, _ in keys])
    vv = np.stack([decode_e4m3fn(pb.v_codes[u, h, j]) * pb.scales[1, u, h] for u, j in keys])
    s = (kc @ q) * ks * c                                  # exact log2 scores
    delta = (np.abs(kc) @ np.abs(qt - q)) * ks * c
    w = np.exp2(s - s.max())
    w /= w.sum()
    o = w @ vv
    # p_j = rne(x_j) with x_j = 2^(s~_j - m) phi, phi >= 1 and the reference m a page maximum
    # of the rounded-q scores, so m <= max s~ <= max s + max delta and
    # x_j >= 2^(s_j - delta_j - max s - max delta); the rounding error is at most 2^-4 x_j
    # (normal range) and 2^-10 absolute (subnormal range)
    x_lo = np.exp2(s - delta - s.max() - delta.max())
    rho = np.maximum(2.0 ** -4, 2.0 ** -10 / x_lo)
    E = np.exp2(delta) * (1 + rho) - 1
    # O_lowp - O = sum_j w_j eta_j (v_j - O) / sum_j w_j (1 + eta_j), with eta_j >= -1
    den = 1 - float(w @ np.minimum(E, 1.0))
    assert den > 0
    return (w * E) @ np.abs(vv - o) / den


@pytest.mark.parametrize("seed,q_scale", [(0, 1.0), (1, 1.0), (2, 4.0)])
def test_lowp_within_rounding_bound_of_exact(seed, q_scale):
    inp = tiny_problem(T=64, Hq=4, Hkv=2, D=16, P=8, S=5, seed=seed, q_scale=q_scale)
    pb = _pb(inp)
    worst = 0.0
    for h in range(pb.H_kv):
        for t in range(pb.T):
            a = attention_query_lowp(pb, h, t)
            b = attention_query(pb, h, t)
            for r in range(pb.G):
                bound = _row_bound(pb, h, t, r)
                err = np.abs(a[r] - b[r])
                assert np.all(err <= bound + 1e-12), (h, t, r)
                worst = max(worst, float(err.max()))
    assert worst > 1e-4                              # the rounding is visible
