"""The two-part e4m3fn split of a bf16 Q row that the attention kernel feeds to the FP8 matrix
cores, checked on the CPU against the accuracy the library header states: after the row is scaled
by a power of two so that its largest magnitude lies in [128, 256), hi = e4m3(x) and
lo = e4m3(x - hi) (round to nearest even) give hi + lo == x for every bf16 x with |x| >= 2^-2, and
|hi + lo - x| <= 2^-10 below.  Every positive bf16 value under 256 is tried (the split is odd in x).
torch's float8_e4m3fn conversion rounds to nearest even, as the gfx950 conversion does in its
default mode."""
import numpy as np
import torch


def _all_bf16_below(limit: float) -> torch.Tensor:
    bits = torch.arange(1, 0x7F80, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    x = bits.float()
    return x[x < limit]


def _split(x: torch.Tensor):
    hi = x.to(torch.float8_e4m3fn).float()
    lo = (x - hi).to(torch.float8_e4m3fn).float()
    return hi, lo


def test_split_is_exact_from_a_quarter_up():
    x = _all_bf16_below(256.0)
    hi, lo = _split(x)
    big = x >= 0.25
    assert big.sum() > 1000
    assert torch.equal((hi + lo)[big], x[big])


def test_split_residual_below_a_quarter():
    x = _all_bf16_below(0.25)
    hi, lo = _split(x)
    err = (hi + lo - x).abs()
    assert err.max().item() <= 2.0 ** -10
    # relative to a row whose largest magnitude is at least 128 after scaling: <= 2^-17
    assert err.max().item() / 128.0 <= 2.0 ** -17


def test_split_on_scaled_random_rows():
    g = np.random.default_rng(5)
    rows = torch.from_numpy(g.standard_normal((256, 128)).astype(np.float32)).to(torch.bfloat16).float()
    amax = rows.abs().amax(dim=1, keepdim=True)
    e = 8 - torch.frexp(amax).exponent              # amax * 2^e in [128, 256)
    x = torch.ldexp(rows, e.float())
    assert torch.all((x.abs().amax(dim=1) >= 128) & (x.abs().amax(dim=1) < 256))
    hi, lo = _split(x)
    err = (hi + lo - x).abs()
    assert torch.all(err[x.abs() >= 0.25] == 0)
    assert (err / x.abs().amax(dim=1, keepdim=True)).max().item() <= 2.0 ** -17
