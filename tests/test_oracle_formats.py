"""Pins of the oracle's number formats (CPU).

FP8 E4M3 ("fn": no infinities, 0x7f/0xff NaN, max 448) and MX E2M1 with
E8M0 block exponents, both rounding to nearest with ties to even and
saturating to the largest finite magnitude.  Pinned against torch's
float8_e4m3fn decoding (a library routine) and a brute-force nearest search
over the decoded value table (ties broken towards the even code).
"""
import math

import numpy as np
import pytest
import torch

from video_diffusion_dit_frame_amd.synth import bf16_bits_to_f32


def e4m3_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # OCP MX v1.0 E2M1 table


def brute_nearest(x, table_pos):
    """Nearest entry of a sorted magnitude table, ties to the even code,
    saturating; sign copied from x.  Returns integer codes."""
    a = np.abs(x)[:, None]
    d = np.abs(a - table_pos[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.arange(len(table_pos))[None, :]
    # prefer even codes among ties
    score = np.where(cand, (codes % 2) * 1000 + codes, 10**9)
    c = score.argmin(axis=1)
    c = np.where(np.abs(x) >= table_pos[-1], len(table_pos) - 1, c)
    return c


def all_bf16_finite():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(h)
    return f[np.isfinite(f)].astype(np.float64)


def test_e4m3_decode_matches_torch(orc):
    tab = e4m3_table()
    for c in range(256):
        v = orc.e4m3_value(c)
        if math.isnan(tab[c]):
            assert math.isnan(v), c
        else:
            assert v == tab[c], (c, v, tab[c])


def test_e2m1_decode_table(orc):
    for c in range(16):
        want = E2M1_POS[c & 7] * (-1.0 if c & 8 else 1.0)
        assert orc.e2m1_value(c) == want


def test_e4m3_roundtrip_all_codes(orc):
    for c in range(256):
        v = orc.e4m3_value(c)
        if math.isnan(v):
            continue
        assert orc.e4m3_encode(v) == c


def test_e2m1_roundtrip_all_codes(orc):
    for c in range(16):
        assert orc.e2m1_encode(orc.e2m1_value(c)) == c


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -7, 3.0, 448.0 / 7.5])
def test_e4m3_encode_exhaustive_bf16(orc, scale):
    x = all_bf16_finite() * scale
    x = x[np.abs(x) < 1e6]
    got = orc.e4m3_encode(x)
    tab = e4m3_table()[:127]  # positive finite magnitudes, codes 0..126
    want = brute_nearest(x, tab) | np.where(np.signbit(x), 0x80, 0)
    assert np.array_equal(got, want.astype(np.uint8))


def test_e4m3_encode_vs_torch_cast_in_range(orc):
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1e-2, 20000),
                        rng.normal(0, 1e-3, 5000)]).astype(np.float32)
    got = orc.e4m3_encode(x.astype(np.float64))
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_e4m3_saturates(orc):
    for v in [448.0, 449.0, 463.9, 464.0, 500.0, 1e30]:
        assert orc.e4m3_encode(v) == 0x7E
        assert orc.e4m3_encode(-v) == 0xFE
    # subnormal boundaries: 2^-10 is a tie between 0 and 2^-9 -> 0 (even)
    assert orc.e4m3_encode(2.0 ** -10) == 0
    assert orc.e4m3_encode(1.5 * 2.0 ** -9) == 2  # tie between 1 and 2 -> even code 2
    assert orc.e4m3_encode(-0.0) == 0x80


@pytest.mark.parametrize("scale", [1.0, 0.25, 5.0])
def test_e2m1_encode_exhaustive_bf16(orc, scale):
    x = all_bf16_finite() * scale
    x = x[np.abs(x) < 1e4]
    got = orc.e2m1_encode(x)
    want = brute_nearest(x, E2M1_POS) | np.where(np.signbit(x), 8, 0)
    assert np.array_equal(got, want.astype(np.uint8))


def test_e2m1_saturation_band(orc):
    # (6, 8) is what an MX block can produce above the largest element; it clips to 6
    for v in [6.0, 6.5, 7.0, 7.99]:
        assert orc.e2m1_encode(v) == 7
        assert orc.e2m1_encode(-v) == 15
    assert orc.e2m1_encode(5.0) == 6     # tie 4 / 6 -> even code (4.0 = code 6)
    assert orc.e2m1_encode(0.25) == 0    # tie 0 / 0.5 -> 0
    assert orc.e2m1_encode(0.75) == 2    # tie 0.5 / 1 -> 1.0 (code 2)


def test_mx_exponent_closed_form(orc):
    rng = np.random.default_rng(1)
    vals = np.concatenate([2.0 ** np.arange(-140, 128, dtype=np.float64),
                           rng.lognormal(0, 20, 2000)])
    for a in vals:
        if not np.isfinite(a) or a == 0:
            continue
        m, e = math.frexp(a)
        want = max(-127, min(127, (e - 1) - 2))
        assert orc.mx_exponent(a) == want, a
    assert orc.mx_exponent(0.0) == -127
    # the block max lands in [4, 8) after scaling unless clamped
    for a in [1.0, 1.999, 3.0, 1e-3, 7e5]:
        E = orc.mx_exponent(a)
        assert 4.0 <= a * 2.0 ** -E < 8.0


def test_weight_mx_exponent_is_smallest_unclipped(orc):
    """Attention-weight blocks: the smallest X with amax 2^-X <= 6, found by
    brute force; amax = 1 (a block holding the running maximum) and values
    just below it share X = -2, so rounding below 1 never moves the scale."""
    rng = np.random.default_rng(2)
    vals = np.concatenate([2.0 ** np.arange(-120, 1, dtype=np.float64), 0.75 * 2.0 ** np.arange(-100, 1.0),
                           rng.uniform(0, 1, 3000), np.exp(-rng.uniform(0, 80, 2000))])
    for a in vals:
        X = -127
        while a * 2.0 ** -X > 6.0:
            X += 1
        assert orc.mx_exponent_w(a) == X, a
        if X > -127:
            assert a * 2.0 ** -(X - 1) > 6.0
    assert orc.mx_exponent_w(0.0) == -127
    assert orc.mx_exponent_w(1.0) == -2 and orc.mx_exponent_w(1.0 - 1e-7) == -2
    assert orc.mx_exponent_w(0.75) == -3 and orc.mx_exponent_w(0.75 + 1e-9) == -2


def test_bf16_round_matches_torch_cast(orc):
    """The oracle's bfloat16 rounding of binary32 values equals PyTorch's
    float32 -> bfloat16 conversion (nearest, ties to even): random bit
    patterns across the normal and subnormal range, exact midpoints, and
    values just beside them."""
    rng = np.random.default_rng(4)
    u = rng.integers(0, 0x7F800000, size=20000, dtype=np.uint32)           # finite positives
    mid = (rng.integers(0, 0x7F7F, size=2000, dtype=np.uint32) << 16) | 0x8000  # exact ties
    near = np.concatenate([mid - 1, mid + 1])
    bits = np.concatenate([u, mid, near, np.array([1, 0x00400000, 0x007FFFFF, 0x00800000], np.uint32)])
    bits = np.concatenate([bits, bits | 0x80000000])
    x = bits.view(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.bf16_round(float(v)) for v in x])
    assert np.array_equal(got, ref)
