"""Pins of the oracle's operand quantization (CPU).

Q/K: INT8 with one fp32 step per 64-token block (amax/127; the uniform
nearest-integer quantizer of DraftAttention2 App. B.2, used for Q K^T by the
8-bit path of App. C.1), MXFP4 per token and 32 channels.  V: FP8 with one
scale per channel over all tokens, MXFP4 per channel and 32 consecutive keys
of a block.  Every rule is recomputed here with numpy/torch (independent of
the oracle's C code): fp32 division and product via numpy float32, codes via
numpy's round-half-even, torch's float8 cast or a brute-force nearest search,
exponents via frexp.
"""
import numpy as np
import pytest
import torch

from video_diffusion_dit_frame_amd import synth
from video_diffusion_dit_frame_amd.synth import bf16_bits_to_f32
from tests.test_oracle_formats import E2M1_POS, brute_nearest


def _inputs(F=2, Hv=16, Wv=16, d=64, B=1, H=2, seed=21, outliers=True):
    return synth.make_qkv(B, H, F, Hv, Wv, d, seed, outliers)


def torch_e4m3(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def int8_codes(prod32):
    """Nearest integer, ties to even, as two's complement bytes."""
    r = np.clip(np.rint(prod32.astype(np.float64)), -127, 127)
    return r.astype(np.int8).view(np.uint8)


def mx_exp(amax):
    m, e = np.frexp(amax)
    E = np.clip(e.astype(np.int64) - 1 - 2, -127, 127)
    return np.where(amax == 0, -127, E)


def e2m1_brute(x):
    return (brute_nearest(x.reshape(-1), E2M1_POS) | np.where(np.signbit(x.reshape(-1)), 8, 0)).reshape(x.shape)


def test_quant_qk_rules(orc):
    F, Hv, Wv = 2, 16, 16
    q, _, _ = _inputs(F, Hv, Wv)
    o = orc.quant_qk(q, F, Hv, Wv)
    perm = orc.layout(F, Hv, Wv)
    X = bf16_bits_to_f32(q)[:, :, perm, :]  # reordered, fp32 exact
    B, H, N, d = X.shape
    G = X.reshape(B, H, N // 64, 64 * d)
    amax = np.abs(G).max(axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    inv = (np.float32(127.0) / amax).astype(np.float32)
    assert np.array_equal(o["s8"], s)
    prod = (G * inv[..., None]).astype(np.float32)
    assert np.array_equal(o["c8"].reshape(G.shape), int8_codes(prod).reshape(G.shape))
    # the extreme codes are reached: the block's largest |x| maps to +-127
    c = o["c8"].view(np.int8).reshape(G.shape)
    assert (np.abs(c).max(axis=-1) == 127).all()
    # MX: per token, 32 channels
    T = X.reshape(B, H, N, d // 32, 32).astype(np.float64)
    E = mx_exp(np.abs(T).max(axis=-1))
    assert np.array_equal(o["e4"].astype(np.int64) - 127, E)
    scaled = T * np.exp2(-E)[..., None]
    assert np.array_equal(o["c4"].reshape(T.shape), e2m1_brute(scaled).astype(np.uint8))


def test_quant_v_rules(orc):
    F, Hv, Wv = 2, 8, 24
    _, _, v = _inputs(F, Hv, Wv)
    o = orc.quant_v(v, F, Hv, Wv)
    perm = orc.layout(F, Hv, Wv)
    X = bf16_bits_to_f32(v)
    B, H, N, d = X.shape
    amax = np.abs(X).max(axis=2)  # per channel over all tokens
    assert np.array_equal(o["s8"], (amax / np.float32(448.0)).astype(np.float32))
    inv = (np.float32(448.0) / amax).astype(np.float32)
    Xr = X[:, :, perm, :]
    prod = (Xr * inv[:, :, None, :]).astype(np.float32)
    assert np.array_equal(o["c8"], torch_e4m3(prod).reshape(o["c8"].shape))
    # MX along keys: [B,H,R,2,32,d]
    T = Xr.reshape(B, H, N // 64, 2, 32, d).astype(np.float64)
    E = mx_exp(np.abs(T).max(axis=4))
    assert np.array_equal(o["e4"].astype(np.int64) - 127, E)
    scaled = T * np.exp2(-E)[:, :, :, :, None, :]
    assert np.array_equal(o["c4"].reshape(T.shape), e2m1_brute(scaled).astype(np.uint8))


def test_quant_zero_block_and_power_of_two(orc):
    F, Hv, Wv, d = 1, 8, 16, 64
    X = np.zeros((1, 1, F * Hv * Wv, d), np.uint16)
    # block 1 (tokens of the right 8x8 cell): every value 2.0 exactly (bf16 0x4000)
    perm = orc.layout(F, Hv, Wv)
    X[0, 0, perm[64:], :] = 0x4000
    o = orc.quant_qk(X, F, Hv, Wv)
    assert o["s8"][0, 0, 0] == 1.0 and (o["c8"][0, 0, :64] == 0).all()
    assert o["s8"][0, 0, 1] == np.float32(2.0) / np.float32(127.0)
    assert (o["c8"][0, 0, 64:] == 127).all()  # x * 127/amax = 127 exactly
    assert (o["e4"][0, 0, :64] == 0).all() and (o["c4"][0, 0, :64] == 0).all()
    # amax = 2 -> E = 1 - 2 = -1, 2 * 2^1 = 4 -> code 6
    assert (o["e4"][0, 0, 64:] == 126).all() and (o["c4"][0, 0, 64:] == 6).all()


def test_quant_saturating_group(orc):
    """amax = 7 -> E = 0; 7 lies in the (6, 8) band and clips to 6 (code 7)."""
    F, Hv, Wv, d = 1, 8, 8, 32
    X = np.full((1, 1, 64, d), 0x3F80, np.uint16)  # 1.0
    X[0, 0, 5, 3] = 0x40E0  # 7.0
    o = orc.quant_qk(X, F, Hv, Wv)
    perm = orc.layout(F, Hv, Wv)
    pos = int(np.where(perm == 5)[0][0])
    assert o["e4"][0, 0, pos, 0] == 127
    assert o["c4"][0, 0, pos, 3] == 7
    assert o["c4"][0, 0, pos, 0] == 2  # 1.0


@pytest.mark.parametrize("which", ["qk", "v"])
def test_quant_error_within_half_step(orc, which):
    F, Hv, Wv = 1, 16, 16
    q, _, v = _inputs(F, Hv, Wv)
    X = q if which == "qk" else v
    o = orc.quant_qk(X, F, Hv, Wv) if which == "qk" else orc.quant_v(X, F, Hv, Wv)
    perm = orc.layout(F, Hv, Wv)
    Xr = bf16_bits_to_f32(X)[:, :, perm, :].astype(np.float64)
    B, H, N, d = Xr.shape
    val8 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    if which == "qk":
        # uniform quantizer: every value within half a step (App. B.2), up to
        # the fp32 rounding of the step and of x * 127/amax
        s = np.repeat(o["s8"], 64, axis=2)[..., None].astype(np.float64)
        deq = o["c8"].view(np.int8).astype(np.float64) * s
        assert (np.abs(deq - Xr) <= s * (0.5 + 2.0 ** -16)).all()
        return
    s = o["s8"][:, :, None, :].astype(np.float64)
    deq = val8[o["c8"]] * s
    # relative spacing of e4m3 is at most 2^-3; subnormal step 2^-9 * s
    err = np.abs(deq - Xr)
    assert (err <= np.maximum(np.abs(Xr) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 1e-12)).all()
