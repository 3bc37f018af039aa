"""GPU parity on ragged spatial partitions (DraftAttention2 Sec. 3.3: a ragged
2D partition of each frame with balanced token counts, minimum perimeter, the
minimum number of blocks and under one block of padding per frame; App. C.1:
padding excluded from n_a and from attention).

Frames whose sides are not multiples of 8, covering every kernel variant:
20 x 28 (regions of 62..63 tokens: at most 4 padding slots), 17 x 31 (58..59:
at most 16), 84 x 48 (the latent of a 1344 x 768 video: full regions of
ragged shape) and 12 x 16 (bands of 4 and 8 rows).  Bit-exact: the quantized
operands (padding slots zero), the pooled descriptors over the valid tokens,
draft keys, tier maps and schedules.  Attention against the oracle (rel-L2
<= 1e-3, every element within 5e-3) for the
plan's map and for tier families with every phase, in contiguous and
[B,N,H,d] strided storage, and with a text prefix."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import gpu_common as G
from video_diffusion_dit_frame_amd import synth

pytestmark = pytest.mark.gpu

# (B, H, F, Hv, Wv, d, seed, outliers, hi, lo)
R20x28 = (1, 2, 2, 20, 28, 64, 41, True, 1500, 3500)
R17x31 = (1, 2, 2, 17, 31, 128, 42, True, 1500, 3500)
R84x48 = (1, 1, 2, 84, 48, 128, 43, True, 1000, 3000)
R12x16 = (2, 1, 3, 12, 16, 64, 44, False, 2500, 2500)
CASES = [R20x28, R17x31, R84x48, R12x16]
IDS = ["20x28", "17x31", "84x48", "12x16"]


def _case(c):
    B, H, F, Hv, Wv, d, seed, outl, hi, lo = c
    q, k, v = G.inputs(B, H, F, Hv, Wv, d, seed, outl)
    return dict(B=B, H=H, F=F, Hv=Hv, Wv=Wv, d=d, hi=hi, lo=lo, q=q, k=k, v=v)


def _sample(R):
    """Query regions checked on the larger layouts (all on small ones)."""
    return None if R <= 60 else np.array(sorted({0, 1, R // 3, R // 2, R - 2, R - 1}), np.int32)


def _check_rows(c, o, tier, what, strided=False):
    F, Hv, Wv = c["F"], c["Hv"], c["Wv"]
    R = tier.shape[-1]
    qb = _sample(R)
    ref, amb = O.attention(c["q"], c["k"], c["v"], tier, F, Hv, Wv, qblocks=qb, amb=True)
    if qb is not None:
        perm = O.layout(F, Hv, Wv)
        pos = (qb[:, None] * 64 + np.arange(64)).ravel()
        tok = perm[pos]
        keep = tok >= 0
        got = np.zeros(ref.shape, np.float64).reshape(o.shape[0], o.shape[1], -1, o.shape[-1])
        got[:, :, keep] = o[:, :, tok[keep]]
        return G.check_close(got.reshape(ref.shape), ref, what, amb=amb)
    return G.check_close(o, ref, what, amb=amb)


@pytest.fixture(scope="module", params=CASES, ids=IDS)
def case(request):
    c = _case(request.param)
    P, qd, kd = G.run_plan(c["q"], c["k"], c["F"], c["Hv"], c["Wv"], c["hi"], c["lo"])
    o = G.run_attention(P, qd, kd, c["v"])
    c.update(P=P, qd=qd, kd=kd, o=o.cpu().numpy())
    c["oracle_plan"] = O.plan(c["q"], c["k"], c["F"], c["Hv"], c["Wv"], c["hi"], c["lo"],
                              descriptors=True)
    return c


def test_layout_is_ragged(case):
    P = case["P"]
    L = P.layout
    tok, nv = O.partition(case["Hv"], case["Wv"])
    assert L.Rf == tok.shape[0] and np.array_equal(L.slots(), tok)


def test_operands_bit_exact(case):
    P, F, Hv, Wv = case["P"], case["F"], case["Hv"], case["Wv"]
    for name, x in (("Q", case["q"]), ("K", case["k"])):
        o = O.quant_qk(x, F, Hv, Wv)
        assert np.array_equal(G.host(P.debug(name + "_I8"), np.uint8).reshape(o["c8"].shape), o["c8"]), name
        assert np.array_equal(G.host(P.debug(name + "_I8_SCALE"), np.float32).reshape(o["s8"].shape), o["s8"]), name
        assert np.array_equal(G.host(P.debug(name + "_MX"), np.uint8).reshape(o["c4"].shape), o["c4"]), name
        assert np.array_equal(G.host(P.debug(name + "_MX_SCALE"), np.uint8).reshape(o["e4"].shape), o["e4"]), name
    o = O.quant_v(case["v"], F, Hv, Wv)
    assert np.array_equal(G.host(P.debug("V_FP8"), np.uint8).reshape(o["c8"].shape), o["c8"])
    assert np.array_equal(G.host(P.debug("V_FP8_SCALE"), np.float32).reshape(o["s8"].shape), o["s8"])
    assert np.array_equal(G.host(P.debug("V_MX"), np.uint8).reshape(o["c4"].shape), o["c4"])
    assert np.array_equal(G.host(P.debug("V_MX_SCALE"), np.uint8).reshape(o["e4"].shape), o["e4"])


def test_plan_bit_exact(case):
    P, op = case["P"], case["oracle_plan"]
    for name, key, dt in (("Q_AVG", "qavg", np.float64), ("K_AVG", "kavg", np.float64),
                          ("Q_MAX", "qmax", np.float32), ("K_MAX", "kmax", np.float32)):
        got = G.host(P.debug(name), dt).reshape(op[key].shape)
        assert np.array_equal(got, op[key]), name
    keys = G.host(P.debug("KEYS"), np.uint32).reshape(op["keys"].shape)
    assert np.array_equal(keys, op["keys"])
    tier = P.tier_map().cpu().numpy()
    assert np.array_equal(tier, op["tier"])
    sch = G.host(P.debug("SCHEDULE"), np.int32).reshape(op["tier"].shape[:3] + (-1,))
    assert np.array_equal(sch, G.schedule_from_tier(op["tier"]))


def test_attention_plan_map(case):
    rl, ma = _check_rows(case, case["o"], case["oracle_plan"]["tier"], "plan map")
    print("%dx%d plan map: rel_l2 %.3e max_abs %.3e" % (case["Hv"], case["Wv"], rl, ma))


def _families(B, H, R, seed):
    rng = np.random.default_rng(seed)
    t = rng.choice(np.array([0, 4, 8, 16], np.uint8), size=(B, H, R, R), p=[0.4, 0.2, 0.2, 0.2])
    t[:, :, ::3, :] = 0
    return {
        "mixed16": rng.choice(np.array([0, 4, 8, 16], np.uint8), size=(B, H, R, R)),
        "quantized": rng.choice(np.array([0, 4, 8], np.uint8), size=(B, H, R, R)),
        "all16": np.full((B, H, R, R), 16, np.uint8),
        "empty_rows": t,
    }


@pytest.mark.parametrize("c", CASES, ids=IDS)
@pytest.mark.parametrize("family", ["mixed16", "quantized", "all16", "empty_rows"])
def test_attention_tier_families(c, family):
    c = _case(c)
    R = O.regions(c["F"], c["Hv"], c["Wv"])
    tier = _families(c["B"], c["H"], R, 7)[family]
    from video_diffusion_dit_frame_amd import da2

    qd, kd = G.dev(c["q"]), G.dev(c["k"])
    L = da2.Layout.for_tensor(qd, c["F"], c["Hv"], c["Wv"])
    P = da2.Plan(L)
    P.plan_from_tier_map(qd, kd, torch.from_numpy(tier).cuda())
    o = G.run_attention(P, qd, kd, c["v"]).cpu().numpy()
    _check_rows(c, o, tier, family)


def test_strided_storage_matches_contiguous():
    c = _case(R17x31)
    P, qd, kd = G.run_plan(c["q"], c["k"], c["F"], c["Hv"], c["Wv"], c["hi"], c["lo"])
    o = G.run_attention(P, qd, kd, c["v"]).cpu()
    P2, qd2, kd2 = G.run_plan(c["q"], c["k"], c["F"], c["Hv"], c["Wv"], c["hi"], c["lo"], layout_bnhd=True)
    o2 = G.run_attention(P2, qd2, kd2, c["v"], layout_bnhd=True).cpu()
    assert torch.equal(o, o2)


def test_prefix_on_ragged_layout():
    """Text prefix with a ragged video partition: the prefix rows' dense video
    tiles and the video rows' 16-bit tiles both mask padding slots."""
    from tests.test_gpu_prefix import run_prefixed

    c = _case(R20x28)
    Lp = 70
    qp, kp, vp = synth.make_prefix(c["B"], c["H"], Lp, c["d"], 45)
    R = O.regions(c["F"], c["Hv"], c["Wv"])
    tier = _families(c["B"], c["H"], R, 8)["mixed16"]
    o, op, _ = run_prefixed(c["q"], c["k"], c["v"], qp, kp, vp, c["F"], c["Hv"], c["Wv"], tier=tier,
                            valid=[60])
    r, rp, amb = O.attention_pfx(c["q"], c["k"], c["v"], tier, c["F"], c["Hv"], c["Wv"],
                                 qp, kp, vp, [60], amb=True)
    G.check_close(o, r, "ragged + prefix video rows", amb=amb)
    G.check_close(op, rp, "ragged + prefix prefix rows")
