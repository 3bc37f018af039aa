"""GPU parity at block capacity C = 128 ([DA2] App. C.2: R_f = ceil(H_v W_v /
C); the operator study of Sec. 4 runs at C = 128).  Regions hold 128 slots:
the plan (pooling, draft map, ranking) works on regions, attention on tiles
of 64 slots, every tile of a region pair taking the pair's tier.

Frames: 16 x 16 (two full regions per frame), 24 x 40 (eight regions of 120
tokens: a partial second tile in every region), 12 x 20 (two of 120) and
48 x 80 (the Wan 720p latent: 30 full regions per frame).  Bit-exact: the
slot table against the oracle's partition, the quantized operands (INT8
steps per 64-slot tile), the pooled descriptors over 128-slot regions, the
draft keys, tier maps and the tile schedules.  Attention against the oracle
(rel-L2 <= 1e-3, every element within 5e-3 beyond its band bound) for the
plan's map, for tier families with every phase and with a text prefix; the
Wan-14B 720p layer at full size on sampled heads.  Block-mean tiles are
refused at C = 128."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import gpu_common as G
from video_diffusion_dit_frame_amd import configs, synth

pytestmark = pytest.mark.gpu

CAP = 128
TPR = CAP // 64

# (B, H, F, Hv, Wv, d, seed, outliers, hi, lo)
C16 = (1, 2, 2, 16, 16, 64, 61, False, 2000, 3000)
C24x40 = (2, 1, 3, 24, 40, 128, 62, True, 1500, 3500)
C12x20 = (1, 2, 2, 12, 20, 128, 63, True, 1000, 3000)
C48x80 = (1, 1, 2, 48, 80, 128, 64, True, 1000, 3000)
CASES = [C16, C24x40, C12x20, C48x80]
IDS = ["16x16", "24x40", "12x20", "48x80"]


def _case(c):
    B, H, F, Hv, Wv, d, seed, outl, hi, lo = c
    q, k, v = G.inputs(B, H, F, Hv, Wv, d, seed, outl)
    return dict(B=B, H=H, F=F, Hv=Hv, Wv=Wv, d=d, hi=hi, lo=lo, q=q, k=k, v=v)


def _sample(T):
    """Query tiles checked on the larger layouts (all on small ones)."""
    return None if T <= 60 else np.array(sorted({0, 1, T // 3, T // 2, T - 2, T - 1}), np.int32)


def _check_rows(c, o, tier, what):
    F, Hv, Wv = c["F"], c["Hv"], c["Wv"]
    T = tier.shape[-1] * TPR
    qb = _sample(T)
    ref, amb = O.attention(c["q"], c["k"], c["v"], tier, F, Hv, Wv, qblocks=qb, amb=True, cap=CAP)
    if qb is not None:
        perm = O.layout(F, Hv, Wv, cap=CAP)
        tok = perm[(qb[:, None] * 64 + np.arange(64)).ravel()]
        keep = tok >= 0
        got = np.zeros(ref.shape, np.float64).reshape(o.shape[0], o.shape[1], -1, o.shape[-1])
        got[:, :, keep] = o[:, :, tok[keep]]
        return G.check_close(got.reshape(ref.shape), ref, what, amb=amb)
    return G.check_close(o, ref, what, amb=amb)


@pytest.fixture(scope="module", params=CASES, ids=IDS)
def case(request):
    c = _case(request.param)
    P, qd, kd = G.run_plan(c["q"], c["k"], c["F"], c["Hv"], c["Wv"], c["hi"], c["lo"], cap=CAP)
    o = G.run_attention(P, qd, kd, c["v"])
    c.update(P=P, qd=qd, kd=kd, o=o.cpu().numpy())
    c["oracle_plan"] = O.plan(c["q"], c["k"], c["F"], c["Hv"], c["Wv"], c["hi"], c["lo"],
                              descriptors=True, cap=CAP)
    return c


def test_layout(case):
    L = case["P"].layout
    tok, nv = O.partition_c(case["Hv"], case["Wv"], CAP)
    assert L.R == O.regions(case["F"], case["Hv"], case["Wv"], cap=CAP) and L.Rf == tok.shape[0]
    assert L.T == TPR * L.R and np.array_equal(L.slots(), tok)


def test_operands_bit_exact(case):
    P, F, Hv, Wv = case["P"], case["F"], case["Hv"], case["Wv"]
    for name, x in (("Q", case["q"]), ("K", case["k"])):
        o = O.quant_qk(x, F, Hv, Wv, cap=CAP)
        for dbg, key, dt in (("_I8", "c8", np.uint8), ("_I8_SCALE", "s8", np.float32),
                             ("_MX", "c4", np.uint8), ("_MX_SCALE", "e4", np.uint8)):
            got = G.host(P.debug(name + dbg), dt).reshape(o[key].shape)
            assert np.array_equal(got, o[key]), name + dbg
    o = O.quant_v(case["v"], F, Hv, Wv, cap=CAP)
    for dbg, key, dt in (("V_FP8", "c8", np.uint8), ("V_FP8_SCALE", "s8", np.float32),
                         ("V_MX", "c4", np.uint8), ("V_MX_SCALE", "e4", np.uint8)):
        assert np.array_equal(G.host(P.debug(dbg), dt).reshape(o[key].shape), o[key]), dbg


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
    B, H, R, _ = op["tier"].shape
    sch = G.host(P.debug("SCHEDULE"), np.int32).reshape(B, H, R * TPR, -1)
    assert np.array_equal(sch, G.schedule_from_tier(op["tier"], TPR))


def test_attention_plan_map(case):
    rl, ma = _check_rows(case, case["o"], case["oracle_plan"]["tier"], "C=128 plan map")
    print("C=128 %dx%d plan map: rel_l2 %.3e max_abs %.3e" % (case["Hv"], case["Wv"], rl, ma))


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


def _import_plan(c, tier):
    from video_diffusion_dit_frame_amd import da2

    qd, kd = G.dev(c["q"]), G.dev(c["k"])
    L = da2.Layout.for_tensor(qd, c["F"], c["Hv"], c["Wv"], cap=CAP)
    P = da2.Plan(L)
    P.plan_from_tier_map(qd, kd, torch.from_numpy(tier).cuda())
    return P, qd, kd


@pytest.mark.parametrize("c", CASES[:3], ids=IDS[:3])
@pytest.mark.parametrize("family", ["mixed16", "quantized", "all16", "empty_rows"])
def test_attention_tier_families(c, family):
    c = _case(c)
    R = O.regions(c["F"], c["Hv"], c["Wv"], cap=CAP)
    tier = _families(c["B"], c["H"], R, 7)[family]
    P, qd, kd = _import_plan(c, tier)
    assert np.array_equal(P.tier_map().cpu().numpy(), tier)
    o = G.run_attention(P, qd, kd, c["v"]).cpu().numpy()
    _check_rows(c, o, tier, "C=128 " + family)


def test_block_means_refused():
    from video_diffusion_dit_frame_amd import da2

    c = _case(C16)
    qd, kd = G.dev(c["q"]), G.dev(c["k"])
    L = da2.Layout.for_tensor(qd, c["F"], c["Hv"], c["Wv"], cap=CAP)
    P = da2.Plan(L)
    with pytest.raises(da2.Da2Error):
        P.plan(qd, kd, 1000, 3000, skip_means=True)
    # an imported block-mean code is an unknown value: a skip
    R = L.R
    tier = np.where(np.arange(R * R).reshape(1, 1, R, R) % 2 == 0, 8, 1).astype(np.uint8)
    tier = np.repeat(np.repeat(tier, c["B"], 0), c["H"], 1)
    P.plan_from_tier_map(qd, kd, torch.from_numpy(tier).cuda())
    want = np.where(tier == 1, 0, tier).astype(np.uint8)
    assert np.array_equal(P.tier_map().cpu().numpy(), want)
    o = G.run_attention(P, qd, kd, c["v"]).cpu().numpy()
    _check_rows(c, o, want, "C=128 imported block means")


def test_prefix():
    """A text prefix at C = 128: video rows and prefix rows against the
    oracle."""
    from video_diffusion_dit_frame_amd import da2

    B, H, F, Hv, Wv, d = 2, 1, 2, 24, 40, 128
    Lp, valid = 77, np.array([77, 30], np.int32)
    q, k, v = G.inputs(B, H, F, Hv, Wv, d, 65, True)
    qp, kp, vp = synth.make_prefix(B, H, Lp, d, 66)
    R = O.regions(F, Hv, Wv, cap=CAP)
    tier = _families(B, H, R, 9)["mixed16"]
    qj, kj, vj = (G.dev(np.concatenate([a, b], axis=2)) for a, b in ((qp, q), (kp, k), (vp, v)))
    oj = torch.empty(qj.shape, dtype=torch.float32, device="cuda")
    L = da2.Layout.for_tensor(qj[:, :, Lp:], F, Hv, Wv, prefix=Lp, cap=CAP)
    P = da2.Plan(L)
    P.plan_from_tier_map(qj[:, :, Lp:], kj[:, :, Lp:], torch.from_numpy(tier).cuda())
    vd = torch.from_numpy(valid).cuda()
    P.attention_prefixed(qj[:, :, Lp:], kj[:, :, Lp:], vj[:, :, Lp:], oj[:, :, Lp:], qj[:, :, :Lp],
                         kj[:, :, :Lp], vj[:, :, :Lp], oj[:, :, :Lp], vd)
    torch.cuda.synchronize()
    o = oj.cpu().numpy()
    ref, refp, amb = O.attention_pfx(q, k, v, tier, F, Hv, Wv, qp, kp, vp, valid, amb=True, cap=CAP)
    G.check_close(o[:, :, Lp:], ref, "C=128 prefix: video rows", amb=amb)
    G.check_close(o[:, :, :Lp], refp, "C=128 prefix: prefix rows")


def test_layer_full_size():
    """The Wan-14B 720p layer at C = 128 in the benchmark's launch layout:
    heads 0 and 39 (draft keys, tier map, schedule bit-exact; four query
    tiles against the oracle)."""
    w = configs.WORKLOADS["wan14b-720p-c128"]
    hi, lo = w.budgets[0]
    q, k, v = G.inputs(w.B, w.H, w.F, w.Hv, w.Wv, w.d, w.seed, w.outliers)
    P, qd, kd = G.run_plan(q, k, w.F, w.Hv, w.Wv, hi, lo, w.lam, layout_bnhd=True, cap=CAP)
    o32 = G.run_attention(P, qd, kd, v, torch.float32, layout_bnhd=True)
    R, T, d = w.R, w.T, w.d
    assert P.layout.R == R and P.layout.T == T
    keys = G.host(P.debug("KEYS"), np.uint32).reshape(w.B, w.H, R, R)
    tier = P.tier_map().cpu().numpy()
    sched = G.host(P.debug("SCHEDULE"), np.int32).reshape(w.B, w.H, T, T + 3)
    perm = O.layout(w.F, w.Hv, w.Wv, cap=CAP)
    tiles = np.array(sorted({0, T // 3, (2 * T) // 3, T - 1}), np.int32)
    rows = np.concatenate([perm[t * 64:(t + 1) * 64] for t in tiles])
    for h in (0, 39):
        qh, kh, vh = (np.ascontiguousarray(x[:1, h:h + 1]) for x in (q, k, v))
        ref_plan = O.plan(qh, kh, w.F, w.Hv, w.Wv, hi, lo, w.lam, cap=CAP)
        assert np.array_equal(keys[:1, h:h + 1], ref_plan["keys"]), h
        assert np.array_equal(tier[:1, h:h + 1], ref_plan["tier"]), h
        assert np.array_equal(sched[:1, h:h + 1], G.schedule_from_tier(ref_plan["tier"], TPR)), h
        ref, amb = O.attention(qh, kh, vh, ref_plan["tier"], w.F, w.Hv, w.Wv, qblocks=tiles, amb=True, cap=CAP)
        idx = torch.from_numpy(rows.astype(np.int64)).cuda()
        got = o32[0, h].index_select(0, idx).cpu().numpy().astype(np.float64)
        rl, ma = G.check_close(got, ref.reshape(-1, d), "wan14b-720p C=128 h%d" % h, amb=amb.reshape(-1, d))
        dn = O.dense(qh, kh, vh, rows[::16])[0, 0]
        print("wan14b-720p C=128 h%d: rel_l2 %.2e max_abs %.2e vs oracle; rel_l2 %.2e vs dense fp64"
              % (h, rl, ma, G.rel_l2(got[::16], dn)))
