"""GPU parity of the 16-bit tier (the paper's 16-bit path, bf16 operands):
three-level plans bit-exact against the oracle (draft keys, tier map with
T16 / T8 / T4 quotas, schedule) and the phased attention with a 16-bit phase
against the oracle (rel-L2 <= 1e-3, every element within 5e-3), for plan tier maps at the paper's allocations and
for synthetic tier families that exercise every phase order and boundary.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import gpu_common as G

pytestmark = pytest.mark.gpu

# (B, H, F, Hv, Wv, d, seed, outliers)
TINY = (1, 2, 4, 16, 16, 64, 20260926, False)
MEDIUM = (1, 2, 2, 64, 72, 128, 11, True)
RAGGED = (2, 1, 3, 24, 40, 128, 12, True)

# (full, hi, lo) basis points: the paper's 85/0/7.5/7.5 allocation (skip,
# 4-bit, 8-bit, 16-bit), one with every tier present, and all 16-bit
BUDGETS = [(750, 750, 0), (500, 1500, 3000), (10000, 0, 0)]


def _inputs(c):
    B, H, F, Hv, Wv, d, seed, outl = c
    q, k, v = G.inputs(B, H, F, Hv, Wv, d, seed, outl)
    return F, Hv, Wv, q, k, v


CASES = [(w, b) for w in (TINY, RAGGED) for b in BUDGETS] + [(MEDIUM, BUDGETS[0]), (MEDIUM, BUDGETS[2])]
IDS = ["%s-%s" % (w, b) for w in ("tiny", "ragged") for b in ("85-0-7.5-7.5", "mixed", "all16")] + [
    "medium-85-0-7.5-7.5", "medium-all16"]


@pytest.mark.parametrize("which,budget", CASES, ids=IDS)
def test_three_tier_plan_and_attention(which, budget):
    full, hi, lo = budget
    F, Hv, Wv, q, k, v = _inputs(which)
    P, qd, kd = G.run_plan(q, k, F, Hv, Wv, hi, lo, full=full)
    o = G.run_attention(P, qd, kd, v).cpu().numpy()
    ref = O.plan(q, k, F, Hv, Wv, hi, lo, full_bp=full)
    keys = G.host(P.debug("KEYS"), np.uint32).reshape(ref["keys"].shape)
    assert np.array_equal(keys, ref["keys"])
    tier = P.tier_map().cpu().numpy()
    assert np.array_equal(tier, ref["tier"])
    R = tier.shape[-1]
    t16, t8c, tk = O.quotas3(R * R, full, hi, lo)
    assert ((tier == 16).sum(axis=(2, 3)) == t16).all()
    assert ((tier == 8).sum(axis=(2, 3)) == t8c - t16).all()
    assert ((tier == 4).sum(axis=(2, 3)) == tk - t8c).all()
    sch = G.host(P.debug("SCHEDULE"), np.int32).reshape(tier.shape[:3] + (-1,))
    assert np.array_equal(sch, G.schedule_from_tier(tier))
    r, amb = O.attention(q, k, v, tier, F, Hv, Wv, amb=True)
    rl, ma = G.check_close(o, r, "budget %s" % (budget,), amb=amb)
    rows = np.arange(0, q.shape[2], 97, dtype=np.int32)
    dn = O.dense(q, k, v, rows)
    print("16/8/4 = %s: rel_l2 %.3e max_abs %.3e vs oracle; rel_l2 %.3e vs dense fp64"
          % (budget, rl, ma, G.rel_l2(o[:, :, rows], dn)))


def _families(B, H, R, seed):
    rng = np.random.default_rng(seed)
    fam = {
        "all16": np.full((B, H, R, R), 16, np.uint8),
        "mixed16": rng.choice(np.array([0, 4, 8, 16], np.uint8), size=(B, H, R, R)),
        # 16-bit then MXFP4 with no FP8 tile: no change of value units
        "16_then_4": rng.choice(np.array([0, 4, 16], np.uint8), size=(B, H, R, R)),
        # 16-bit then FP8 only: units change once each way
        "16_then_8": rng.choice(np.array([0, 8, 16], np.uint8), size=(B, H, R, R)),
    }
    t = rng.choice(np.array([0, 4, 8, 16], np.uint8), size=(B, H, R, R), p=[0.4, 0.2, 0.2, 0.2])
    t[:, :, ::3, :] = 0          # empty query regions
    fam["empty_rows"] = t
    s = np.zeros((B, H, R, R), np.uint8)
    s[:, :, :, R // 2] = 16      # a single 16-bit tile per row,
    s[:, :, 1::2, 0] = 4         # with one MXFP4 tile on odd rows
    fam["single16"] = s
    return fam


@pytest.mark.parametrize("which", [TINY, RAGGED], ids=["tiny", "ragged"])
def test_tier16_families(which):
    from video_diffusion_dit_frame_amd import da2

    F, Hv, Wv, q, k, v = _inputs(which)
    qd, kd, vd = G.dev(q), G.dev(k), G.dev(v)
    L = da2.Layout.for_tensor(qd, F, Hv, Wv)
    P = da2.Plan(L)
    B, H, N, d = q.shape
    R = N // 64
    for name, tier in _families(B, H, R, 9).items():
        P.plan_from_tier_map(qd, kd, torch.from_numpy(tier).cuda())
        o = torch.empty(vd.shape, dtype=torch.float32, device="cuda")
        P.attention(qd, kd, vd, o)
        got = o.cpu().numpy()
        assert np.array_equal(P.tier_map().cpu().numpy(), tier)
        sch = G.host(P.debug("SCHEDULE"), np.int32).reshape(tier.shape[:3] + (-1,))
        assert np.array_equal(sch, G.schedule_from_tier(tier)), name
        ref, amb = O.attention(q, k, v, tier, F, Hv, Wv, amb=True)
        G.check_close(got, ref, name, amb=amb)
        if name == "empty_rows":
            dead = O.layout(F, Hv, Wv).reshape(R, 64)[::3].reshape(-1)
            assert (got[:, :, dead] == 0).all()


def test_tier16_strided_layout_matches_contiguous():
    """[B, N, H, d] storage: the 16-bit phase reads Q and K rows in place
    with the token stride, and gives results identical to [B, H, N, d]."""
    F, Hv, Wv, q, k, v = _inputs(MEDIUM)
    P1, q1, k1 = G.run_plan(q, k, F, Hv, Wv, 1500, 3500, full=500)
    o1 = G.run_attention(P1, q1, k1, v).cpu().numpy()
    P2, q2, k2 = G.run_plan(q, k, F, Hv, Wv, 1500, 3500, full=500, layout_bnhd=True)
    o2 = G.run_attention(P2, q2, k2, v, layout_bnhd=True)
    assert np.array_equal(P1.tier_map().cpu().numpy(), P2.tier_map().cpu().numpy())
    assert np.array_equal(o1, o2.cpu().numpy())


def test_tier16_bf16_output():
    F, Hv, Wv, q, k, v = _inputs(TINY)
    P, qd, kd = G.run_plan(q, k, F, Hv, Wv, 2000, 3000, full=1000)
    o32 = G.run_attention(P, qd, kd, v).cpu()
    o16 = G.run_attention(P, qd, kd, v, torch.bfloat16).cpu()
    assert torch.equal(o16, o32.to(torch.bfloat16))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("full,hi,lo", [(10000, 0, 0), (5000, 0, 5000), (5000, 5000, 0), (3000, 3000, 4000)])
def test_tier16_single_region_and_two_frames(d, full, hi, lo):
    """R = 1 and a two-frame layer with the 16-bit tier present."""
    for F, Hv, Wv in ((1, 8, 8), (2, 8, 16)):
        q, k, v = G.inputs(1, 2, F, Hv, Wv, d, 41 + d + full, True)
        P, qd, kd = G.run_plan(q, k, F, Hv, Wv, hi, lo, full=full)
        o = G.run_attention(P, qd, kd, v).cpu().numpy()
        ref_plan = O.plan(q, k, F, Hv, Wv, hi, lo, full_bp=full)
        tier = P.tier_map().cpu().numpy()
        assert np.array_equal(tier, ref_plan["tier"])
        ref, amb = O.attention(q, k, v, tier, F, Hv, Wv, amb=True)
        G.check_close(o, ref, "F%d %dx%d d%d (%d,%d,%d)" % (F, Hv, Wv, d, full, hi, lo), amb=amb)
