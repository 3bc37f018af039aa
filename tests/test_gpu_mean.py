"""GPU parity of block-mean tiles ([Triage] abstract: a skipped tile replaced
by its block means; scored with the average-branch draft logit of
DraftAttention2 Eq. 2 and weighted by the key region's token count) against
the oracle (rel-L2 <= 1e-3, every element within 5e-3): plans with skip replacement (tier maps bit-exact), tier maps
mixing block-mean tiles with every other tier, rows of block-mean tiles only,
a ragged layout, a text prefix, and the Wan-14B-720p layer at full size.  The
error against dense fp64 attention with and without skip replacement is
printed for the same plan."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import gpu_common as G
from video_diffusion_dit_frame_amd import synth

pytestmark = pytest.mark.gpu
MEAN = 1

# (B, H, F, Hv, Wv, d, seed, outliers, hi, lo)
TINY = (1, 2, 4, 16, 16, 64, 51, False, 2500, 2500)
MEDIUM = (1, 2, 2, 64, 72, 128, 52, True, 1500, 3500)
RAGGED = (1, 2, 2, 20, 28, 128, 53, True, 1000, 3000)


def _inputs(c):
    B, H, F, Hv, Wv, d, seed, outl, hi, lo = c
    q, k, v = G.inputs(B, H, F, Hv, Wv, d, seed, outl)
    return F, Hv, Wv, hi, lo, q, k, v


@pytest.mark.parametrize("c", [TINY, MEDIUM, RAGGED], ids=["tiny", "medium", "ragged"])
def test_plan_with_skip_replacement(c):
    F, Hv, Wv, hi, lo, q, k, v = _inputs(c)
    from video_diffusion_dit_frame_amd import da2

    qd, kd = G.dev(q), G.dev(k)
    P = da2.Plan(da2.Layout.for_tensor(qd, F, Hv, Wv))
    P.plan(qd, kd, hi, lo, skip_means=True)
    o = G.run_attention(P, qd, kd, v).cpu().numpy()
    ref_plan = O.plan(q, k, F, Hv, Wv, hi, lo, skip_means=True)
    tier = P.tier_map().cpu().numpy()
    assert np.array_equal(tier, ref_plan["tier"])
    assert (tier == MEAN).any()
    r, amb = O.attention(q, k, v, tier, F, Hv, Wv, amb=True)
    rl, ma = G.check_close(o, r, "skip replacement", amb=amb)
    # the same plan without replacement, both against dense fp64
    P0 = da2.Plan(da2.Layout.for_tensor(qd, F, Hv, Wv))
    P0.plan(qd, kd, hi, lo)
    o0 = G.run_attention(P0, qd, kd, v).cpu().numpy()
    rows = np.arange(0, q.shape[2], 37, dtype=np.int32)
    dn = O.dense(q, k, v, rows)
    print("%s: rel_l2 %.2e vs oracle; vs dense fp64: skipped %.3f, block means %.3f"
          % (c[3:5], rl, G.rel_l2(o0[:, :, rows], dn), G.rel_l2(o[:, :, rows], dn)))


def _families(B, H, R, seed):
    rng = np.random.default_rng(seed)
    only = np.full((B, H, R, R), MEAN, np.uint8)
    only[:, :, 0::2, :] = rng.choice(np.array([0, 4, 8, 16], np.uint8), size=(B, H, (R + 1) // 2, R))
    return {
        "all": rng.choice(np.array([0, MEAN, 4, 8, 16], np.uint8), size=(B, H, R, R)),
        "mean_and_4": rng.choice(np.array([MEAN, 4], np.uint8), size=(B, H, R, R), p=[0.8, 0.2]),
        "mean_only_rows": only,
        "all_mean": np.full((B, H, R, R), MEAN, np.uint8),
    }


@pytest.mark.parametrize("c", [TINY, MEDIUM, RAGGED], ids=["tiny", "medium", "ragged"])
@pytest.mark.parametrize("family", ["all", "mean_and_4", "mean_only_rows", "all_mean"])
def test_mean_tier_families(c, family):
    F, Hv, Wv, hi, lo, q, k, v = _inputs(c)
    from video_diffusion_dit_frame_amd import da2

    R = O.regions(F, Hv, Wv)
    tier = _families(q.shape[0], q.shape[1], R, 9)[family]
    qd, kd = G.dev(q), G.dev(k)
    P = da2.Plan(da2.Layout.for_tensor(qd, F, Hv, Wv))
    P.plan_from_tier_map(qd, kd, torch.from_numpy(tier).cuda())
    o = G.run_attention(P, qd, kd, v).cpu().numpy()
    r, amb = O.attention(q, k, v, tier, F, Hv, Wv, amb=True)
    G.check_close(o, r, family, amb=amb)


def test_mean_tiles_with_prefix():
    from tests.test_gpu_prefix import run_prefixed

    F, Hv, Wv, hi, lo, q, k, v = _inputs(MEDIUM)
    qp, kp, vp = synth.make_prefix(1, 2, 90, 128, 54)
    R = O.regions(F, Hv, Wv)
    tier = _families(1, 2, R, 10)["all"]
    o, op, _ = run_prefixed(q, k, v, qp, kp, vp, F, Hv, Wv, tier=tier, valid=[77])
    r, rp, amb = O.attention_pfx(q, k, v, tier, F, Hv, Wv, qp, kp, vp, [77], amb=True)
    G.check_close(o, r, "mean + prefix video rows", amb=amb)
    G.check_close(op, rp, "mean + prefix prefix rows")


def test_skip_replacement_full_size():
    """Wan-14B-720p layer with skip replacement, [B,N,H,d] storage, two heads
    sampled (plan bit-exact, four query regions against the oracle)."""
    from video_diffusion_dit_frame_amd import configs

    w = configs.WORKLOADS["wan14b-720p"]
    hi, lo = w.budgets[0]
    q, k, v = G.inputs(w.B, w.H, w.F, w.Hv, w.Wv, w.d, w.seed, w.outliers)
    from video_diffusion_dit_frame_amd import da2

    qd, kd = G.dev(q), G.dev(k)
    qd = qd.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    kd = kd.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    P = da2.Plan(da2.Layout.for_tensor(qd, w.F, w.Hv, w.Wv))
    P.plan(qd, kd, hi, lo, w.lam, skip_means=True)
    o = G.run_attention(P, qd, kd, v, layout_bnhd=True)
    tier = P.tier_map().cpu().numpy()
    perm = O.layout(w.F, w.Hv, w.Wv)
    R = w.R
    regions = np.array([0, R // 3, (2 * R) // 3, R - 1], np.int32)
    rows = np.concatenate([perm[a * 64:(a + 1) * 64] for a in regions])
    for h in (0, 39):
        sl = lambda x: np.ascontiguousarray(x[:, h:h + 1])
        qh, kh, vh = sl(q), sl(k), sl(v)
        ref_plan = O.plan(qh, kh, w.F, w.Hv, w.Wv, hi, lo, w.lam, skip_means=True)
        assert np.array_equal(tier[:, h:h + 1], ref_plan["tier"])
        r, amb = O.attention(qh, kh, vh, ref_plan["tier"], w.F, w.Hv, w.Wv, qblocks=regions, amb=True)
        got = o[0, h].index_select(0, torch.from_numpy(rows.astype(np.int64)).cuda()).cpu().numpy()
        rl, ma = G.check_close(got, r.reshape(-1, w.d), "wan14b skip replacement h%d" % h,
                               amb=amb.reshape(-1, w.d))
        dn = O.dense(qh, kh, vh, rows[::16])[0, 0]
        print("wan14b-720p h%d skip replacement: rel_l2 %.2e vs oracle; %.3f vs dense fp64"
              % (h, rl, G.rel_l2(got[::16], dn)))
