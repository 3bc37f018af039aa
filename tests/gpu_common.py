"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding and the CPU oracle on the same seeded inputs."""
import numpy as np
import torch

from oracle import oracle as O
from video_diffusion_dit_frame_amd import synth

RTOL_L2 = 1e-3
ATOL_MAX = 5e-3


def inputs(B, H, F, Hv, Wv, d, seed, outliers=True):
    return synth.make_qkv(B, H, F, Hv, Wv, d, seed, outliers)


def dev(x):
    from video_diffusion_dit_frame_amd import da2

    return da2.to_device_bf16(x)


def host(t, dtype):
    return t.cpu().numpy().view(dtype)


def run_plan(q, k, F, Hv, Wv, hi, lo, lam=0.2, scope=0, layout_bnhd=False, full=0, cap=64):
    """Plan on the GPU (block capacity cap).  Returns (plan, qd, kd) keeping
    the tensors alive."""
    from video_diffusion_dit_frame_amd import da2

    qd, kd = dev(q), dev(k)
    if layout_bnhd:
        qd = qd.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        kd = kd.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    L = da2.Layout.for_tensor(qd, F, Hv, Wv, cap=cap)
    P = da2.Plan(L)
    P.plan(qd, kd, hi, lo, lam, scope, full_bp=full)
    return P, qd, kd


def run_attention(P, qd, kd, v, out_dtype=torch.float32, layout_bnhd=False):
    vd = dev(v)
    if layout_bnhd:  # [B,N,H,d] storage
        vd = vd.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        B, H, N, d = vd.shape
        o = torch.empty((B, N, H, d), dtype=out_dtype, device="cuda").permute(0, 2, 1, 3)
    else:
        o = torch.empty(vd.shape, dtype=out_dtype, device="cuda")
    P.attention(qd, kd, vd, o)
    torch.cuda.synchronize()
    return o


def schedule_from_tier(tier, tpr=1):
    """Expected schedule rows from a region tier map, one per query tile
    (tpr tiles per region): tile counts n16, n8, n4, then the key tiles of
    the 16-bit key regions ascending, 8-bit ascending, MXFP4 ascending, -1
    padding."""
    B, H, R, _ = tier.shape
    T = R * tpr
    out = np.full((B, H, T, T + 3), -1, np.int32)
    for b in range(B):
        for h in range(H):
            for a in range(R):
                lists = [np.nonzero(tier[b, h, a] == p)[0] for p in (16, 8, 4)]
                cat = np.concatenate(lists)
                tiles = (cat[:, None] * tpr + np.arange(tpr)).ravel()
                for i in range(tpr):
                    out[b, h, a * tpr + i, :3] = [len(x) * tpr for x in lists]
                    out[b, h, a * tpr + i, 3:3 + len(tiles)] = tiles
    return out


def rel_l2(x, ref):
    den = np.linalg.norm(ref)
    return np.linalg.norm(x - ref) / den if den > 0 else np.linalg.norm(x)


def report(got, ref, what="", dense=None):
    """Print the comparison with the oracle (and with dense fp64 attention on
    sampled rows) before it is asserted, so a failing case still shows its
    numbers."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    msg = "%s: vs oracle rel_l2 %.3e max_abs %.3e" % (what, rel_l2(got, ref), d.max() if d.size else 0.0)
    if dense is not None:
        msg += " | vs dense fp64 rel_l2 %.3e" % rel_l2(np.asarray(dense[0], np.float64), dense[1])
    print(msg, flush=True)


def check_close(got, ref, what="", amb=None):
    """Parity of the attention output with the oracle: rel-L2 <= 1e-3 over
    the compared rows, and every element within 5e-3 of the oracle plus the
    oracle's band bound amb for that element (the most the output can move
    when the weight codes whose decision lies within the GPU weights'
    precision band, 2^-16 relative, are taken either way: both results are
    correct).  amb=None: no band (outputs of unquantized weights only).
    Prints the plain and the band-aware numbers before asserting."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rl = rel_l2(got, ref)
    err = np.abs(got - ref)
    ma = err.max() if got.size else 0.0
    ex = (err - (0.0 if amb is None else np.asarray(amb, np.float64))).max() if got.size else 0.0
    if ma > ATOL_MAX:
        print("%s: max_abs %.3e exceeds %.0e; beyond the band bound %.3e" % (what, ma, ATOL_MAX, ex), flush=True)
    assert rl <= RTOL_L2 and ex <= ATOL_MAX, "%s rel_l2=%.3e max_abs=%.3e beyond band %.3e" % (what, rl, ma, ex)
    return rl, ma
