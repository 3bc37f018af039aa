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


def run_plan(q, k, F, Hv, Wv, hi, lo, lam=0.2, scope=0, layout_bnhd=False, full=0):
    """Plan on the GPU.  Returns (plan, qd, kd) keeping the tensors alive."""
    from video_diffusion_dit_frame_amd import da2

    qd, kd = dev(q), dev(k)
    if layout_bnhd:
        qd = qd.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        kd = kd.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    L = da2.Layout.for_tensor(qd, F, Hv, Wv)
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


def schedule_from_tier(tier):
    """Expected schedule rows from a tier map: n16, n8, n4, the 16-bit key
    regions ascending, FP8 ascending, MXFP4 ascending, -1 padding."""
    B, H, R, _ = tier.shape
    out = np.full((B, H, R, R + 3), -1, np.int32)
    for b in range(B):
        for h in range(H):
            for a in range(R):
                lists = [np.nonzero(tier[b, h, a] == p)[0] for p in (16, 8, 4)]
                out[b, h, a, :3] = [len(x) for x in lists]
                cat = np.concatenate(lists)
                out[b, h, a, 3:3 + len(cat)] = cat
    return out


def rel_l2(x, ref):
    den = np.linalg.norm(ref)
    return np.linalg.norm(x - ref) / den if den > 0 else np.linalg.norm(x)


def check_kp(got, ref, allow, what=""):
    """Parity against the kernel-precision oracle: rel-L2 <= 1e-3 overall and
    every element within 5e-3 plus its allowance (undetermined decisions and
    matrix-core accumulation bounds)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rl = rel_l2(got, ref)
    diff = np.abs(got - ref)
    excess = diff - (ATOL_MAX + allow)
    ma = diff.max() if got.size else 0.0
    assert rl <= RTOL_L2, "%s rel_l2=%.3e (max_abs %.3e)" % (what, rl, ma)
    assert (excess <= 0).all(), "%s element beyond 5e-3 + allowance by %.3e (max_abs %.3e, rel_l2 %.3e)" % (
        what, excess.max(), ma, rl)
    return rl, ma


def check_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rl = rel_l2(got, ref)
    ma = np.abs(got - ref).max() if got.size else 0.0
    assert rl <= RTOL_L2 and ma <= ATOL_MAX, "%s rel_l2=%.3e max_abs=%.3e" % (what, rl, ma)
    return rl, ma
