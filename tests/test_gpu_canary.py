"""Canary runs: the workspace and the output filled with NaN patterns before
the call must give the same plan and output, bit for bit, as a workspace
and output filled with zeros, with no NaN left in the output.  A kernel that
reads workspace it has not written in this call, or leaves an output
element unwritten, fails here (0xFF bytes are a NaN in fp32 and fp64 and -1
in the integer tables)."""
import numpy as np
import pytest
import torch

from tests import gpu_common as G

pytestmark = pytest.mark.gpu

# (B, H, F, Hv, Wv, d, seed, hi, lo, full, skip_means, cap)
CASES = {
    "grid": (1, 2, 2, 64, 72, 128, 31, 1500, 3500, 0, False, 64),
    "ragged": (2, 1, 3, 24, 40, 128, 32, 1000, 3000, 0, False, 64),
    "three_tier": (1, 2, 2, 32, 40, 128, 33, 1000, 2000, 1000, False, 64),
    "block_means": (1, 2, 2, 32, 40, 64, 34, 1000, 3000, 0, True, 64),
    "capacity128": (1, 2, 3, 24, 40, 128, 35, 1000, 3000, 0, False, 128),
}


def _run(case, fill):
    from video_diffusion_dit_frame_amd import da2

    B, H, F, Hv, Wv, d, seed, hi, lo, full, means, cap = case
    q, k, v = G.inputs(B, H, F, Hv, Wv, d, seed, True)
    qd, kd, vd = G.dev(q), G.dev(k), G.dev(v)
    L = da2.Layout.for_tensor(qd, F, Hv, Wv, cap=cap)
    ws = torch.full((L.workspace_bytes,), fill, dtype=torch.uint8, device="cuda")
    P = da2.Plan(L, workspace=ws)
    P.plan(qd, kd, hi, lo, full_bp=full, skip_means=means)
    o = torch.empty(vd.shape, dtype=torch.float32, device="cuda")
    o.view(torch.uint8).fill_(fill)
    P.attention(qd, kd, vd, o)
    torch.cuda.synchronize()
    return P.tier_map().cpu().numpy(), G.host(P.debug("KEYS"), np.uint32), o.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_nan_canary_workspace_and_output(name):
    print("canary case %s" % name, flush=True)
    t0, k0, o0 = _run(CASES[name], 0)
    t1, k1, o1 = _run(CASES[name], 0xFF)
    assert np.array_equal(t0, t1)
    assert np.array_equal(k0, k1)
    assert not np.isnan(o1).any()
    assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32))
