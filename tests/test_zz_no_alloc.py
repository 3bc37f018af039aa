"""The entry point for callers that cannot allocate (da2_forward_noalloc,
its workspace a static device array inside the library) against da2_plan +
da2_attention on a caller-owned workspace: the same kernels on the same
inputs, so the outputs must agree bit for bit.  Two calls in a row on one
GPU, the second on a smaller problem (a ragged layout), so the second call
starts from the first call's bytes in the shared array."""
import numpy as np
import pytest
import torch

from tests import gpu_common as G

pytestmark = pytest.mark.gpu

# (B, H, F, Hv, Wv, d, seed, hi, lo, skip_means, out dtype)
CASES = [
    (1, 2, 2, 64, 72, 128, 11, 1500, 3500, False, torch.float32),
    (1, 1, 2, 20, 28, 128, 12, 1000, 3000, True, torch.bfloat16),
]


def _run(case):
    from video_diffusion_dit_frame_amd import da2

    B, H, F, Hv, Wv, d, seed, hi, lo, sm, dt = case
    q, k, v = G.inputs(B, H, F, Hv, Wv, d, seed)
    qd, kd, vd = G.dev(q), G.dev(k), G.dev(v)
    L = da2.Layout.for_tensor(qd, F, Hv, Wv)
    assert L.workspace_bytes <= da2.noalloc_bytes()
    P = da2.Plan(L)
    P.plan(qd, kd, hi, lo, skip_means=sm)
    ref = torch.empty(vd.shape, dtype=dt, device="cuda")
    P.attention(qd, kd, vd, ref)
    o = torch.full(vd.shape, float("nan"), dtype=dt, device="cuda")
    da2.forward_noalloc(L, qd, kd, vd, o, hi, lo, skip_means=sm)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ref.float().cpu().numpy()


def test_noalloc_matches_workspace_entry_points():
    for case in CASES:
        print("no-alloc call", case[:9], flush=True)
        got, ref = _run(case)
        assert np.isfinite(got).all()
        assert np.array_equal(got, ref), case
