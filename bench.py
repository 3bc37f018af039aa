#!/usr/bin/env python3
"""Benchmark of the DraftAttention2 hot path on one MI355X.

One step = the whole hot path on one layer of synthetic video-DiT
activations: da2_plan (Q/K preparation, draft scoring, ranking, schedule)
followed by da2_attention (V preparation, phased 16-bit/8-bit/MXFP4 attention
with the output written back in token order).  Inputs are resident in HBM before the
timed region; Q/K/V use the [B, N, H, d] storage of DiT attention layers.

With --prefix Lp the layer is joint text-video attention (App. C.1 of the
paper): a text prefix of Lp tokens (the first --prefix-valid of them valid)
precedes the video tokens in the same [B, Lp + N, H, d] tensors, and the
step's attention call is da2_attention_prefixed.

Prints one JSON line.  value = dense-equivalent attention TFLOP/s of the
complete step (4 B H N^2 d per step; with a prefix, 4 B H (Lp + N)(nv + N) d
over the nv valid prefix keys); roofline = the attention kernel against
the tier-weighted MFMA peak (its achieved executed FLOP/s over
(F16 + F8 + F4) / (F16/P16 + F8/P8 + F4/P4)); cpu_baseline = the CPU oracle timed on a
bounded sample and extrapolated to the same unit.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2500.0   # TFLOP/s, MI355X dense bf16 MFMA
PEAK_FP8 = 5000.0    # TFLOP/s, MI355X dense FP8 MFMA
PEAK_FP4 = 10100.0   # TFLOP/s, MI355X dense FP4 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b-720p")
    ap.add_argument("--budget", type=int, default=0, help="index into the workload's budget list")
    ap.add_argument("--full-bp", type=int, default=0, help="16-bit share (basis points)")
    ap.add_argument("--hi-bp", type=int, default=None, help="FP8 share, overriding --budget")
    ap.add_argument("--lo-bp", type=int, default=None, help="MXFP4 share, overriding --budget")
    ap.add_argument("--prefix", type=int, default=0, help="text-prefix tokens (joint attention)")
    ap.add_argument("--prefix-valid", type=int, default=None,
                    help="valid prefix keys per sequence (default: all)")
    ap.add_argument("--skip-means", action="store_true",
                    help="replace skipped tiles by block-mean tiles (tier 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain copy kernel of 1 GiB before the steps (reference for "
                         "HBM byte counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_attn_wan14b-720p_traffic.json")
ATTN_SOURCE = os.path.join(ROOT, "video_diffusion_dit_frame_amd", "csrc", "k_attn.hip")


def measured_traffic(workload, budget, full_bp):
    """HBM bytes per attention-kernel launch from the committed counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or None
    when there is none for this workload or the kernel source has changed
    since the counters were taken."""
    import hashlib

    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        with open(ATTN_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if rec.get("kernel_source_sha256") != sha or rec.get("workload") != workload \
            or rec.get("budget_bp") != budget or rec.get("full_bp", 0) != full_bp:
        return None
    return float(rec["hbm_bytes_per_launch"])


def cpu_baseline(w, q, k, v, hi, lo, full):
    """Time the oracle (as it stands) on one head: the full plan, then tiered
    attention on 1 query region and on 401 evenly spaced ones (about 10 s of
    CPU work on 16 host cores).  The per-head
    fixed part (operand quantization) and the per-region part follow from the
    two timings; the head total is extrapolated to all regions and heads."""
    from oracle import oracle as O

    qs, ks, vs = q[:1, :1].copy(), k[:1, :1].copy(), v[:1, :1].copy()
    t0 = time.perf_counter()
    pl = O.plan(qs, ks, w.F, w.Hv, w.Wv, hi, lo, w.lam, full_bp=full)
    t_plan = time.perf_counter() - t0
    R = w.R
    n_many = 401
    sel1 = np.array([R // 2], np.int32)
    selm = np.array([(j * R) // n_many for j in range(n_many)], np.int32)
    t0 = time.perf_counter()
    O.attention(qs, ks, vs, pl["tier"], w.F, w.Hv, w.Wv, qblocks=sel1)
    t1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.attention(qs, ks, vs, pl["tier"], w.F, w.Hv, w.Wv, qblocks=selm)
    tm = time.perf_counter() - t0
    per_region = max((tm - t1) / (n_many - 1), 1e-9)
    per_head_fixed = max(t1 - per_region, 0.0)
    t_head = t_plan + per_head_fixed + per_region * R
    total = t_head * w.B * w.H
    dense_flop = 4.0 * w.B * w.H * float(w.N) ** 2 * w.d
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return {
        "value": dense_flop / total / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": ("1 of %d heads: full plan (%.2f s), tiered attention on 1 and on %d query "
                   "regions (%.2f s, %.2f s); per-head fixed %.2f s + %.4f s per region, "
                   "extrapolated to %d regions x %d heads = %.0f s"
                   % (w.B * w.H, t_plan, n_many, t1, tm, per_head_fixed, per_region, R,
                      w.B * w.H, total)),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this operator shards over (batch, head) with no "
              "exchange, so a multi-GPU run is not part of this benchmark (got --gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    from video_diffusion_dit_frame_amd import configs, da2, synth

    w = configs.WORKLOADS[args.workload]
    hi, lo = w.budgets[args.budget]
    hi = hi if args.hi_bp is None else args.hi_bp
    lo = lo if args.lo_bp is None else args.lo_bp
    full = args.full_bp
    dev = torch.device("cuda:0")
    print("[bench] generating %s inputs (B=%d H=%d N=%d d=%d)" % (w.name, w.B, w.H, w.N, w.d),
          file=sys.stderr, flush=True)
    q, k, v = synth.make_qkv(w.B, w.H, w.F, w.Hv, w.Wv, w.d, w.seed, w.outliers)
    Lp = args.prefix
    nv = Lp if args.prefix_valid is None else min(max(args.prefix_valid, 0), Lp)
    if Lp:
        qp, kp, vp = synth.make_prefix(w.B, w.H, Lp, w.d, w.seed + 7)
        q, k, v = (np.concatenate([a, b], axis=2) for a, b in ((qp, q), (kp, k), (vp, v)))
        del qp, kp, vp

    def to_bnhd(x):
        t = da2.to_device_bf16(x)                 # [B, H, Lp + N, d]
        t = t.permute(0, 2, 1, 3).contiguous()    # [B, Lp + N, H, d] storage
        return t.permute(0, 2, 1, 3)              # [B, H, Lp + N, d] view

    qj, kj, vj = to_bnhd(q), to_bnhd(k), to_bnhd(v)
    qd, kd, vd = qj[:, :, Lp:], kj[:, :, Lp:], vj[:, :, Lp:]
    if args.calibrate_copy:
        # a plain copy kernel: reads and writes exactly 2^30 bytes
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    oj = torch.empty((w.B, Lp + w.N, w.H, w.d), dtype=torch.bfloat16, device=dev).permute(0, 2, 1, 3)
    o = oj[:, :, Lp:]
    L = da2.Layout.for_tensor(qd, w.F, w.Hv, w.Wv, prefix=Lp)
    P = da2.Plan(L)
    stream = torch.cuda.current_stream()
    valid = torch.full((w.B,), nv, dtype=torch.int32, device=dev) if Lp else None

    def attend():
        if Lp:
            P.attention_prefixed(qd, kd, vd, o, qj[:, :, :Lp], kj[:, :, :Lp], vj[:, :, :Lp],
                                 oj[:, :, :Lp], valid, stream)
        else:
            P.attention(qd, kd, vd, o, stream)

    sm = args.skip_means

    def step():
        P.plan(qd, kd, hi, lo, w.lam, 0, stream, full_bp=full, skip_means=sm)
        attend()

    print("[bench] warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    P.timing(True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        P.plan(qd, kd, hi, lo, w.lam, 0, stream, full_bp=full, skip_means=sm)
        ev[i][1].record(stream)
        attend()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    plan_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    attn_call_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
    kt = P.timing_read()
    attn_kernel_ms = float(np.mean(kt)) if len(kt) else float("nan")
    P.timing(False)
    print("[bench] timed %d steps: %.3f ms/step (plan %.3f, attention call %.3f, kernel %.3f)"
          % (args.steps, ms_step, plan_ms, attn_call_ms, attn_kernel_ms), file=sys.stderr, flush=True)

    # work accounting (head-scope quotas, identical for every (b, h))
    R = w.R
    t16, t8c, tk = da2.quotas3(R * R, full, hi, lo)
    tile_flop = 4.0 * 64 * 64 * w.d
    f16 = w.B * w.H * t16 * tile_flop
    f8 = w.B * w.H * (t8c - t16) * tile_flop
    f4 = w.B * w.H * (tk - t8c) * tile_flop
    # prefix interactions run on the 16-bit path.  The attention kernel
    # (k_attn, the timed one) does the video rows x valid prefix keys; the
    # prefix rows x (valid prefix keys + video keys) run in k_attn_prefix,
    # outside the timed kernel and outside this roofline.
    f16 += 4.0 * w.B * w.H * w.d * float(w.N) * nv
    fx = f16 + f8 + f4
    dense_flop = 4.0 * w.B * w.H * float(Lp + w.N) * float(nv + w.N) * w.d
    t_attn = attn_kernel_ms * 1e-3
    wsum = f16 / PEAK_BF16 + f8 / PEAK_FP8 + f4 / PEAK_FP4
    peak_eff = fx / wsum if fx > 0 else PEAK_FP8
    achieved = fx / t_attn / 1e12
    util = wsum / 1e12 / t_attn

    out = {
        "metric": "dense-equiv attention TFLOP/s + tier-weighted MFMA util, Wan-14B-720p layer",
        "value": dense_flop / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16+" if full or Lp else "") + "int8+fp8_e4m3+mxfp4 (attention), f64 (draft scoring)",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "head_dim": w.d,
                   "frames": w.F, "height": w.Hv, "width": w.Wv, "tokens": w.N, "regions": R,
                   "budget_bp": ({"bf16": full} if full else {}) | {"fp8": hi, "mxfp4": lo},
                   "lambda": w.lam, "ranking": "head",
                   "storage": "[B,N,H,d] bf16", "output": "bf16"}
                  | ({"prefix": Lp, "prefix_valid": nv} if Lp else {})
                  | ({"skip_means": True} if sm else {}),
        "plan_ms": plan_ms,
        "attention_call_ms": attn_call_ms,
        "attention_kernel_ms": attn_kernel_ms,
        "dense_equiv_tflops_attention_kernel": dense_flop / t_attn / 1e12,
        "tier_weighted_mfma_util": util,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak_eff, "unit": "TFLOP/s",
                     "frac": achieved / peak_eff,
                     "traffic": None if Lp or sm else measured_traffic(w.name, [hi, lo], full),
                     "kernel": "k_attn",
                     "peak_basis": "tier-weighted bf16 2.5 / FP8 5.0 / FP4 10.1 PFLOP/s"},
    }
    if not args.no_cpu_baseline and not Lp and not sm:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, hi, lo, full)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
