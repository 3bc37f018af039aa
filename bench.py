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
the MFMA peak weighted by where each product runs (16-bit tier: bf16; 8-bit
tier: Q K^T on INT8, P V on bf16; MXFP4 tier: FP4), i.e. its achieved
algorithmic FLOP/s over F / sum(F_part / P_part); cpu_baseline = the CPU
oracle timed on a bounded sample and extrapolated to the same unit.  The
same CPU leg checks the GPU result: one extra call with an fp32 output
after the timed steps, compared on the sampled query regions of head 0
with the oracle (rel-L2, max-abs, max-abs beyond the oracle's band bound)
and, on sampled rows, with dense fp64 attention ("accuracy").

--sweep runs the workload's budget points in turn (default workload: the
Wan-14B CFG pair at B = 2), one JSON line per point.  --cold-l2 writes
1 GiB before every timed step, so every step starts with cold caches, and
times the steps with events that exclude the flush.
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
PEAK_INT8 = 5000.0   # TOPS, MI355X dense INT8 MFMA
PEAK_FP4 = 10100.0   # TFLOP/s, MI355X dense FP4 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b-720p")
    ap.add_argument("--budget", type=int, default=0, help="index into the workload's budget list")
    ap.add_argument("--full-bp", type=int, default=0, help="16-bit share (basis points)")
    ap.add_argument("--hi-bp", type=int, default=None, help="8-bit share (INT8 Q K^T, FP8 weights and values; basis points), overriding --budget")
    ap.add_argument("--lo-bp", type=int, default=None, help="MXFP4 share (basis points), overriding --budget")
    ap.add_argument("--prefix", type=int, default=0, help="text-prefix tokens (joint attention)")
    ap.add_argument("--prefix-valid", type=int, default=None,
                    help="valid prefix keys per sequence (default: all)")
    ap.add_argument("--skip-means", action="store_true",
                    help="replace skipped tiles by block-mean tiles (tier 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain copy kernel of 1 GiB before the steps (reference for "
                         "HBM byte counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="every budget point of the workload (default sweep-wan14b-cfg), one line each")
    ap.add_argument("--cold-l2", action="store_true",
                    help="flush the caches with a 1 GiB write before every timed step")
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


N_ACC_REGIONS = 16   # query regions of head 0 compared with the oracle
N_ACC_DENSE = 64     # of their rows compared with dense fp64 attention


def cpu_baseline(w, q, k, v, hi, lo, full, sm, gpu_head0, tier_head0):
    """The CPU leg: time the oracle (as it stands) on one head -- the full
    plan, then tiered attention on 1 query region and on 401 evenly spaced
    ones (about 10 s of CPU work on 16 host cores).  The per-head fixed part
    (operand quantization) and the per-region part follow from the two
    timings; the head total is extrapolated to all regions and heads.  The
    same leg compares the GPU result of head 0 (gpu_head0: fp32 [N, d] in
    token order, tier_head0: its tier map) with the oracle on
    N_ACC_REGIONS query regions and with dense fp64 attention on
    N_ACC_DENSE of their rows.  Returns (cpu_baseline, accuracy)."""
    from oracle import oracle as O

    qs, ks, vs = q[:1, :1].copy(), k[:1, :1].copy(), v[:1, :1].copy()
    t0 = time.perf_counter()
    pl = O.plan(qs, ks, w.F, w.Hv, w.Wv, hi, lo, w.lam, full_bp=full, skip_means=sm, cap=w.cap)
    t_plan = time.perf_counter() - t0
    R = w.T   # query tiles of 64 rows (the regions at capacity 64)
    n_many = 401
    sel1 = np.array([R // 2], np.int32)
    selm = np.array([(j * R) // n_many for j in range(n_many)], np.int32)
    t0 = time.perf_counter()
    O.attention(qs, ks, vs, pl["tier"], w.F, w.Hv, w.Wv, qblocks=sel1, cap=w.cap)
    t1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    ref_m = O.attention(qs, ks, vs, pl["tier"], w.F, w.Hv, w.Wv, qblocks=selm, cap=w.cap)
    tm = time.perf_counter() - t0
    per_region = max((tm - t1) / (n_many - 1), 1e-9)
    per_head_fixed = max(t1 - per_region, 0.0)
    t_head = t_plan + per_head_fixed + per_region * R
    total = t_head * w.B * w.H
    dense_flop = 4.0 * w.B * w.H * float(w.N) ** 2 * w.d
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    base = {
        "value": dense_flop / total / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": ("1 of %d heads: full plan (%.2f s), tiered attention on 1 and on %d query "
                   "tiles of 64 rows (%.2f s, %.2f s); per-head fixed %.2f s + %.4f s per tile, "
                   "extrapolated to %d tiles x %d heads = %.0f s"
                   % (w.B * w.H, t_plan, n_many, t1, tm, per_head_fixed, per_region, R,
                      w.B * w.H, total)),
    }
    # accuracy of the GPU result on sampled query regions of head 0
    acc_regions = np.array([(j * R) // N_ACC_REGIONS for j in range(N_ACC_REGIONS)], np.int32)
    ref, amb = O.attention(qs, ks, vs, pl["tier"], w.F, w.Hv, w.Wv, qblocks=acc_regions, amb=True, cap=w.cap)
    perm = O.layout(w.F, w.Hv, w.Wv, cap=w.cap)
    tok = perm[(acc_regions[:, None] * 64 + np.arange(64)).ravel()]
    keep = tok >= 0
    ref = ref.reshape(-1, w.d)[keep]
    amb = amb.reshape(-1, w.d)[keep]
    got = gpu_head0[tok[keep]].astype(np.float64)
    err = np.abs(got - ref)
    rows = tok[keep][np.linspace(0, keep.sum() - 1, N_ACC_DENSE).astype(np.int64)]
    dn = O.dense(qs, ks, vs, rows.astype(np.int32))[0, 0]
    gd = gpu_head0[rows].astype(np.float64)

    def rel(a, b):
        return float(np.linalg.norm(a - b) / np.linalg.norm(b))

    accuracy = {
        "head": [0, 0],
        "tier_map_bit_exact": bool(np.array_equal(tier_head0, pl["tier"][0, 0])),
        "vs_oracle": {"rows": int(keep.sum()), "query_regions": N_ACC_REGIONS, "rel_l2": rel(got, ref),
                      "max_abs": float(err.max()), "max_abs_beyond_band": float((err - amb).max())},
        "vs_dense_fp64": {"rows": N_ACC_DENSE, "rel_l2": rel(gd, dn), "max_abs": float(np.abs(gd - dn).max())},
        "output": "fp32 (one extra call after the timed steps)",
    }
    return base, accuracy


def measure(args, w, hi, lo, full, q, k, v, torch, da2, synth):
    """One workload point: warmup, timed steps, roofline, CPU leg.  Returns
    the JSON record."""
    dev = torch.device("cuda:0")
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
    L = da2.Layout.for_tensor(qd, w.F, w.Hv, w.Wv, prefix=Lp, cap=w.cap)
    P = da2.Plan(L)
    stream = torch.cuda.current_stream()
    valid = torch.full((w.B,), nv, dtype=torch.int32, device=dev) if Lp else None
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev) if args.cold_l2 else None

    def attend(out=o, outp=oj[:, :, :Lp]):
        if Lp:
            P.attention_prefixed(qd, kd, vd, out, qj[:, :, :Lp], kj[:, :, :Lp], vj[:, :, :Lp], outp, valid, stream)
        else:
            P.attention(qd, kd, vd, out, stream)

    sm = args.skip_means

    def step():
        P.plan(qd, kd, hi, lo, w.lam, 0, stream, full_bp=full, skip_means=sm)
        attend()

    print("[bench] %s budget (bf16 %d, 8-bit %d, MXFP4 %d): warmup %d"
          % (w.name, full, hi, lo, args.warmup), file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    P.timing(True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(float(i))   # 1 GiB written: caches cold for the step
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
    if flush is not None:
        # the flush is not part of the step: time the steps by their events
        ms_step = float(np.mean([a.elapsed_time(c) for a, _, c in ev]))
    kt = P.timing_read()
    attn_kernel_ms = float(np.mean(kt)) if len(kt) else float("nan")
    P.timing(False)
    print("[bench] timed %d steps: %.3f ms/step (plan %.3f, attention call %.3f, kernel %.3f)"
          % (args.steps, ms_step, plan_ms, attn_call_ms, attn_kernel_ms), file=sys.stderr, flush=True)

    # work accounting (head-scope quotas, identical for every (b, h)); a
    # region pair of capacity cap is (cap / 64)^2 tiles of 64 x 64
    R = w.R
    t16, t8c, tk = da2.quotas3(R * R, full, hi, lo)
    tile_flop = 4.0 * 64 * 64 * w.d * (w.cap // 64) ** 2
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
    # where each product runs: 8-bit tier Q K^T on INT8, its P V on bf16
    wsum = f16 / PEAK_BF16 + 0.5 * f8 / PEAK_INT8 + 0.5 * f8 / PEAK_BF16 + f4 / PEAK_FP4
    peak_eff = fx / wsum if fx > 0 else PEAK_INT8
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
                   "capacity": w.cap,
                   "budget_bp": ({"bf16": full} if full else {}) | {"8bit": hi, "mxfp4": lo},
                   "lambda": w.lam, "ranking": "head",
                   "storage": "[B,N,H,d] bf16", "output": "bf16",
                   "caches": "cold (1 GiB written before every step)" if flush is not None else "warm"}
                  | ({"prefix": Lp, "prefix_valid": nv} if Lp else {})
                  | ({"skip_means": True} if sm else {}),
        "plan_ms": plan_ms,
        "attention_call_ms": attn_call_ms,
        "attention_kernel_ms": attn_kernel_ms,
        "dense_equiv_tflops_attention_kernel": dense_flop / t_attn / 1e12,
        "tier_weighted_mfma_util": util,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak_eff, "unit": "TFLOP/s",
                     "frac": achieved / peak_eff,
                     "traffic": None if Lp or sm or flush is not None
                     else measured_traffic(w.name, [hi, lo], full),
                     "kernel": "k_attn",
                     "peak_basis": "bf16 2.5 PFLOP/s for the 16-bit tier and the 8-bit tier's P V, "
                                   "INT8 5.0 POPS for the 8-bit tier's Q K^T, FP4 10.1 for MXFP4, "
                                   "weighted by algorithmic flops"},
    }
    if not args.no_cpu_baseline and not Lp:
        # one more call with an fp32 output, for the CPU leg's accuracy check
        o32 = torch.empty((w.B, w.N, w.H, w.d), dtype=torch.float32, device=dev).permute(0, 2, 1, 3)
        attend(o32)
        torch.cuda.synchronize()
        gpu_head0 = o32[0, 0].cpu().numpy()
        tier_head0 = P.tier_map()[0, 0].cpu().numpy()
        del o32
        print("[bench] CPU leg: oracle baseline and accuracy", file=sys.stderr, flush=True)
        out["cpu_baseline"], out["accuracy"] = cpu_baseline(w, q, k, v, hi, lo, full, sm, gpu_head0, tier_head0)
    del P, L, qj, kj, vj, oj, flush
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this operator shards over (batch, head) with no "
              "exchange, so a multi-GPU run is not part of this benchmark (got --gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    from video_diffusion_dit_frame_amd import configs, da2, synth

    name = "sweep-wan14b-cfg" if args.sweep and args.workload == "wan14b-720p" else args.workload
    w = configs.WORKLOADS[name]
    print("[bench] generating %s inputs (B=%d H=%d N=%d d=%d)" % (w.name, w.B, w.H, w.N, w.d),
          file=sys.stderr, flush=True)
    q, k, v = synth.make_qkv(w.B, w.H, w.F, w.Hv, w.Wv, w.d, w.seed, w.outliers)
    points = list(w.budgets) if args.sweep else [w.budgets[args.budget]]
    for hi, lo in points:
        hi = hi if args.hi_bp is None or args.sweep else args.hi_bp
        lo = lo if args.lo_bp is None or args.sweep else args.lo_bp
        out = measure(args, w, hi, lo, args.full_bp, q, k, v, torch, da2, synth)
        print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
