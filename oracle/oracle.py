"""ctypes front end of the CPU oracle (liboracle.so, built from da2_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product library
never loads this module or the shared object behind it.

All tensors are numpy arrays.  Q/K/V are uint16 bfloat16 bit patterns,
contiguous [B, H, N, d] with tokens in (frame, y, x) raster order.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "da2_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
BLK = 64

GCC_CMD = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-o", _LIB, _SRC, "-lm"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C, no contraction, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = list(GCC_CMD)
        cmd[cmd.index(_LIB)] = tmp
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        P = C.c_void_p
        i32, i64, f64 = C.c_int32, C.c_int64, C.c_double
        L.or_layout.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P]
        L.or_layout.restype = C.c_int
        L.or_regions.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int]
        L.or_regions.restype = C.c_int
        L.or_partition.argtypes = [C.c_int, C.c_int, P, P]
        L.or_partition.restype = C.c_int
        L.or_partition_bands.argtypes = [C.c_int, C.c_int, C.POINTER(C.c_int), P,
                                         C.POINTER(C.c_int64)]
        L.or_partition_bands.restype = C.c_int
        L.or_partition_c.argtypes = [C.c_int, C.c_int, C.c_int, P, P]
        L.or_partition_c.restype = C.c_int
        L.or_partition_bands_c.argtypes = [C.c_int, C.c_int, C.c_int, C.POINTER(C.c_int), P, P,
                                           C.POINTER(C.c_int64)]
        L.or_partition_bands_c.restype = C.c_int
        L.or_pool_head.argtypes = [P, C.c_int, P, C.c_int, C.c_int, P, P]
        L.or_exp_constants.argtypes = [P]
        L.or_exp.argtypes = [f64]
        L.or_exp.restype = f64
        L.or_draft_keys_head.argtypes = [P, P, P, P, C.c_int, C.c_int, f64, P, P]
        L.or_draft_logits_head.argtypes = [P, P, P, P, C.c_int, C.c_int, P, P]
        L.or_quotas.argtypes = [i64, i32, i32, i32, P, P, P]
        L.or_bf16_round.argtypes = [f64]
        L.or_bf16_round.restype = f64
        L.or_rank_head.argtypes = [P, C.c_int, C.c_int, i64, i64, i64, P]
        L.or_plan.argtypes = [C.c_int] * 7 + [P, P, i32, i32, i32, f64, C.c_int, C.c_int, P, P, P, P, P, P]
        L.or_plan.restype = C.c_int
        L.or_e4m3_value.argtypes = [C.c_int]
        L.or_e4m3_value.restype = f64
        L.or_e2m1_value.argtypes = [C.c_int]
        L.or_e2m1_value.restype = f64
        L.or_e4m3_encode.argtypes = [f64]
        L.or_e4m3_encode.restype = C.c_uint8
        L.or_e2m1_encode.argtypes = [f64]
        L.or_e2m1_encode.restype = C.c_uint8
        L.or_mx_exponent.argtypes = [f64]
        L.or_mx_exponent.restype = C.c_int
        L.or_mx_exponent_w.argtypes = [f64]
        L.or_mx_exponent_w.restype = C.c_int
        L.or_quant_qk.argtypes = [C.c_int] * 7 + [P, P, P, P, P]
        L.or_quant_qk.restype = C.c_int
        L.or_quant_v.argtypes = [C.c_int] * 7 + [P, P, P, P, P]
        L.or_quant_v.restype = C.c_int
        L.or_attention.argtypes = [C.c_int] * 7 + [P, P, P, P, C.c_int, P, P, P]
        L.or_attention.restype = C.c_int
        L.or_attention_trace.argtypes = [C.c_int] * 5 + [P, P, P, P, C.c_int, i64,
                                                         P, P, P, P, P, P, P, P]
        L.or_attention_trace.restype = i64
        L.or_attention_pfx.argtypes = [C.c_int] * 7 + [P, P, P, C.c_int, P, P, P, P, C.c_int,
                                                       P, C.c_int, P, C.c_int, P, P, P, P]
        L.or_attention_pfx.restype = C.c_int
        L.or_dense.argtypes = [C.c_int] * 4 + [P, P, P, C.c_int, P, P]
        L.or_dense.restype = C.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


def _u16(x):
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16, x.dtype
    return x


# ---------------------------------------------------------------- layout
def regions(F, Hv, Wv, cap=BLK) -> int:
    """R = F R_f regions of the partition at block capacity cap; raises when
    the frame has none."""
    R = lib().or_regions(F, Hv, Wv, cap)
    if R < 0:
        raise ValueError("no partition of a %d x %d frame" % (Hv, Wv))
    return R


def layout(F, Hv, Wv, cap=BLK) -> np.ndarray:
    """perm [R cap]: original token of each reordered position, -1 for padding."""
    perm = np.empty(regions(F, Hv, Wv, cap) * cap, dtype=np.int32)
    lib().or_layout(F, Hv, Wv, cap, _p(perm))
    return perm


def partition(Hv, Wv):
    """One frame's slot table: (tok [R_f, 64] int32 with y*Wv + x or -1,
    nvalid [R_f])."""
    Rf = -(-Hv * Wv // BLK)
    tok = np.empty((Rf, BLK), np.int32)
    nv = np.empty(Rf, np.int32)
    if lib().or_partition(Hv, Wv, _p(tok), _p(nv)) < 0:
        raise ValueError("no partition of a %d x %d frame" % (Hv, Wv))
    return tok, nv


def partition_bands(Hv, Wv):
    """(orientation 0 rows / 1 columns, band heights, total perimeter)."""
    o = C.c_int()
    per = C.c_int64()
    bands = np.empty(Hv + Wv, np.int32)
    m = lib().or_partition_bands(Hv, Wv, C.byref(o), _p(bands), C.byref(per))
    if m < 0:
        raise ValueError("no partition of a %d x %d frame" % (Hv, Wv))
    return o.value, bands[:m].copy(), per.value


def partition_c(Hv, Wv, cap):
    """The same partition for block capacity cap: (tok [R_f, cap], nvalid)."""
    Rf = -(-Hv * Wv // cap)
    tok = np.empty((Rf, cap), np.int32)
    nv = np.empty(Rf, np.int32)
    if lib().or_partition_c(Hv, Wv, cap, _p(tok), _p(nv)) < 0:
        raise ValueError("no partition of a %d x %d frame" % (Hv, Wv))
    return tok, nv


def partition_bands_c(Hv, Wv, cap):
    """(orientation, band heights, pieces per band, total perimeter) for
    block capacity cap."""
    o = C.c_int()
    per = C.c_int64()
    bands = np.empty(Hv + Wv, np.int32)
    pieces = np.empty(Hv + Wv, np.int32)
    m = lib().or_partition_bands_c(Hv, Wv, cap, C.byref(o), _p(bands), _p(pieces), C.byref(per))
    if m < 0:
        raise ValueError("no partition of a %d x %d frame" % (Hv, Wv))
    return o.value, bands[:m].copy(), pieces[:m].copy(), per.value


# ---------------------------------------------------------------- draft
def pool_head(X: np.ndarray, F, Hv, Wv, cap=BLK):
    """X: [N, d] uint16 -> (avg [R, d] f64, max [R, d] f32) over the R
    regions of capacity cap."""
    X = _u16(X)
    N, d = X.shape
    R = regions(F, Hv, Wv, cap)
    perm = layout(F, Hv, Wv, cap)
    avg = np.empty((R, d), np.float64)
    mx = np.empty((R, d), np.float32)
    lib().or_pool_head(_p(X), d, _p(perm), R, cap, _p(avg), _p(mx))
    return avg, mx


def exp_constants() -> np.ndarray:
    out = np.empty(17, np.float64)
    lib().or_exp_constants(_p(out))
    return out


def exp_spec(x) -> np.ndarray:
    f = lib().or_exp
    x = np.asarray(x, dtype=np.float64)
    return np.array([f(float(v)) for v in x.reshape(-1)]).reshape(x.shape)


def draft_keys_head(qa, ka, qm, km, lam, want_A=False):
    qa = np.ascontiguousarray(qa, np.float64)
    ka = np.ascontiguousarray(ka, np.float64)
    qm = np.ascontiguousarray(qm, np.float32)
    km = np.ascontiguousarray(km, np.float32)
    R, d = qa.shape
    keys = np.empty((R, R), np.uint32)
    A = np.empty((R, R), np.float64) if want_A else None
    lib().or_draft_keys_head(_p(qa), _p(ka), _p(qm), _p(km), R, d, float(lam), _p(keys),
                             _p(A) if want_A else None)
    return (keys, A) if want_A else keys


def draft_logits_head(qa, ka, qm, km):
    qa = np.ascontiguousarray(qa, np.float64)
    ka = np.ascontiguousarray(ka, np.float64)
    qm = np.ascontiguousarray(qm, np.float32)
    km = np.ascontiguousarray(km, np.float32)
    R, d = qa.shape
    La = np.empty((R, R), np.float64)
    Lm = np.empty((R, R), np.float64)
    lib().or_draft_logits_head(_p(qa), _p(ka), _p(qm), _p(km), R, d, _p(La), _p(Lm))
    return La, Lm


def quotas3(n, full_bp, hi_bp, lo_bp):
    """Cumulative quotas (T16, T16 + T8, T16 + T8 + T4) of n pairs."""
    t16, t8c, tk = C.c_int64(), C.c_int64(), C.c_int64()
    lib().or_quotas(int(n), int(full_bp), int(hi_bp), int(lo_bp), C.byref(t16), C.byref(t8c),
                    C.byref(tk))
    return t16.value, t8c.value, tk.value


def quotas(n, hi_bp, lo_bp):
    """(T8, T8 + T4) with no 16-bit share."""
    _, t8, tk = quotas3(n, 0, hi_bp, lo_bp)
    return t8, tk


def rank_head(keys: np.ndarray, T8, Tk, scope=0, T16=0) -> np.ndarray:
    """Tiers of one head's [R,R] keys; T8 and Tk are cumulative counts
    (T16 + T8, T16 + T8 + T4)."""
    keys = np.ascontiguousarray(keys, np.uint32)
    R = keys.shape[0]
    tier = np.empty((R, R), np.uint8)
    lib().or_rank_head(_p(keys), R, int(scope), int(T16), int(T8), int(Tk), _p(tier))
    return tier


def plan(q, k, F, Hv, Wv, hi_bp, lo_bp, lam=0.2, scope=0, descriptors=False, full_bp=0,
         skip_means=False, cap=BLK):
    """Full plan for [B,H,N,d] inputs -> dict(keys [B,H,R,R] u32, tier u8, ...)
    over the R regions of block capacity cap.  full_bp: share of the 16-bit
    tier (basis points); skip_means: pairs outside the quotas become
    block-mean tiles (tier 1) instead of skipped (cap = 64 only)."""
    q = _u16(q)
    k = _u16(k)
    B, H, N, d = q.shape
    R = regions(F, Hv, Wv, cap)
    keys = np.empty((B, H, R, R), np.uint32)
    tier = np.empty((B, H, R, R), np.uint8)
    out = {"keys": keys, "tier": tier}
    ptrs = [None] * 4
    if descriptors:
        out["qavg"] = np.empty((B, H, R, d), np.float64)
        out["kavg"] = np.empty((B, H, R, d), np.float64)
        out["qmax"] = np.empty((B, H, R, d), np.float32)
        out["kmax"] = np.empty((B, H, R, d), np.float32)
        ptrs = [_p(out[n]) for n in ("qavg", "kavg", "qmax", "kmax")]
    rc = lib().or_plan(B, H, F, Hv, Wv, cap, d, _p(q), _p(k), int(full_bp), int(hi_bp), int(lo_bp), float(lam),
                       int(scope), int(bool(skip_means)), _p(keys), _p(tier), *ptrs)
    if rc:
        raise ValueError("bad shape")
    return out


# ---------------------------------------------------------------- formats
def bf16_round(x: float) -> float:
    return lib().or_bf16_round(float(x))


def e4m3_value(code: int) -> float:
    return lib().or_e4m3_value(int(code))


def e2m1_value(code: int) -> float:
    return lib().or_e2m1_value(int(code))


def e4m3_encode(x) -> np.ndarray:
    f = lib().or_e4m3_encode
    x = np.asarray(x, dtype=np.float64)
    return np.array([f(float(v)) for v in x.reshape(-1)], np.uint8).reshape(x.shape)


def e2m1_encode(x) -> np.ndarray:
    f = lib().or_e2m1_encode
    x = np.asarray(x, dtype=np.float64)
    return np.array([f(float(v)) for v in x.reshape(-1)], np.uint8).reshape(x.shape)


def mx_exponent(amax: float) -> int:
    return lib().or_mx_exponent(float(amax))


def mx_exponent_w(amax: float) -> int:
    """E8M0 exponent of a block of attention weights (no clipping)."""
    return lib().or_mx_exponent_w(float(amax))


def quant_qk(X, F, Hv, Wv, cap=BLK):
    """-> dict(c8 [B,H,Np,d] u8, s8 [B,H,T] f32, c4 [B,H,Np,d] u8, e4 [B,H,Np,d/32] u8),
    position axis in reordered order (Np = cap R, padding slots included; T =
    Np / 64 tiles)."""
    X = _u16(X)
    B, H, N, d = X.shape
    Np = regions(F, Hv, Wv, cap) * cap
    T = Np // BLK
    o = {"c8": np.empty((B, H, Np, d), np.uint8), "s8": np.empty((B, H, T), np.float32),
         "c4": np.empty((B, H, Np, d), np.uint8), "e4": np.empty((B, H, Np, d // 32), np.uint8)}
    assert lib().or_quant_qk(B, H, F, Hv, Wv, cap, d, _p(X), _p(o["c8"]), _p(o["s8"]), _p(o["c4"]),
                             _p(o["e4"])) == 0
    return o


def quant_v(X, F, Hv, Wv, cap=BLK):
    """-> dict(c8 [B,H,Np,d], s8 [B,H,d], c4 [B,H,Np,d], e4 [B,H,T,2,d])."""
    X = _u16(X)
    B, H, N, d = X.shape
    Np = regions(F, Hv, Wv, cap) * cap
    T = Np // BLK
    o = {"c8": np.empty((B, H, Np, d), np.uint8), "s8": np.empty((B, H, d), np.float32),
         "c4": np.empty((B, H, Np, d), np.uint8), "e4": np.empty((B, H, T, 2, d), np.uint8)}
    assert lib().or_quant_v(B, H, F, Hv, Wv, cap, d, _p(X), _p(o["c8"]), _p(o["s8"]), _p(o["c4"]),
                            _p(o["e4"])) == 0
    return o


# ---------------------------------------------------------------- attention
def _restore(x, F, Hv, Wv, cap=BLK):
    """[B,H,T,64,d] rows in reordered position order -> [B,H,N,d] in original
    token order (padding slots dropped)."""
    B, H = x.shape[:2]
    d = x.shape[-1]
    perm = layout(F, Hv, Wv, cap)
    keep = perm >= 0
    full = np.empty((B, H, F * Hv * Wv, d), np.float64)
    full[:, :, perm[keep], :] = x.reshape(B, H, -1, d)[:, :, keep]
    return full


def attention(q, k, v, tier, F, Hv, Wv, qblocks=None, amb=False, cap=BLK):
    """Tiered attention with a [B,H,R,R] tier map over the regions of block
    capacity cap.  qblocks=None: all rows, returned [B,H,N,d] in original
    token order.  Otherwise qblocks are query tiles (64 positions each) and
    the result is [B,H,len(qblocks),64,d]; row (j,i) is original token
    perm[qblocks[j]*64+i] (zero for a padding slot).  amb=True also
    returns, laid out alike, the bound on how far each output can move when
    every weight-code decision inside the precision band (OR_AMB_REL) is
    taken either way: (out, amb)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    tier = np.ascontiguousarray(tier, np.uint8)
    B, H, N, d = q.shape
    R = regions(F, Hv, Wv, cap)
    assert tier.shape == (B, H, R, R)
    qb = None if qblocks is None else np.ascontiguousarray(qblocks, np.int32)
    nq = R * cap // BLK if qb is None else len(qb)
    out = np.empty((B, H, nq, BLK, d), np.float64)
    ab = np.empty((B, H, nq, BLK, d), np.float64) if amb else None
    rc = lib().or_attention(B, H, F, Hv, Wv, cap, d, _p(q), _p(k), _p(v), _p(tier), nq,
                            None if qb is None else _p(qb), _p(out), None if ab is None else _p(ab))
    if rc:
        raise ValueError("attention: bad shape or tier map")
    if qb is None:
        out = _restore(out, F, Hv, Wv, cap)
        ab = None if ab is None else _restore(ab, F, Hv, Wv, cap)
    return (out, ab) if amb else out


def _pfx_args(q, k, v, tier, qp, kp, vp, valid, qblocks, cap):
    q, k, v, qp, kp, vp = (_u16(x) for x in (q, k, v, qp, kp, vp))
    tier = np.ascontiguousarray(tier, np.uint8)
    B, H, N, d = q.shape
    Lp = qp.shape[2]
    assert qp.shape == kp.shape == vp.shape == (B, H, Lp, d)
    R = tier.shape[2]
    assert tier.shape == (B, H, R, R)
    va = None if valid is None else np.ascontiguousarray(valid, np.int32)
    assert va is None or va.shape == (B,)
    qb = None if qblocks is None else np.ascontiguousarray(qblocks, np.int32)
    nq = R * cap // BLK if qb is None else len(qb)
    return q, k, v, tier, qp, kp, vp, va, qb, nq, (B, H, N, d, Lp, R)


def _prows(prefix_rows, Lp):
    """prefix_rows: True (all Lp rows), False (none) or row indices."""
    if prefix_rows is True:
        return Lp, None
    if prefix_rows is False or prefix_rows is None:
        return 0, None
    pr = np.ascontiguousarray(prefix_rows, np.int32)
    assert ((pr >= 0) & (pr < Lp)).all()
    return len(pr), pr


def attention_pfx(q, k, v, tier, F, Hv, Wv, qp, kp, vp, valid=None, pt=16, qblocks=None,
                  prefix_rows=True, amb=False, cap=BLK):
    """Tiered attention with a text prefix (App. C.1).  q, k, v: video
    [B,H,N,d]; qp, kp, vp: prefix [B,H,Lp,d]; valid: [B] valid prefix keys
    (None: all).  pt: precision of the prefix interactions (16 or 32).
    prefix_rows: True (all), False (none) or the prefix query rows wanted.
    Returns (video rows laid out as attention(), prefix rows [B,H,np,d] or
    None), and with amb=True also the video rows' band bound (prefix rows
    take only unquantized weights)."""
    q, k, v, tier, qp, kp, vp, va, qb, nq, (B, H, N, d, Lp, R) = _pfx_args(
        q, k, v, tier, qp, kp, vp, valid, qblocks, cap)
    npr, pr = _prows(prefix_rows, Lp)
    out = np.empty((B, H, nq, BLK, d), np.float64)
    outp = np.empty((B, H, npr, d), np.float64) if prefix_rows is not False else None
    ab = np.empty((B, H, nq, BLK, d), np.float64) if amb else None
    rc = lib().or_attention_pfx(B, H, F, Hv, Wv, cap, d, _p(q), _p(k), _p(v), Lp, _p(qp), _p(kp),
                                _p(vp), None if va is None else _p(va), pt, _p(tier), nq,
                                None if qb is None else _p(qb), npr,
                                None if pr is None else _p(pr), _p(out),
                                None if outp is None else _p(outp),
                                None if ab is None else _p(ab))
    assert rc == 0
    if qblocks is None:
        out = _restore(out, F, Hv, Wv, cap)
        ab = None if ab is None else _restore(ab, F, Hv, Wv, cap)
    return (out, outp, ab) if amb else (out, outp)


def attention_trace(q, k, v, tier, F, Hv, Wv, u, maxn=None, cap=BLK):
    """One head ([N,d] inputs, [R,R] tier over the regions of capacity cap),
    one reordered query position u."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    tier = np.ascontiguousarray(tier, np.uint8)
    N, d = q.shape
    if maxn is None:
        maxn = N + 64
    key = np.empty(maxn, np.int32)
    tt = np.empty(maxn, np.int32)
    s, w, wq, m = (np.empty(maxn, np.float64) for _ in range(4))
    Z = C.c_double()
    out = np.empty(d, np.float64)
    n = lib().or_attention_trace(F, Hv, Wv, cap, d, _p(q), _p(k), _p(v), _p(tier), int(u), maxn,
                                 _p(key), _p(tt), _p(s), _p(w), _p(wq), _p(m), C.byref(Z),
                                 _p(out))
    n = min(n, maxn)
    return {"key": key[:n], "tier": tt[:n], "s": s[:n], "w": w[:n], "wq": wq[:n], "m": m[:n],
            "Z": Z.value, "out": out}


def dense(q, k, v, rows):
    """fp64 softmax attention over all keys for original-order rows -> [B,H,len,d]."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, H, N, d = q.shape
    rows = np.ascontiguousarray(rows, np.int32)
    out = np.empty((B, H, len(rows), d), np.float64)
    lib().or_dense(B, H, N, d, _p(q), _p(k), _p(v), len(rows), _p(rows), _p(out))
    return out
