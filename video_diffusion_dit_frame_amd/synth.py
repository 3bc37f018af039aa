"""Seeded synthetic inputs shaped like video-DiT attention layers.

This module is the only code shared by the HIP path's tests/benchmark and the
CPU oracle's tests.  It draws random tensors and holds none of the method's
arithmetic.

Recipe (the pages give no activation statistics, so these are this
project's choices, stated once here and in the design notes):

* generator: numpy ``Generator(PCG64(seed))``; tensors are drawn per
  (batch, head) in order, Q then K then V;
* base: ``X = z + a * phi`` with ``z ~ N(0, 1)`` and ``a = 1.0``;
* smooth per-frame field: ``phi(f, y, x) = sum_m cos(2 pi (kt f/F + ky y/H
  + kx x/W) + ph_m) * u_m`` over 8 wave vectors drawn without replacement
  from ``{0,1} x {0,1,2}^2`` minus the zero vector, ``ph_m ~ U[0, 2 pi)``,
  ``u_m ~ N(0, I_d) * sqrt(2/8)``; Q and K share one field per (b, h) so the
  attention has local structure, V has its own;
* outliers (``outliers=True``): 4 channels per (b, h) chosen without
  replacement; Q is multiplied by 4 there, K gets +8 (a constant channel
  offset), V is multiplied by 4;
* the fp32 result is rounded to bfloat16 (round to nearest even).

Tensors come back as ``uint16`` bit patterns of bfloat16, shape
``[B, H, N, d]`` with tokens in (frame, y, x) raster order.
"""
from __future__ import annotations

import numpy as np

A_SMOOTH = 1.0
N_WAVES = 8
N_OUTLIERS = 4


def _wave_vectors():
    return [(kt, ky, kx) for kt in (0, 1) for ky in (0, 1, 2) for kx in (0, 1, 2)
            if (kt, ky, kx) != (0, 0, 0)]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even), returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _field(rng, F, Hv, Wv, d, grid):
    waves = _wave_vectors()
    pick = rng.choice(len(waves), size=N_WAVES, replace=False)
    ph = rng.uniform(0.0, 2.0 * np.pi, size=N_WAVES)
    u = rng.standard_normal((N_WAVES, d), dtype=np.float32) * np.float32(np.sqrt(2.0 / N_WAVES))
    f, y, x = grid
    cosv = np.empty((F * Hv * Wv, N_WAVES), dtype=np.float32)
    for m, w in enumerate(pick):
        kt, ky, kx = waves[w]
        arg = 2.0 * np.pi * (kt * f / F + ky * y / Hv + kx * x / Wv) + ph[m]
        cosv[:, m] = np.cos(arg).astype(np.float32).reshape(-1)
    return cosv @ u


def make_qkv(B, H, F, Hv, Wv, d, seed, outliers=True):
    """Return (q, k, v) as uint16 bfloat16 bits, each [B, H, N, d]."""
    N = F * Hv * Wv
    rng = np.random.Generator(np.random.PCG64(seed))
    grid = np.meshgrid(np.arange(F, dtype=np.float64), np.arange(Hv, dtype=np.float64),
                       np.arange(Wv, dtype=np.float64), indexing="ij")
    out = [np.empty((B, H, N, d), dtype=np.uint16) for _ in range(3)]
    a = np.float32(A_SMOOTH)
    for b in range(B):
        for h in range(H):
            phi_qk = _field(rng, F, Hv, Wv, d, grid)
            phi_v = _field(rng, F, Hv, Wv, d, grid)
            ch = rng.choice(d, size=N_OUTLIERS, replace=False) if outliers else None
            for t in range(3):
                z = rng.standard_normal((N, d), dtype=np.float32)
                z += a * (phi_v if t == 2 else phi_qk)
                if ch is not None:
                    if t == 0:
                        z[:, ch] *= np.float32(4.0)
                    elif t == 1:
                        z[:, ch] += np.float32(8.0)
                    else:
                        z[:, ch] *= np.float32(4.0)
                out[t][b, h] = f32_to_bf16_bits(z)
    return tuple(out)


def make_prefix(B, H, Lp, d, seed):
    """Text-prefix tokens for joint text-video attention, (qp, kp, vp) as
    uint16 bfloat16 bits, each [B, H, Lp, d].

    Recipe: generator ``Generator(PCG64(seed))``; per (batch, head) one
    shared direction ``mu ~ N(0, I_d)`` (text tokens of one prompt cluster),
    then ``Q = z + mu``, ``K = z + mu``, ``V = z`` with fresh ``z ~ N(0, 1)``
    per tensor, rounded to bfloat16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = [np.empty((B, H, Lp, d), dtype=np.uint16) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            mu = rng.standard_normal(d, dtype=np.float32)
            for t in range(3):
                z = rng.standard_normal((Lp, d), dtype=np.float32)
                if t < 2:
                    z += mu
                out[t][b, h] = f32_to_bf16_bits(z)
    return tuple(out)


def prefix_valid(B, Lp, seed):
    """Valid prefix lengths per batch element (prompt lengths before the
    padding), uniform in [1, Lp]; int32 [B]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(1, Lp + 1, size=B).astype(np.int32)
