"""Pins of the oracle's ragged spatial partition (CPU; DraftAttention2 Sec. 3.3:
a ragged 2D partition of each frame with balanced token counts, the smallest
total perimeter among candidate partitions, the minimum number of blocks and
less than one block of padding per frame; App. C.2: R_f = ceil(H_v W_v / C);
App. C.1: n_a counts valid tokens and excludes padding).

* frames with sides multiple of 8: the partition is the 8x8 grid with raster
  slots, the layout the rest of the suite pins;
* every ragged frame: every token in exactly one region, R_f regions, each
  connected, 48..64 valid tokens, valid slots first in raster order, less
  than 64 padding slots in all;
* the reported perimeter equals a recount from the slot table, and no
  candidate of the family (every band composition of either orientation,
  enumerated exhaustively on small frames) beats it; the chosen one follows
  the stated tie order;
* pooled descriptors average and maximise over the valid tokens only;
  quantized operands hold zero codes in padding slots and per-block scales
  from the valid tokens;
* attention over a ragged layout: the full tier everywhere equals dense
  softmax attention over all tokens, and with skipped region pairs it
  equals brute-force masked attention.
"""
import itertools
import math

import numpy as np
import pytest

from video_diffusion_dit_frame_amd import synth
from video_diffusion_dit_frame_amd.synth import bf16_bits_to_f32
from tests.test_oracle_attention import dense_np

RAGGED = [(84, 48), (60, 60), (12, 16), (34, 60), (45, 80), (30, 44), (20, 28), (17, 31),
          (9, 100), (7, 7), (8, 6), (13, 40), (40, 13)]


def f64(x):
    return bf16_bits_to_f32(x).astype(np.float64)


def region_map(tok, Hv, Wv):
    reg = np.full(Hv * Wv, -1, np.int64)
    for r in range(tok.shape[0]):
        for t in tok[r]:
            if t >= 0:
                assert reg[t] == -1
                reg[t] = r
    return reg.reshape(Hv, Wv)


def perimeter(reg):
    """Edges between a cell and a cell of another region or the border."""
    Hv, Wv = reg.shape
    pad = np.full((Hv + 2, Wv + 2), -2, np.int64)
    pad[1:-1, 1:-1] = reg
    c = pad[1:-1, 1:-1]
    return int(sum((c != pad[1 + dy:Hv + 1 + dy, 1 + dx:Wv + 1 + dx]).sum()
                   for dy, dx in ((-1, 0), (1, 0), (0, -1), (0, 1))))


@pytest.mark.parametrize("Hv,Wv", [(8, 8), (16, 24), (48, 80), (24, 40), (64, 72), (32, 48)])
def test_multiple_of_8_is_the_grid(orc, Hv, Wv):
    tok, nv = orc.partition(Hv, Wv)
    Ry, Rx = Hv // 8, Wv // 8
    want = np.empty((Ry * Rx, 64), np.int32)
    for ry in range(Ry):
        for rx in range(Rx):
            for i in range(64):
                want[ry * Rx + rx, i] = (8 * ry + i // 8) * Wv + 8 * rx + i % 8
    assert np.array_equal(tok, want) and (nv == 64).all()
    o, bands, per = orc.partition_bands(Hv, Wv)
    assert o == 0 and (bands == 8).all() and per == 32 * Ry * Rx


@pytest.mark.parametrize("Hv,Wv", RAGGED)
def test_partition_properties(orc, Hv, Wv):
    tok, nv = orc.partition(Hv, Wv)
    Rf = math.ceil(Hv * Wv / 64)
    assert tok.shape == (Rf, 64)
    reg = region_map(tok, Hv, Wv)
    assert (reg >= 0).all()                                   # every token once
    assert (nv >= 48).all() and (nv <= 64).all()
    assert Rf * 64 - Hv * Wv < 64                             # under one block of padding
    assert nv.max() - nv.min() <= 16
    for r in range(Rf):
        cells = tok[r, :nv[r]]
        assert (cells >= 0).all() and (tok[r, nv[r]:] == -1).all()
        assert (np.diff(cells) > 0).all()                     # raster order
        # connected: flood fill over 4-neighbours inside the region
        inside = set(int(c) for c in cells)
        seen, stack = {int(cells[0])}, [int(cells[0])]
        while stack:
            c = stack.pop()
            y, x = divmod(c, Wv)
            for ny, nx in ((y - 1, x), (y + 1, x), (y, x - 1), (y, x + 1)):
                n = ny * Wv + nx
                if 0 <= ny < Hv and 0 <= nx < Wv and n in inside and n not in seen:
                    seen.add(n)
                    stack.append(n)
        assert len(seen) == nv[r], (r, len(seen), nv[r])
    o, bands, per = orc.partition_bands(Hv, Wv)
    assert per == perimeter(reg)
    assert bands.sum() == (Hv if o == 0 else Wv)


def _candidate(Hv, Wv, orient, hs):
    """Region map of one candidate: bands hs of rows (orient 0) or columns,
    each walked as a column snake and cut into ceil(hL/64) balanced pieces.
    None when a piece is under 48 tokens."""
    E, L = (Hv, Wv) if orient == 0 else (Wv, Hv)
    reg = np.empty((E, L), np.int64)
    base, line0 = 0, 0
    for h in hs:
        n = h * L
        k = -(-n // 64)
        q, rem = divmod(n, k)
        if q < 48:
            return None
        order = [(line0 + (t if col % 2 == 0 else h - 1 - t), col) for col in range(L) for t in range(h)]
        sizes = [q + 1] * rem + [q] * (k - rem)
        it = iter(order)
        for p, sz in enumerate(sizes):
            for _ in range(sz):
                reg[next(it)] = base + p
        base += k
        line0 += h
    return reg if orient == 0 else reg.T


def _compositions(E):
    for cuts in itertools.product((0, 1), repeat=E - 1):
        hs, h = [], 1
        for c in cuts:
            if c:
                hs.append(h)
                h = 1
            else:
                h += 1
        hs.append(h)
        yield hs


@pytest.mark.parametrize("Hv,Wv", [(9, 12), (12, 9), (10, 13), (11, 14), (13, 11), (8, 14), (14, 10),
                                   (7, 16), (15, 13), (16, 7), (6, 16)])
def test_partition_is_the_best_candidate(orc, Hv, Wv):
    """Exhaustive search over every band composition of both orientations."""
    Rf = math.ceil(Hv * Wv / 64)
    best = None
    for orient in (0, 1):
        E = Hv if orient == 0 else Wv
        for hs in _compositions(E):
            reg = _candidate(Hv, Wv, orient, hs)
            if reg is None or reg.max() + 1 != Rf:
                continue
            key = (perimeter(reg), orient, len(hs), hs)
            if best is None or key < best[0]:
                best = (key, reg)
    if best is None:
        with pytest.raises(ValueError):
            orc.partition(Hv, Wv)
        return
    tok, _ = orc.partition(Hv, Wv)
    got = region_map(tok, Hv, Wv)
    assert np.array_equal(got, best[1]), best[0]


@pytest.mark.parametrize("Hv,Wv", [(20, 28), (17, 31)])
def test_pooling_and_quantization_over_valid_tokens(orc, Hv, Wv):
    F, d = 2, 64
    q, _, _ = synth.make_qkv(1, 1, F, Hv, Wv, d, 5, True)
    X = f64(q[0, 0])
    perm = orc.layout(F, Hv, Wv)
    R = perm.size // 64
    avg, mx = orc.pool_head(q[0, 0], F, Hv, Wv)
    qq = orc.quant_qk(q, F, Hv, Wv)
    for a in range(R):
        valid = perm[a * 64:(a + 1) * 64]
        valid = valid[valid >= 0]
        G = X[valid]
        assert np.array_equal(avg[a], G.sum(axis=0) / len(valid))
        assert np.array_equal(mx[a], G.max(axis=0).astype(np.float32))
        amax = np.float32(np.abs(G).max())
        assert qq["s8"][0, 0, a] == np.float32(amax / np.float32(448.0))
        pad = slice(a * 64 + len(valid), (a + 1) * 64)
        assert (qq["c8"][0, 0, pad] == 0).all() and (qq["c4"][0, 0, pad] == 0).all()


@pytest.mark.parametrize("Hv,Wv", [(20, 28), (17, 31)])
def test_attention_on_ragged_layout(orc, Hv, Wv):
    F, d = 2, 64
    q, k, v = synth.make_qkv(1, 2, F, Hv, Wv, d, 6, True)
    R = orc.regions(F, Hv, Wv)
    full = np.full((1, 2, R, R), 32, np.uint8)
    out = orc.attention(q, k, v, full, F, Hv, Wv)
    for h in range(2):
        ref, _ = dense_np(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]))
        assert np.abs(out[0, h] - ref).max() <= 1e-12
    rng = np.random.default_rng(1)
    tier = np.where(rng.random((1, 2, R, R)) < 0.5, 32, 0).astype(np.uint8)
    out = orc.attention(q, k, v, tier, F, Hv, Wv)
    perm = orc.layout(F, Hv, Wv)
    blk = np.empty(F * Hv * Wv, np.int64)
    blk[perm[perm >= 0]] = np.nonzero(perm >= 0)[0] // 64
    for h in range(2):
        mask = tier[0, h][blk[:, None], blk[None, :]] > 0
        ref, _ = dense_np(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), mask)
        assert np.abs(out[0, h] - ref).max() <= 1e-12
    # kernel-precision decisions on the same layout stay close to fp64 ones
    t3 = rng.choice(np.array([0, 4, 8, 16], np.uint8), size=(1, 2, R, R))
    ex = orc.attention(q, k, v, t3, F, Hv, Wv)
    kp, al = orc.attention_kp(q, k, v, t3, F, Hv, Wv)
    assert (al >= 0).all()
    assert np.linalg.norm(kp - ex) / np.linalg.norm(ex) <= 3e-3
