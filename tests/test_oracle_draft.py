"""Pins of the oracle's layout, pooling, exp and draft map (CPU)."""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from video_diffusion_dit_frame_amd import synth
from video_diffusion_dit_frame_amd.synth import bf16_bits_to_f32


# ------------------------------------------------------------------ layout
@pytest.mark.parametrize("F,Hv,Wv", [(1, 8, 8), (4, 16, 16), (3, 24, 40), (2, 48, 80)])
def test_layout_regions_are_8x8_squares(orc, F, Hv, Wv):
    perm = orc.layout(F, Hv, Wv)
    N = F * Hv * Wv
    assert np.array_equal(np.sort(perm), np.arange(N))
    f, rem = np.divmod(perm, Hv * Wv)
    y, x = np.divmod(rem, Wv)
    R = N // 64
    f, y, x = (t.reshape(R, 64) for t in (f, y, x))
    # one frame per region, one 8x8 cell of the grid, all 64 offsets in raster order
    assert (f == f[:, :1]).all()
    assert (y // 8 == y[:, :1] // 8).all() and (x // 8 == x[:, :1] // 8).all()
    assert np.array_equal((y % 8) * 8 + (x % 8), np.tile(np.arange(64), (R, 1)))
    # regions frame-major, then raster over the 8x8 grid
    cell = (f[:, 0] * (Hv // 8) + y[:, 0] // 8) * (Wv // 8) + x[:, 0] // 8
    assert np.array_equal(cell, np.arange(R))


def test_layout_restore_inverts_reorder(orc):
    perm = orc.layout(3, 16, 24)
    X = np.random.default_rng(0).normal(size=(perm.size, 5))
    reordered = X[perm]
    restored = np.empty_like(X)
    restored[perm] = reordered
    assert np.array_equal(restored, X)


def test_small_frame_is_one_region(orc):
    """A frame of fewer than 64 tokens is one region (R_f = 1) holding all of
    them in raster order, the remaining slots padding (5 x 7 = 35 tokens)."""
    perm = orc.layout(2, 5, 7)
    assert perm.size == 2 * 64
    for f in range(2):
        blk = perm[64 * f:64 * f + 64]
        assert np.array_equal(blk[:35], 35 * f + np.arange(35)) and (blk[35:] == -1).all()


# ------------------------------------------------------------------ pooling
def _head(F=2, Hv=16, Wv=24, d=64, seed=3, outliers=True):
    q, k, v = synth.make_qkv(1, 1, F, Hv, Wv, d, seed, outliers)
    return q[0, 0], k[0, 0], v[0, 0]


def test_pool_brute_force(orc):
    F, Hv, Wv = 2, 16, 24
    q, _, _ = _head(F, Hv, Wv)
    avg, mx = orc.pool_head(q, F, Hv, Wv)
    X = bf16_bits_to_f32(q).astype(np.float64)
    perm = orc.layout(F, Hv, Wv)
    G = X[perm].reshape(-1, 64, X.shape[1])
    # sums of 64 bf16 values are exact in fp64, so numpy's pairwise mean agrees bit for bit
    assert np.array_equal(avg, G.mean(axis=1))
    assert np.array_equal(mx, G.max(axis=1).astype(np.float32))


def test_pool_constant_region(orc):
    F, Hv, Wv, d = 1, 8, 16, 32
    X = np.full((F * Hv * Wv, d), 0x3FC0, np.uint16)  # 1.5 everywhere
    avg, mx = orc.pool_head(X, F, Hv, Wv)
    assert (avg == 1.5).all() and (mx == 1.5).all()


def test_pool_bilinearity(orc):
    """Eq. (1)-(2): avgQ_a . avgK_b / sqrt(d) is the mean token logit of the
    64x64 pair block."""
    F, Hv, Wv = 1, 16, 16
    q, k, _ = _head(F, Hv, Wv)
    qa, _ = orc.pool_head(q, F, Hv, Wv)
    ka, _ = orc.pool_head(k, F, Hv, Wv)
    perm = orc.layout(F, Hv, Wv)
    Q = bf16_bits_to_f32(q).astype(np.float64)[perm].reshape(-1, 64, q.shape[1])
    K = bf16_bits_to_f32(k).astype(np.float64)[perm].reshape(-1, 64, k.shape[1])
    for a in range(Q.shape[0]):
        for b in range(K.shape[0]):
            mean_logit = (Q[a] @ K[b].T).mean()
            assert abs(qa[a] @ ka[b] - mean_logit) <= 1e-12 * max(1.0, abs(mean_logit))


# ------------------------------------------------------------------ exp
def test_exp_constants_from_exact_values(orc):
    getcontext().prec = 60
    ln2 = Decimal(2).ln()
    c = orc.exp_constants()
    hi, lo, inv = c[0], c[1], c[2]
    # head has at most 32 significant bits so k*hi is exact for |k| < 2^21
    m, e = math.frexp(hi)
    assert (Fraction(m) * 2 ** 32).denominator == 1
    assert abs(Decimal(hi) + Decimal(lo) - ln2) < Decimal(2) ** -85
    assert inv == float(1 / ln2)
    for j in range(14):
        assert c[3 + j] == float(Fraction(1, math.factorial(j)))


def test_exp_spec_vs_libm(orc):
    x = np.concatenate([np.linspace(-708.0, 0.0, 60001), -np.logspace(-12, 2.8, 20000),
                        [0.0, -1e-300, -0.5 * math.log(2), -708.0]])
    got = orc.exp_spec(x)
    want = np.exp(x)
    ulp = np.spacing(want)
    assert (np.abs(got - want) <= 1.0 * ulp).all()
    assert orc.exp_spec([-708.0001, -800.0, -1e308]).tolist() == [0.0, 0.0, 0.0]


# ------------------------------------------------------------------ draft map
def _descs(F=2, Hv=16, Wv=16, d=64, seed=9):
    q, k, _ = _head(F, Hv, Wv, d, seed)
    qa, qm = orc_pool(q, F, Hv, Wv)
    ka, km = orc_pool(k, F, Hv, Wv)
    return qa, ka, qm, km


def orc_pool(x, F, Hv, Wv):
    from oracle import oracle

    return oracle.pool_head(x, F, Hv, Wv)


@pytest.mark.parametrize("lam", [0.0, 0.2, 0.7, 1.0])
def test_draft_map_is_mixture_of_row_softmaxes(orc, lam):
    qa, ka, qm, km = _descs()
    d = qa.shape[1]
    keys, A = orc.draft_keys_head(qa, ka, qm, km, lam, want_A=True)
    pa = scipy.special.softmax(qa @ ka.T / math.sqrt(d), axis=1)
    pm = scipy.special.softmax(qm.astype(np.float64) @ km.astype(np.float64).T / math.sqrt(d), axis=1)
    want = (1 - lam) * pa + lam * pm
    assert np.allclose(A, want, rtol=1e-13, atol=1e-300)
    R = A.shape[0]
    assert np.all(np.abs(A.sum(axis=1) - 1.0) <= R * 2.0 ** -52)
    # key = bits of fp32(A)
    assert np.array_equal(keys, A.astype(np.float32).view(np.uint32))
    if lam == 0.0:
        assert np.allclose(A, pa, rtol=1e-13)
    if lam == 1.0:
        assert np.allclose(A, pm, rtol=1e-13)


def test_draft_keys_order_like_scores(orc):
    """Positive floats order like their bit patterns, so ranking keys compare
    as the fp32 scores do."""
    qa, ka, qm, km = _descs(seed=11)
    keys, A = orc.draft_keys_head(qa, ka, qm, km, 0.2, want_A=True)
    f = A.astype(np.float32).reshape(-1)
    kk = keys.reshape(-1)
    o1 = np.argsort(f, kind="stable")
    o2 = np.argsort(kk, kind="stable")
    assert np.array_equal(f[o1], f[o2])


def _fma(x, y, z):
    """Correctly rounded fused multiply-add via exact rationals."""
    return float(Fraction(x) * Fraction(y) + Fraction(z))


def test_draft_keys_bitwise_reference(orc):
    """Keys re-derived step by step in Python doubles (exact fma through
    rationals, sequential sums, IEEE division), pinning the fixed evaluation
    order the GPU must reproduce bit for bit."""
    F_, Hv, Wv, d = 1, 16, 32, 64
    q, k, _ = _head(F_, Hv, Wv, d, 5)
    qa, qm = orc.pool_head(q, F_, Hv, Wv)
    ka, km = orc.pool_head(k, F_, Hv, Wv)
    lam = 0.2
    keys = orc.draft_keys_head(qa, ka, qm, km, lam)
    La, Lm = orc.draft_logits_head(qa, ka, qm, km)
    R = qa.shape[0]
    inv_sqrt_d = 1.0 / math.sqrt(d)

    def probs(X, Y, a, Lo):
        L = []
        for b in range(R):
            acc = 0.0
            for c in range(d):
                acc = _fma(float(X[a, c]), float(Y[b, c]), acc)
            L.append(acc * inv_sqrt_d)
        assert np.array_equal(np.array(L), Lo[a])
        m = max(L)
        e = [float(orc.exp_spec([x - m])[0]) for x in L]
        Z = 0.0
        for x in e:
            Z += x
        return [x / Z for x in e]

    for a in range(R):
        pa = probs(qa, ka, a, La)
        pm = probs(qm.astype(np.float64), km.astype(np.float64), a, Lm)
        A = [(1.0 - lam) * x + lam * y for x, y in zip(pa, pm)]
        want = np.array(A, np.float64).astype(np.float32).view(np.uint32)
        assert np.array_equal(keys[a], want), a


def test_draft_logits_fma_order_full_mantissas(orc):
    """With 53-bit descriptors the products are inexact, so this separates a
    fused chain from separate multiply/add or any other summation order."""
    rng = np.random.default_rng(17)
    R, d = 6, 64
    qa, ka = rng.normal(size=(R, d)), rng.normal(size=(R, d))
    qm, km = rng.normal(size=(R, d)).astype(np.float32), rng.normal(size=(R, d)).astype(np.float32)
    La, _ = orc.draft_logits_head(qa, ka, qm, km)
    inv_sqrt_d = 1.0 / math.sqrt(d)
    for a in range(R):
        for b in range(R):
            acc = 0.0
            for c in range(d):
                acc = _fma(float(qa[a, c]), float(ka[b, c]), acc)
            assert La[a, b] == acc * inv_sqrt_d
