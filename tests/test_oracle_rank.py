"""Pins of the oracle's quotas and ranking (CPU)."""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_quotas_golden(orc):
    with open(os.path.join(GOLDEN, "quotas.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        n = case["R"] ** 2
        T8, Tk = orc.quotas(n, case["hi_bp"], case["lo_bp"])
        assert (T8, Tk - T8) == (case["T8"], case["T4"]), case


def test_quotas_round_half_up(orc):
    # 1 bp of 5000 pairs is 0.5 -> rounds up; of 4999 pairs 0.4999 -> down
    assert orc.quotas(5000, 1, 0) == (1, 1)
    assert orc.quotas(4999, 1, 0) == (0, 0)
    assert orc.quotas(7, 10000, 0) == (7, 7)
    assert orc.quotas(7, 0, 0) == (0, 0)


def brute_rank(keys, T8, Tk, scope):
    R = keys.shape[0]
    tier = np.zeros((R, R), np.uint8)
    if scope == 0:
        flat = keys.reshape(-1).astype(np.int64)
        order = np.lexsort((np.arange(flat.size), -flat))  # key desc, index asc
        t = np.zeros(flat.size, np.uint8)
        t[order[:Tk]] = 4
        t[order[:T8]] = 8
        return t.reshape(R, R)
    for a in range(R):
        row = keys[a].astype(np.int64)
        order = np.lexsort((np.arange(R), -row))
        tier[a, order[:Tk]] = 4
        tier[a, order[:T8]] = 8
    return tier


@pytest.mark.parametrize("scope", [0, 1])
@pytest.mark.parametrize("R,levels", [(16, 5), (37, 1000), (64, 2), (50, 2**31)])
def test_rank_matches_lexsort(orc, scope, R, levels):
    rng = np.random.default_rng(R * 7 + levels % 97 + scope)
    keys = rng.integers(0, levels, size=(R, R)).astype(np.uint32) + np.uint32(0x30000000)
    n = R * R if scope == 0 else R
    for hi, lo in [(1000, 3000), (2500, 2500), (0, 6000), (10000, 0), (0, 0), (1, 1)]:
        T8, Tk = orc.quotas(n, hi, lo)
        got = orc.rank_head(keys, T8, Tk, scope)
        assert np.array_equal(got, brute_rank(keys, T8, Tk, scope)), (hi, lo)
        cnt = lambda t: (got == t).sum() if scope == 0 else (got == t).sum(axis=1)
        assert np.all(cnt(8) == T8) and np.all(cnt(4) == Tk - T8)


def test_rank_all_equal_keys_follow_index(orc):
    R = 12
    keys = np.full((R, R), 0x3C000000, np.uint32)
    T8, Tk = orc.quotas(R * R, 1000, 3000)
    t = orc.rank_head(keys, T8, Tk, 0).reshape(-1)
    assert (t[:T8] == 8).all() and (t[T8:Tk] == 4).all() and (t[Tk:] == 0).all()


def test_rank_head_equals_row_when_single_region(orc):
    keys = np.array([[0x3F800000]], np.uint32)
    for hi, lo in [(10000, 0), (0, 10000), (0, 0), (4000, 4000)]:
        T8, Tk = orc.quotas(1, hi, lo)
        assert np.array_equal(orc.rank_head(keys, T8, Tk, 0), orc.rank_head(keys, T8, Tk, 1))


def test_rank_larger_scores_get_higher_precision(orc):
    """Sec. 3.2: higher precision to larger draft mass, skip for the rest."""
    rng = np.random.default_rng(3)
    R = 40
    A = rng.dirichlet(np.ones(R), size=R).astype(np.float32)
    keys = A.view(np.uint32)
    T8, Tk = orc.quotas(R * R, 1000, 3000)
    t = orc.rank_head(keys, T8, Tk, 0)
    assert A[t == 8].min() >= A[t == 4].max()
    assert A[t == 4].min() >= A[t == 0].max()


@pytest.mark.parametrize("scope", [0, 1])
def test_rank_three_tiers_matches_lexsort(orc, scope):
    """16-bit, FP8 and MXFP4 tiers from one ranking: the T16 largest keys
    (ties by ascending index) get 16, the next T8 get 8, the next T4 get 4."""
    rng = np.random.default_rng(11 + scope)
    R = 24
    keys = rng.integers(0, 40, size=(R, R)).astype(np.uint32)  # many ties
    n = R * R if scope == 0 else R
    T16, T8c, Tk = orc.quotas3(n, 1200, 2000, 3500)
    got = orc.rank_head(keys, T8c, Tk, scope, T16=T16)
    rows = [np.arange(R * R)] if scope == 0 else [a * R + np.arange(R) for a in range(R)]
    want = np.zeros(R * R, np.uint8)
    for idx in rows:
        k = keys.reshape(-1)[idx]
        order = idx[np.lexsort((idx, -k.astype(np.int64)))]
        want[order[:T16]] = 16
        want[order[T16:T8c]] = 8
        want[order[T8c:Tk]] = 4
    assert np.array_equal(got.reshape(-1), want)
    assert (got == 16).sum() == (T16 if scope == 0 else R * T16)


def test_quotas_three_levels_pages_allocations(orc):
    """Allocations the pages report (shares of 0/4/8/16-bit tiles): 85/0/7.5/7.5
    and 13.4/64.9/21.6/0, on maps where the shares are whole pair counts."""
    # 7.5% 16-bit, 7.5% 8-bit, no 4-bit, 85% skipped; R = 1260 (R^2 * 0.075 = 119070)
    assert orc.quotas3(1260 * 1260, 750, 750, 0) == (119070, 238140, 238140)
    # 0% 16-bit, 21.6% 8-bit, 64.9% 4-bit, 13.4% skipped; R = 100
    assert orc.quotas3(100 * 100, 0, 2160, 6490) == (0, 2160, 8650)
