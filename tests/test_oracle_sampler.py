"""Pins of the oracle's sampler (阶段四 4.3 采样): closed forms on small
vocabularies, the roulette as an interval lookup over prefix sums,
temperature -> 0 and top_p -> 0 limits."""
import math

import numpy as np
import pytest

import oracle
from oracle.sampler import sample, nucleus, argmax


def _page_roulette(probs, kept, u):
    """The roulette of 阶段四 4.3 (采样), stated as an interval lookup: kept
    token i owns the interval (C_{i-1}, C_i] of the running kept mass C (in
    vocabulary order), and the draw r = u * C_last falls in exactly one of
    them.  Bisection over the prefix sums finds the first kept token whose
    running sum reaches r; a rounding overshoot past the total picks the
    last kept token."""
    kept_idx = np.nonzero(np.asarray(kept, dtype=bool))[0]
    c = np.cumsum(np.asarray(probs, dtype=np.float64)[kept_idx])
    j = int(np.searchsorted(c, u * c[-1], side="left"))
    return int(kept_idx[min(j, kept_idx.size - 1)])


def test_argmax_first_index():
    assert argmax([1.0, 3.0, 3.0, 2.0]) == 1
    assert sample([1.0, 3.0, 3.0], 0.0, 0.9, 0.7)["token"] == 1


def test_closed_form_no_top_p():
    # weights proportional to 1, 2, 3 at temperature 1: boundaries at 1/6, 3/6
    l = np.log([1.0, 2.0, 3.0])
    for u, want in ((0.0, 0), (0.1, 0), (0.16, 0), (0.17, 1), (0.49, 1), (0.51, 2), (0.999, 2)):
        assert sample(l, 1.0, 1.0, u)["token"] == want, u


def test_temperature_scales_logits():
    # at temperature 2 the weights become sqrt(1), sqrt(4), sqrt(9) = 1, 2, 3
    l = np.log([1.0, 4.0, 9.0])
    for u, want in ((0.1, 0), (0.3, 1), (0.6, 2)):
        assert sample(l, 2.0, 1.0, u)["token"] == want


def test_top_p_keeps_crossing_token():
    # weights 1, 2, 3, 4 (sum 10); descending cumulative 0.4, 0.7, 0.9, 1.0
    q = np.array([1.0, 2.0, 3.0, 4.0])
    assert nucleus(q, 0.5).tolist() == [False, False, True, True]
    assert nucleus(q, 0.7).tolist() == [False, False, True, True]   # reaches 0.7 exactly
    assert nucleus(q, 0.71).tolist() == [False, True, True, True]
    assert nucleus(q, 0.1).tolist() == [False, False, False, True]
    assert nucleus(q, 1.0).all()
    l = np.log(q)
    # kept {2, 3}, kept sum 7, walked in index order: boundary at 3/7
    assert sample(l, 1.0, 0.5, 0.42)["token"] == 2
    assert sample(l, 1.0, 0.5, 0.43)["token"] == 3


def test_top_p_ties_go_to_lower_index():
    q = np.array([2.0, 1.0, 2.0, 1.0])
    assert nucleus(q, 0.25).tolist() == [True, False, False, False]
    assert nucleus(q, 0.34).tolist() == [True, False, True, False]
    assert nucleus(q, 0.7).tolist() == [True, True, True, False]


@pytest.mark.parametrize("seed", range(5))
def test_matches_page_loop(seed):
    r = np.random.default_rng(seed)
    l = r.normal(size=300) * 3
    for T, p in ((0.7, 0.95), (1.0, 0.5), (1.5, 1.0)):
        q = np.exp((l - l.max()) / T)
        kept = nucleus(q, p)
        for u in r.random(50):
            got = sample(l, T, p, u)
            if got["gap"] < 1e-12:
                continue
            assert got["token"] == _page_roulette(q.tolist(), kept.tolist(), u)
            assert kept[got["token"]]


def test_grid_counts_closed_form():
    r = np.random.default_rng(7)
    l = r.normal(size=40)
    T, p, N = 0.8, 0.9, 4096
    q = np.exp((l - l.max()) / T)
    kept = nucleus(q, p)
    idx = np.nonzero(kept)[0]
    C = np.cumsum(q[idx]) / q[idx].sum()
    counts = np.zeros(40, dtype=int)
    for n in range(N):
        counts[sample(l, T, p, n / N)["token"]] += 1
    # u = n/N lands on token idx[i] iff C[i-1] < u <= C[i]  (first cum >= u)
    grid = np.arange(N) / N
    prev = np.concatenate([[-1.0], C[:-1]])
    want = np.zeros(40, dtype=int)
    for i, t in enumerate(idx):
        want[t] = np.sum((grid > prev[i]) & (grid <= C[i]))
    np.testing.assert_array_equal(counts, want)
    assert counts[~kept].sum() == 0


def test_low_temperature_and_tiny_top_p_are_argmax():
    r = np.random.default_rng(8)
    for _ in range(20):
        l = r.normal(size=1000)
        srt = np.sort(l)
        if srt[-1] - srt[-2] < 1e-2:
            l[np.argmax(l)] += 1e-2
        a = argmax(l)
        for u in (0.0, 0.3, 0.999999):
            assert sample(l, 1e-4, 0.95, u)["token"] == a
            assert sample(l, 1.0, 1e-9, u)["token"] == a
            assert sample(l, 0.0, 0.95, u)["token"] == a


def test_underflow_keeps_one_token():
    l = np.array([0.0, -1e4, -2e4])
    assert sample(l, 0.5, 0.95, 0.99)["token"] == 0


# ---- min-p (a reading: keep q >= min(min_p, 1) * max q, intersected with top-p)

def test_min_p_closed_form():
    # weights 8, 4, 2, 1 (max 8); min_p 0.3 keeps weights >= 2.4: {8, 4}
    q = np.array([8.0, 4.0, 2.0, 1.0])
    assert oracle.min_p_mask(q, 0.3).tolist() == [True, True, False, False]
    assert oracle.min_p_mask(q, 0.25).tolist() == [True, True, True, False]   # 2 >= 2 exactly
    assert oracle.min_p_mask(q, 0.0).all()
    l = np.log(q)
    # kept {0, 1}, sum 12, walked in index order: boundary at 8/12
    assert sample(l, 1.0, 1.0, 0.66, min_p=0.3)["token"] == 0
    assert sample(l, 1.0, 1.0, 0.67, min_p=0.3)["token"] == 1
    # top-p 0.5 (8/15 >= 0.5 after the first) is the shorter prefix here
    assert sample(l, 1.0, 0.5, 0.99, min_p=0.3)["token"] == 0
    assert sample(l, 1.0, 0.5, 0.99, min_p=0.3)["n_kept"] == 1


def test_min_p_zero_is_top_p_alone():
    r = np.random.default_rng(11)
    l = r.normal(size=500) * 2
    for u in r.random(40):
        a = sample(l, 0.8, 0.9, u)
        b = sample(l, 0.8, 0.9, u, min_p=0.0)
        assert a["token"] == b["token"] and a["n_kept"] == b["n_kept"]


def test_min_p_one_is_argmax():
    # min_p >= 1 keeps only the largest weight(s): a unique maximum is argmax
    r = np.random.default_rng(12)
    for _ in range(10):
        l = r.normal(size=200)
        for u in (0.0, 0.3, 0.999):
            assert sample(l, 1.3, 1.0, u, min_p=1.0)["token"] == argmax(l)
            assert sample(l, 1.3, 1.0, u, min_p=2.5)["token"] == argmax(l)


def test_min_p_brute_force_interval_lookup():
    # kept set by definition, token by the interval lookup over its prefix sums
    r = np.random.default_rng(13)
    for trial in range(20):
        l = r.normal(size=40) * 3
        T, p, mp = 0.9, float(r.uniform(0.3, 1.0)), float(r.uniform(0.01, 0.5))
        q = np.exp((l - l.max()) / T)
        # top-p kept set, brute force: a token is kept when the mass strictly
        # ahead of it in the (q desc, index asc) order is below p * total
        ahead = np.array([q[(q > q[i]) | ((q == q[i]) & (np.arange(40) < i))].sum()
                          for i in range(40)])
        kept = (ahead < p * q.sum()) | (p >= 1.0)
        kept &= q >= mp * q.max()
        for u in r.random(10):
            got = sample(l, T, p, u, min_p=mp)
            if got["gap"] < 1e-12 or got["min_p_gap"] < 1e-12:
                continue
            assert got["n_kept"] == int(kept.sum())
            assert got["token"] == _page_roulette(q.tolist(), kept.tolist(), u)


def test_nucleus_cut_gap_closed_forms():
    from oracle.sampler import nucleus_cut_gap
    # weights 1, 2, 3, 4: descending shares 0.4, 0.7, 0.9, 1.0
    q = np.array([1.0, 2.0, 3.0, 4.0])
    assert nucleus_cut_gap(q, 0.69) == pytest.approx(0.01)      # cut after 0.7, 0.4 below
    assert nucleus_cut_gap(q, 0.5) == pytest.approx(0.1)        # between 0.4 and 0.7
    assert nucleus_cut_gap(q, 0.7) == pytest.approx(0.0)        # on a boundary
    assert nucleus_cut_gap(q, 0.1) == pytest.approx(0.1)        # first share 0.4; 0 below
    assert nucleus_cut_gap(q, 1.0) == float("inf")
    # the dict carries it; temperature 1 on log weights reproduces q
    r = sample(np.log(q), 1.0, 0.69, 0.3)
    assert r["cut_gap"] == pytest.approx(0.01)
    assert sample(np.log(q), 0.0, 0.69, 0.3)["cut_gap"] == float("inf")


def test_nucleus_cut_gap_bounds_a_moved_cut():
    # moving every weight by less than the cut gap (relative share) leaves the
    # kept set alone; moving one weight across it changes the set
    r = np.random.default_rng(5)
    from oracle.sampler import nucleus_cut_gap
    for _ in range(50):
        q = r.exponential(size=40)
        p = float(r.uniform(0.2, 0.95))
        g = nucleus_cut_gap(q, p)
        eps = 0.2 * g / 2
        q2 = q * (1 + r.uniform(-eps, eps, size=q.size))
        assert np.array_equal(nucleus(q, p), nucleus(q2, p))
