"""Pins of the oracle's elementary pieces: bf16 widening, RMSNorm, SiLU,
softmax top-k, and the sampler's generator."""
import math
import os

import numpy as np
import pytest

import oracle
from oracle.layer import widen, rmsnorm, silu, topk_desc, routing_permutation, router_margin

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_widen_bf16_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80, 0x0000, 0x8000], dtype=np.uint16)
    v = widen(bits)
    assert v[0] == 1.0 and v[1] == -2.0
    assert v[2] == 1.0 + 2.0 ** -7
    assert v[3] == 2.0 ** -133          # smallest bf16 subnormal
    assert math.isinf(v[4]) and v[5] == 0.0 and v[6] == 0.0
    assert math.copysign(1.0, v[6]) == -1.0


def test_rmsnorm_closed_form():
    # mean square of (3, 4) is 12.5
    y = rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.0)
    np.testing.assert_allclose(y, [3 / math.sqrt(12.5), 8 / math.sqrt(12.5)], rtol=1e-15)
    # eps enters under the root
    y = rmsnorm(np.array([3.0, 4.0]), np.ones(2), 0.5)
    np.testing.assert_allclose(y, [3 / math.sqrt(13.0), 4 / math.sqrt(13.0)], rtol=1e-15)


def test_rmsnorm_invariants():
    r = np.random.default_rng(1)
    x = r.normal(size=(5, 64))
    g = np.ones(64)
    y = rmsnorm(x, g, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(rmsnorm(7.5 * x, g, 0.0), y, rtol=1e-13)
    # normalisation is per row: rows do not mix
    np.testing.assert_allclose(rmsnorm(x[2:3], g, 0.0), y[2:3], rtol=1e-15)


def test_silu_values_and_identity():
    assert silu(np.array(0.0)) == 0.0
    np.testing.assert_allclose(silu(np.array([1.0, -1.0])),
                               [0.7310585786300049, -0.2689414213699951], rtol=1e-15)
    z = np.linspace(-30, 30, 121)
    # z*sigma(z) - (-z)*sigma(-z) = z
    np.testing.assert_allclose(silu(z) - silu(-z), z, rtol=1e-13, atol=1e-13)
    assert np.all(np.isfinite(silu(np.array([-1000.0, 1000.0]))))


def test_topk_matches_stable_argsort():
    r = np.random.default_rng(2)
    s = r.normal(size=(300, 256))
    s[:, 17] = s[:, 40]                    # force ties inside the rows
    s[5, :] = 0.0                          # all equal: lowest indices win
    got = topk_desc(s, 6)
    ref = np.argsort(-s, axis=1, kind="stable")[:, :6]
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(got[5], np.arange(6))


def test_routing_permutation_against_sort():
    r = np.random.default_rng(3)
    T, k, E = 97, 6, 33
    idx = np.stack([r.permutation(E)[:k] for _ in range(T)])
    count, offset, perm = routing_permutation(idx, E)
    assert count.sum() == T * k and offset[0] == 0 and offset[-1] == T * k
    assert np.all(np.diff(offset) == count)
    assert sorted(perm.tolist()) == list(range(T * k))
    e_of = idx.reshape(-1)
    tok = np.repeat(np.arange(T), k)
    ref = np.lexsort((tok, e_of))          # expert ascending, then token
    np.testing.assert_array_equal(perm, ref)
    for e in range(E):
        seg = perm[offset[e]:offset[e + 1]]
        assert np.all(e_of[seg] == e)
        assert np.all(np.diff(seg // k) > 0)


def test_router_margin():
    s = np.array([[5.0, 1.0, 4.0, 3.0, 2.0]])
    np.testing.assert_allclose(router_margin(s, 2), [1.0])
    np.testing.assert_allclose(router_margin(s, 3), [1.0])


def test_splitmix64_published_values():
    want = [int(l, 16) for l in open(os.path.join(GOLDEN, "splitmix64_seed0.txt"))
            if l.strip() and not l.startswith("#")]
    g = oracle.SplitMix64(0)
    assert [g.next_u64() for _ in range(3)] == want


def test_splitmix64_float_draw():
    g = oracle.SplitMix64(12345)
    h = oracle.SplitMix64(12345)
    for _ in range(100):
        u = g.next_f32()
        z = h.next_u64()
        assert 0.0 <= u < 1.0
        assert u == (z >> 40) / 16777216.0
        assert np.float32(u) == u          # exactly representable in fp32
