"""Pins of the oracle's RoPE, KV ring and windowed MQA attention."""
import math

import numpy as np
import pytest

from oracle.layer import rope, Ring, attend, layer_forward, softmax
from tests.oracle_fixtures import Cfg, tiny_weights


def test_rope_preserves_norm():
    r = np.random.default_rng(0)
    x = r.normal(size=(64, 128))
    for p in (0, 1, 127, 128, 2047, 16993, 1_000_000):
        y = rope(x, p, 10000.0)
        np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)


def test_rope_identity_at_zero():
    x = np.random.default_rng(1).normal(size=(3, 64))
    np.testing.assert_array_equal(rope(x, 0, 10000.0), x)


def test_rope_pair_layout_and_sign():
    # entry 0 alone turns into pair (0, 1) by angle pos * base^0 = pos
    x = np.zeros(8); x[0] = 1.0
    y = rope(x, 1, 10000.0)
    np.testing.assert_allclose(y[:2], [math.cos(1.0), math.sin(1.0)], rtol=1e-15)
    assert np.all(y[2:] == 0)
    # entry 1 alone: (0, 1) -> (-sin, cos)
    x = np.zeros(8); x[1] = 1.0
    np.testing.assert_allclose(rope(x, 3, 10000.0)[:2], [-math.sin(3.0), math.cos(3.0)], rtol=1e-15)
    # pair i turns by pos * base^(-2i/dh)
    dh, base, p = 8, 10000.0, 5
    for i in range(dh // 2):
        x = np.zeros(dh); x[2 * i] = 1.0
        th = p * base ** (-2.0 * i / dh)
        np.testing.assert_allclose(rope(x, p, base)[2 * i:2 * i + 2],
                                   [math.cos(th), math.sin(th)], rtol=1e-14, atol=1e-15)


def test_rope_relative_position():
    r = np.random.default_rng(2)
    q, k = r.normal(size=128), r.normal(size=128)
    for m, n in ((3, 10), (100, 37), (5000, 5127)):
        lhs = rope(q, m, 10000.0) @ rope(k, n, 10000.0)
        rhs = q @ rope(k, n - m, 10000.0)
        assert abs(lhs - rhs) < 1e-11 * np.linalg.norm(q) * np.linalg.norm(k)


def test_rope_composition_and_tail():
    r = np.random.default_rng(3)
    x = r.normal(size=16)
    np.testing.assert_allclose(rope(rope(x, 7, 100.0), 11, 100.0), rope(x, 18, 100.0), rtol=1e-12, atol=1e-13)
    y = rope(x, 9, 100.0, rope_dim=6)      # only the last 6 entries turn
    np.testing.assert_array_equal(y[:10], x[:10])
    np.testing.assert_allclose(y[10:], rope(x[10:], 9, 100.0), rtol=1e-15)


def test_ring_slots_hold_last_window():
    ring = Ring(4, 2)
    for p in range(11):
        ring.append(np.full(2, p), np.full(2, -p))
        keys, vals, poss = ring.window()
        lo = max(0, p + 1 - 4)
        np.testing.assert_array_equal(poss, np.arange(lo, p + 1))
        np.testing.assert_array_equal(keys[:, 0], poss)
        np.testing.assert_array_equal(vals[:, 0], -poss)


def _attend_scalar(q, keys, vals):
    # textbook scaled-dot-product attention, one head at a time, scalar loops
    H, dh = q.shape
    out = np.zeros((H, dh))
    for h in range(H):
        s = [sum(q[h, i] * kk[i] for i in range(dh)) / math.sqrt(dh) for kk in keys]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        z = sum(e)
        for j, vv in enumerate(vals):
            out[h] += e[j] / z * vv
    return out


def test_attend_textbook_and_special_cases():
    r = np.random.default_rng(4)
    q, keys, vals = r.normal(size=(3, 8)), r.normal(size=(5, 8)), r.normal(size=(5, 8))
    np.testing.assert_allclose(attend(q, keys, vals), _attend_scalar(q, keys, vals), rtol=1e-13)
    # q = 0: uniform weights, the mean of the values
    np.testing.assert_allclose(attend(np.zeros((2, 8)), keys, vals), np.tile(vals.mean(0), (2, 1)), rtol=1e-14)
    # one key: its value
    np.testing.assert_allclose(attend(q, keys[:1], vals[:1]), np.tile(vals[0], (3, 1)), rtol=1e-15)


def _banded_attention(cfg, qkv, W, n_past=0):
    """Brute force: RoPE every row, then a causal band mask over full K/V."""
    T = qkv.shape[0]
    H, dh = cfg.n_heads, cfg.head_dim
    q = np.stack([rope(qkv[t, :H * dh].reshape(H, dh), n_past + t, cfg.rope_base) for t in range(T)])
    k = np.stack([rope(qkv[t, H * dh:H * dh + dh], n_past + t, cfg.rope_base) for t in range(T)])
    v = qkv[:, H * dh + dh:]
    o = np.zeros((T, H, dh))
    idx = np.arange(T)
    for h in range(H):
        s = q[:, h, :] @ k.T / math.sqrt(dh)                 # [T, T]
        mask = (idx[None, :] <= idx[:, None]) & (idx[None, :] > idx[:, None] - W)
        s = np.where(mask, s, -np.inf)
        o[:, h, :] = softmax(s) @ v
    return o.reshape(T, H * dh)


@pytest.mark.parametrize("T,W", [(20, 32), (32, 32), (45, 8), (30, 1)])
def test_layer_attention_equals_banded_brute_force(T, W):
    cfg = Cfg(window=W)
    w = tiny_weights(cfg, seed=T)
    h = np.random.default_rng(T).normal(size=(T, cfg.hidden))
    r = layer_forward(cfg, w, Ring(W, cfg.head_dim), h)
    np.testing.assert_allclose(r["o"], _banded_attention(cfg, r["qkv"], W), rtol=1e-12, atol=1e-13)


def test_window_one_returns_own_value():
    cfg = Cfg(window=1)
    w = tiny_weights(cfg, seed=9)
    h = np.random.default_rng(9).normal(size=(6, cfg.hidden))
    r = layer_forward(cfg, w, Ring(1, cfg.head_dim), h)
    H, dh = cfg.n_heads, cfg.head_dim
    v = r["qkv"][:, H * dh + dh:]
    np.testing.assert_allclose(r["o"].reshape(6, H, dh), np.repeat(v[:, None, :], H, axis=1), rtol=1e-14)


def test_window_equals_full_attention_when_short():
    # with T <= W the window never drops a key: same as unbounded causal attention
    cfg = Cfg(window=64)
    w = tiny_weights(cfg, seed=5)
    h = np.random.default_rng(5).normal(size=(40, cfg.hidden))
    a = layer_forward(cfg, w, Ring(64, cfg.head_dim), h)
    b = layer_forward(Cfg(window=1000), w, Ring(1000, cfg.head_dim), h)
    np.testing.assert_array_equal(a["o"], b["o"])
    np.testing.assert_array_equal(a["out"], b["out"])
