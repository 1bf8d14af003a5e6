"""Pins of the oracle's whole layer: a scalar brute-force re-derivation on
tiny shapes, prefill == decode, snapshot/resume, and closed forms of the
expert mixture."""
import math

import numpy as np
import pytest

from oracle.layer import layer_forward, Ring, stack_prefill, lm_head, embed, rmsnorm
from tests.oracle_fixtures import Cfg, tiny_weights


def _mv(W, x):
    # y[i] = sum_j W[i][j] x[j]  (weights are [out, in])
    return [sum(W[i][j] * x[j] for j in range(len(x))) for i in range(len(W))]


def _brute_layer(cfg, w, h_rows, n_past=0, ring_keys=None, ring_vals=None):
    """The layer of 阶段四 4.2 written with Python scalars and lists only."""
    d, H, dh, W, E, K = (cfg.hidden, cfg.n_heads, cfg.head_dim, cfg.window,
                         cfg.n_experts, cfg.top_k)
    eps, base = cfg.rms_eps, cfg.rope_base
    keys = list(ring_keys or [])
    vals = list(ring_vals or [])
    out_rows = []

    def norm(x, g):
        ms = sum(v * v for v in x) / len(x)
        return [x[i] / math.sqrt(ms + eps) * g[i] for i in range(len(x))]

    def rot(vec, p):
        v = list(vec)
        for i in range(dh // 2):
            th = p * base ** (-2.0 * i / dh)
            a, b = vec[2 * i], vec[2 * i + 1]
            v[2 * i] = a * math.cos(th) - b * math.sin(th)
            v[2 * i + 1] = a * math.sin(th) + b * math.cos(th)
        return v

    for t, h in enumerate(h_rows):
        p = n_past + t
        x = norm(h, w["attn_norm"])
        c = _mv(w["qkv_a"], x)
        qkv = _mv(w["qkv_b"], c)
        qs = [rot(qkv[hh * dh:(hh + 1) * dh], p) for hh in range(H)]
        keys.append(rot(qkv[H * dh:H * dh + dh], p))
        vals.append(qkv[H * dh + dh:H * dh + 2 * dh])
        lo = max(0, len(keys) - W)
        o = []
        for hh in range(H):
            sc = [sum(qs[hh][i] * kk[i] for i in range(dh)) / math.sqrt(dh) for kk in keys[lo:]]
            m = max(sc)
            ex = [math.exp(s - m) for s in sc]
            z = sum(ex)
            o += [sum(ex[j] / z * vals[lo + j][i] for j in range(len(ex))) for i in range(dh)]
        proj = _mv(w["wo"], o)
        h2 = [h[i] + proj[i] for i in range(d)]
        y = norm(h2, w["ffn_norm"])
        s = _mv(w["router"], y)
        m = max(s)
        ex = [math.exp(v - m) for v in s]
        z = sum(ex)
        prob = [v / z for v in ex]
        order = sorted(range(E), key=lambda e: (-s[e], e))[:K]

        def ffn(G, U, D):
            g = _mv(G, y)
            u = _mv(U, y)
            a = [g[i] / (1 + math.exp(-g[i])) * u[i] for i in range(len(g))]
            return _mv(D, a)

        out = list(h2)
        for e in order:
            f = ffn(w["gate"][e], w["up"][e], w["down"][e])
            out = [out[i] + prob[e] * f[i] for i in range(d)]
        f = ffn(w["sh_gate"], w["sh_up"], w["sh_down"])
        out = [out[i] + f[i] for i in range(d)]
        out_rows.append((out, order, [prob[e] for e in order]))
    return out_rows


def test_layer_matches_scalar_brute_force():
    # distinct sizes everywhere so a transposed operand cannot go unnoticed
    cfg = Cfg(hidden=10, n_heads=2, head_dim=4, qkv_rank=3, window=3,
              n_experts=5, top_k=2, ffn_inter=6)
    w = tiny_weights(cfg, seed=11, std=0.5)
    h = np.random.default_rng(11).normal(size=(5, cfg.hidden))
    r = layer_forward(cfg, w, Ring(cfg.window, cfg.head_dim), h)
    wl = {k: v.tolist() for k, v in w.items()}
    ref = _brute_layer(cfg, wl, h.tolist())
    for t, (out, order, probs) in enumerate(ref):
        np.testing.assert_allclose(r["out"][t], out, rtol=1e-12, atol=1e-12)
        assert r["topk_idx"][t].tolist() == order
        np.testing.assert_allclose(r["topk_w"][t], probs, rtol=1e-13)


def test_prefill_equals_token_by_token_decode():
    cfg = Cfg(window=8)
    w = tiny_weights(cfg, seed=12)
    h = np.random.default_rng(12).normal(size=(30, cfg.hidden))
    full = layer_forward(cfg, w, Ring(8, cfg.head_dim), h)
    ring = Ring(8, cfg.head_dim)
    outs = [layer_forward(cfg, w, ring, h[t:t + 1])["out"][0] for t in range(30)]
    np.testing.assert_allclose(np.stack(outs), full["out"], rtol=1e-12, atol=1e-13)


def test_suffix_from_snapshot_equals_full_prefill():
    cfg = Cfg(window=8)
    w = tiny_weights(cfg, seed=13)
    h = np.random.default_rng(13).normal(size=(40, cfg.hidden))
    ring = Ring(8, cfg.head_dim)
    full = layer_forward(cfg, w, ring, h)
    ring2 = Ring(8, cfg.head_dim)
    layer_forward(cfg, w, ring2, h[:29])
    snap = ring2.snapshot()
    suffix = layer_forward(cfg, w, snap, h[29:])
    np.testing.assert_allclose(suffix["out"], full["out"][29:], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(snap.k, ring.k)
    assert snap.pos == ring.pos == 40


def test_identical_experts_closed_form():
    # with every routed expert equal to f, out - h2 = (sum of chosen probs) f + f_shared
    cfg = Cfg()
    w = tiny_weights(cfg, seed=14)
    for key in ("gate", "up", "down"):
        w[key] = np.repeat(w[key][:1], cfg.n_experts, axis=0)
    h = np.random.default_rng(14).normal(size=(7, cfg.hidden))
    r = layer_forward(cfg, w, Ring(cfg.window, cfg.head_dim), h)
    y = r["y"]
    from oracle.layer import silu
    f = (silu(y @ w["gate"][0].T) * (y @ w["up"][0].T)) @ w["down"][0].T
    fs = (silu(y @ w["sh_gate"].T) * (y @ w["sh_up"].T)) @ w["sh_down"].T
    want = r["h2"] + r["topk_w"].sum(1, keepdims=True) * f + fs
    np.testing.assert_allclose(r["out"], want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["probs"].sum(1), 1.0, rtol=1e-14)


def test_zero_expert_weights_leave_the_residual():
    cfg = Cfg()
    w = tiny_weights(cfg, seed=15)
    for key in ("down", "sh_down"):
        w[key] = np.zeros_like(w[key])
    h = np.random.default_rng(15).normal(size=(4, cfg.hidden))
    r = layer_forward(cfg, w, Ring(cfg.window, cfg.head_dim), h)
    np.testing.assert_array_equal(r["out"], r["h2"])


def test_rows_subset_matches_full():
    cfg = Cfg()
    w = tiny_weights(cfg, seed=16)
    h = np.random.default_rng(16).normal(size=(9, cfg.hidden))
    full = layer_forward(cfg, w, Ring(cfg.window, cfg.head_dim), h)
    part = layer_forward(cfg, w, Ring(cfg.window, cfg.head_dim), h, rows=[1, 8])
    np.testing.assert_allclose(part["out"][[1, 8]], full["out"][[1, 8]], rtol=1e-13, atol=1e-14)
    assert np.all(np.isnan(part["out"][[0, 2, 3, 4, 5, 6, 7]]))
    np.testing.assert_array_equal(part["perm"], full["perm"])


def test_stack_and_lm_head():
    cfg = Cfg()
    layers = [tiny_weights(cfg, seed=20 + l) for l in range(3)]
    r = np.random.default_rng(17)
    table = r.normal(size=(50, cfg.hidden))
    ids = r.integers(0, 50, size=11)
    x0 = embed(ids, table)
    np.testing.assert_array_equal(x0, table[ids])
    rings = [Ring(cfg.window, cfg.head_dim) for _ in layers]
    x, infos = stack_prefill(cfg, layers, rings, x0)
    # layer-major result equals feeding each layer's output into the next
    y = x0
    for l, w in enumerate(layers):
        y = layer_forward(cfg, w, Ring(cfg.window, cfg.head_dim), y)["out"]
    np.testing.assert_array_equal(x, y)
    g = 1.0 + 0.1 * r.normal(size=cfg.hidden)
    wl = r.normal(size=(50, cfg.hidden))
    logits = lm_head(x[-1], g, wl, 1e-6)
    xn = rmsnorm(x[-1], g, 1e-6)
    np.testing.assert_allclose(logits, [sum(wl[i, j] * xn[j] for j in range(cfg.hidden)) for i in range(50)], rtol=1e-12)
    np.testing.assert_allclose(lm_head(x[-1], None, wl, 1e-6), wl @ x[-1], rtol=1e-12)
