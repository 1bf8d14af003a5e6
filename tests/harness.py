"""Shared helpers of the GPU parity tests: build a layer on the device from
the seeded generators, run the HIP path through the C ABI, and run the oracle
on host copies of exactly the same stored values."""
from __future__ import annotations

import dataclasses
import sys
import time
from typing import Dict, Optional

import numpy as np
import torch

import synth
import oracle


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def small_shape(**kw) -> synth.LayerShape:
    base = dict(hidden=256, n_heads=4, head_dim=64, qkv_rank=64, window=16, n_experts=8,
                top_k=2, ffn_inter=128, wdtype=synth.BF16)
    base.update(kw)
    return synth.LayerShape(**base)


class GpuLayer:
    """One layer's weights, ring and workspace on the device."""

    def __init__(self, shape: synth.LayerShape, seed: int, max_tokens: int, layer: int = 0,
                 routing: bool = True):
        import moe_dsv4_layer_amd as ds4g
        self.ds4g = ds4g
        self.shape = shape
        self.w = synth.layer_weights(shape, seed, layer=layer, device="cuda")
        self.cfg = ds4g.make_cfg(shape)
        self.cw = ds4g.make_weights(self.w)
        dh = shape.head_dim
        self.ring_k = torch.zeros((shape.window, dh), dtype=torch.float16, device="cuda")
        self.ring_v = torch.zeros((shape.window, dh), dtype=torch.float16, device="cuda")
        self.pos = torch.zeros(1, dtype=torch.int64, device="cuda")
        self.ring = ds4g.make_ring(self.ring_k, self.ring_v, self.pos)
        nb = ds4g.workspace_bytes(self.cfg, max_tokens)
        assert nb > 0
        self.ws = ds4g.alloc_workspace(nb)
        self.max_tokens = max_tokens
        self.routing_on = routing

    def host_weights(self) -> Dict[str, np.ndarray]:
        return synth.weights_to_host(self.w)

    def _routing(self, T):
        if not self.routing_on:
            return None, None
        s = self.shape
        b = {
            "topk_idx": torch.full((T, s.top_k), -1, dtype=torch.int32, device="cuda"),
            "topk_w": torch.zeros((T, s.top_k), dtype=torch.float32, device="cuda"),
            "expert_count": torch.full((s.n_experts,), -1, dtype=torch.int32, device="cuda"),
            "expert_offset": torch.full((s.n_experts + 1,), -1, dtype=torch.int32, device="cuda"),
            "perm": torch.full((T * s.top_k,), -1, dtype=torch.int32, device="cuda"),
            "router_in": torch.zeros((T, s.hidden), dtype=torch.float32, device="cuda"),
            "router_logits": torch.zeros((T, s.n_experts), dtype=torch.float32, device="cuda"),
        }
        return b, self.ds4g.make_routing(b)

    def prefill(self, h: torch.Tensor):
        T = h.shape[0]
        assert T <= self.max_tokens
        x = h.clone().contiguous()
        bufs, r = self._routing(T)
        self.ds4g.layer_prefill(self.cfg, self.cw, self.ring, x, T, self.ws, r)
        torch.cuda.synchronize()
        return x, bufs

    def decode(self, h: torch.Tensor):
        x = h.clone().reshape(-1).contiguous()
        bufs, r = self._routing(1)
        self.ds4g.layer_decode(self.cfg, self.cw, self.ring, x, self.ws, r)
        torch.cuda.synchronize()
        return x, bufs


def to_np(bufs):
    return {k: v.cpu().numpy() for k, v in bufs.items()}


def check_routing(shape, w_host, gpu: dict, orc: dict, rows=None, margin_gate=1e-3,
                  tf_margin=1e-3, label=""):
    """Routing parity.

    Teacher-forced: the oracle router applied to the GPU's own fp32 router
    input must choose the same expert set on every row whose margin there is
    >= tf_margin.  End to end: the GPU's choice equals the oracle's on every
    row whose oracle margin is >= margin_gate.  perm/count/offset must equal
    the oracle grouping of the GPU's own top-k bit for bit.
    """
    k = shape.top_k
    gi = gpu["topk_idx"].astype(np.int64)
    T = gi.shape[0]
    y = gpu["router_in"].astype(np.float64)
    s_tf = y @ oracle.widen(w_host["router"]).T
    tf_idx = oracle.topk_desc(s_tf, k)
    tf_m = oracle.router_margin(s_tf, k)
    ok_tf = tf_m >= tf_margin
    bad_tf = [t for t in range(T) if ok_tf[t] and set(gi[t]) != set(tf_idx[t])]
    assert not bad_tf, f"{label} teacher-forced top-k differs on rows {bad_tf[:10]}"
    # the order inside the top-k follows the logits
    bad_order = [t for t in range(T) if ok_tf[t] and not np.array_equal(gi[t], tf_idx[t])
                 and np.min(np.abs(np.diff(np.sort(s_tf[t])[::-1][:k + 1]))) > 1e-4]
    assert not bad_order, f"{label} top-k order differs on rows {bad_order[:10]}"
    # weights: softmax probabilities of the chosen experts
    p_tf = np.exp(s_tf - s_tf.max(1, keepdims=True))
    p_tf /= p_tf.sum(1, keepdims=True)
    np.testing.assert_allclose(gpu["topk_w"], np.take_along_axis(p_tf, gi, 1), rtol=2e-5,
                               atol=1e-7)
    # end to end
    om = orc["margin"]
    e2e = om >= margin_gate
    bad = [t for t in range(T) if e2e[t] and set(gi[t]) != set(orc["topk_idx"][t])]
    assert not bad, f"{label} end-to-end top-k differs on rows {bad[:10]} (margin>={margin_gate})"
    flips = int(sum(1 for t in range(T) if set(gi[t]) != set(orc["topk_idx"][t])))
    # grouping of the GPU's own choice
    cnt, off, perm = oracle.routing_permutation(gi, shape.n_experts)
    np.testing.assert_array_equal(gpu["expert_count"], cnt)
    np.testing.assert_array_equal(gpu["expert_offset"], off)
    np.testing.assert_array_equal(gpu["perm"], perm)
    return dict(tf_rows=int(ok_tf.sum()), e2e_rows=int(e2e.sum()), flips=flips,
                below_tf=int((~ok_tf).sum()))


def sampler_share_tol(logits, temperature: float) -> float:
    """How far the GPU's kept-mass shares can sit from the oracle's.

    The GPU takes each weight as expf of the fp32 argument (l - max) / T --
    a rounded subtraction and a rounded division, each within 2^-24 of the
    argument, then expf within one ulp (2^-23) -- and sums fixed-point
    masses exactly, each truncated by at most 2^-45.  So a weight moves by
    at most q (2 |x| 2^-24 + 2^-23) + 2^-45 and any running share C/S by at
    most twice the sum of that over the vocabulary, divided by S."""
    if temperature <= 0.0:
        return 0.0
    l = np.asarray(logits, dtype=np.float64)
    x = (l - l.max()) / temperature
    q = np.exp(x)
    dq = q * (2.0 * np.abs(x) * 2.0 ** -24 + 2.0 ** -23) + 2.0 ** -45
    return float(2.0 * dq.sum() / q.sum())


def sampler_excused(ref: dict, logits, temperature: float) -> bool:
    """A GPU/oracle token mismatch is excused only when the draw sits closer
    to a roulette boundary, the top-p cut or the min-p threshold than the
    GPU's fp32 weights can move it (sampler_share_tol)."""
    tol = sampler_share_tol(logits, temperature)
    x_max = float(np.abs((np.asarray(logits, np.float64) - np.max(logits)) / temperature).max()) \
        if temperature > 0 else 0.0
    q_rel = 2.0 * x_max * 2.0 ** -24 + 2.0 ** -23
    return ref["gap"] < tol or ref.get("cut_gap", np.inf) < tol or \
        ref.get("min_p_gap", np.inf) < 2.0 * q_rel
