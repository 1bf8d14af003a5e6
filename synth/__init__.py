"""Seeded synthetic inputs for the ds4 DeepSeek-V4-style layer.

This module is shared by the HIP path's tests/bench and by the oracle's tests.
It holds shapes and random numbers only: none of the layer's arithmetic.

The pages ship no trained weights and no prompts, so every weight is drawn
from N(0, 0.02) (gains from 1 + N(0, 0.02)), hidden states from N(0, 1) and
token ids uniformly over the vocabulary.  Every tensor gets its own torch
generator, seeded from (config seed, layer, tensor index), so the values do
not depend on the order in which tensors are made.  torch's CPU and GPU
generators give different streams: a test that checks the GPU against the
oracle makes the tensors on the GPU and hands the oracle a host copy.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Dimensions of one layer.

    Sizes named on ds4-learning 端到端推理流程 (阶段四 4.2 单层前向): hidden
    4096, 64-head MQA, window 128, 256 experts, top-6 plus a shared expert.
    head_dim, qkv_rank, ffn_inter and rope_base are the workload's own sizes.
    """
    hidden: int
    n_heads: int
    head_dim: int
    qkv_rank: int
    window: int
    n_experts: int
    top_k: int
    ffn_inter: int
    n_shared: int = 1
    rope_dim: int = 0          # 0 means the whole head
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    wdtype: str = BF16

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def qkv_dim(self) -> int:
        return self.n_heads * self.head_dim + 2 * self.head_dim

    @property
    def rope_width(self) -> int:
        return self.rope_dim if self.rope_dim else self.head_dim


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layer: LayerShape
    seed: int
    n_layers: int = 1
    vocab: int = 0
    prompt: int = 0            # prefill tokens
    decode: int = 0            # decode steps
    ring_prefill: int = 0      # positions already in the ring before decode
    temperature: float = 0.0
    top_p: float = 1.0
    snapshot_at: int = 0       # resume point for the prefix-reuse workload


FULL = dict(hidden=4096, n_heads=64, head_dim=128, qkv_rank=1024, window=128,
            n_experts=256, top_k=6, rope_base=10000.0)

WORKLOADS: Dict[str, Workload] = {
    # 2-layer tiny stack, fp32 weights, 64-token prompt then 16 greedy steps
    "tiny_stack": Workload(
        "tiny_stack",
        LayerShape(hidden=256, n_heads=4, head_dim=64, qkv_rank=64, window=128,
                   n_experts=8, top_k=2, ffn_inter=512, wdtype=F32),
        seed=1001, n_layers=2, vocab=1024, prompt=64, decode=16),
    # one full-size layer, single-token decode at position 128 over a full ring
    "layer_decode": Workload(
        "layer_decode", LayerShape(ffn_inter=1024, **FULL), seed=1002,
        ring_prefill=128, decode=1),
    # the same layer, layer-major prefill of 2048 tokens from an empty ring
    "layer_prefill_2048": Workload(
        "layer_prefill_2048", LayerShape(ffn_inter=1024, **FULL), seed=1003,
        prompt=2048),
    # 43-layer stack with expert inter 512, lm_head over 129280 tokens
    "stack43_decode": Workload(
        "stack43_decode", LayerShape(ffn_inter=512, **FULL), seed=1004,
        n_layers=43, vocab=129280, prompt=512, decode=256, temperature=0.7,
        top_p=0.95),
    # 43-layer stack, 16994-token prefill; resume from 16846 with a 148 suffix
    "stack43_resume": Workload(
        "stack43_resume", LayerShape(ffn_inter=512, **FULL), seed=1005,
        n_layers=43, vocab=129280, prompt=16994, snapshot_at=16846),
}

# tensor order fixes each tensor's generator seed; never reorder
LAYER_TENSORS = ("attn_norm", "qkv_a", "qkv_b", "wo", "ffn_norm", "router",
                 "gate", "up", "down", "sh_gate", "sh_up", "sh_down")
GAINS = ("attn_norm", "ffn_norm")
WEIGHT_STD = 0.02


def layer_tensor_shapes(s: LayerShape) -> Dict[str, tuple]:
    """Row-major [out, in] layouts (experts stacked on the leading axis)."""
    I = s.ffn_inter * s.n_shared
    return {
        "attn_norm": (s.hidden,),
        "qkv_a": (s.qkv_rank, s.hidden),
        "qkv_b": (s.qkv_dim, s.qkv_rank),
        "wo": (s.hidden, s.q_dim),
        "ffn_norm": (s.hidden,),
        "router": (s.n_experts, s.hidden),
        "gate": (s.n_experts, s.ffn_inter, s.hidden),
        "up": (s.n_experts, s.ffn_inter, s.hidden),
        "down": (s.n_experts, s.hidden, s.ffn_inter),
        "sh_gate": (I, s.hidden),
        "sh_up": (I, s.hidden),
        "sh_down": (s.hidden, I),
    }


def _seed(*parts: int) -> int:
    # fixed mixing of small integers into a 63-bit seed (splitmix64 finaliser)
    z = 0
    for p in parts:
        z = (z + 0x9E3779B97F4A7C15 + (p & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        z ^= z >> 31
    return z & 0x7FFFFFFFFFFFFFFF


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _store_dtype(wdtype: str) -> torch.dtype:
    return torch.bfloat16 if wdtype == BF16 else torch.float32


def normal(shape, seed_parts, device="cpu", mean=0.0, std=1.0,
           dtype=torch.float32) -> torch.Tensor:
    """N(mean, std) drawn in fp32, rounded to `dtype` (RNE for bf16)."""
    g = _gen(device, *seed_parts)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def layer_weights(s: LayerShape, seed: int, layer: int = 0, device="cpu",
                  experts_chunk: int = 32) -> Dict[str, torch.Tensor]:
    """All weights of one layer, stored in s.wdtype, [out, in] row-major.

    Expert stacks are drawn in chunks of `experts_chunk` experts (each chunk
    with its own generator) so a full-size layer needs little temporary
    memory; the chunk size is part of the recipe and fixed at 32.
    """
    dt = _store_dtype(s.wdtype)
    out = {}
    for i, name in enumerate(LAYER_TENSORS):
        shp = layer_tensor_shapes(s)[name]
        if name in GAINS:
            out[name] = normal(shp, (seed, layer, i), device, 1.0, WEIGHT_STD, dt)
        elif name in ("gate", "up", "down"):
            parts = []
            for c0 in range(0, shp[0], experts_chunk):
                c1 = min(shp[0], c0 + experts_chunk)
                parts.append(normal((c1 - c0,) + shp[1:], (seed, layer, i, c0),
                                    device, 0.0, WEIGHT_STD, dt))
            out[name] = torch.cat(parts, 0) if len(parts) > 1 else parts[0]
        else:
            out[name] = normal(shp, (seed, layer, i), device, 0.0, WEIGHT_STD, dt)
    return out


def head_weights(s: LayerShape, vocab: int, seed: int, device="cpu"):
    """Embedding [vocab, hidden], final-norm gain [hidden], lm_head [vocab, hidden]."""
    dt = _store_dtype(s.wdtype)
    return {
        "embed": normal((vocab, s.hidden), (seed, 9001, 0), device, 0.0, WEIGHT_STD, dt),
        "final_norm": normal((s.hidden,), (seed, 9001, 1), device, 1.0, WEIGHT_STD, dt),
        "lm_head": normal((vocab, s.hidden), (seed, 9001, 2), device, 0.0, WEIGHT_STD, dt),
    }


def hidden(T: int, d: int, seed: int, stream: int = 0, device="cpu",
           attempts: Optional[np.ndarray] = None) -> torch.Tensor:
    """N(0, 1) fp32 hidden states [T, d].

    `attempts[t]` picks which of several independent candidate draws row t
    takes; a test that rejects rows (e.g. for a router-score margin) raises
    that row's attempt number.  attempts=None means all zeros.
    """
    base = normal((T, d), (seed, 7001, stream, 0), device)
    if attempts is None:
        return base
    attempts = np.asarray(attempts)
    assert attempts.shape == (T,)
    for a in sorted(set(int(v) for v in attempts if v != 0)):
        rows = torch.as_tensor(np.nonzero(attempts == a)[0], device=device)
        cand = normal((T, d), (seed, 7001, stream, a), device)
        base[rows] = cand[rows]
    return base


def token_ids(T: int, vocab: int, seed: int, stream: int = 0) -> np.ndarray:
    """Uniform random token ids (stand-in for a tokenized prompt)."""
    g = _gen("cpu", seed, 7002, stream)
    return torch.randint(0, vocab, (T,), generator=g, dtype=torch.int64).numpy().astype(np.int32)


def rng_seed(seed: int) -> int:
    """Initial 64-bit state of the sampler's generator for a workload."""
    return _seed(seed, 7003)


# --------------------------------------------------------------------------
# host views of stored tensors, for the oracle (bit-exact; no arithmetic)

def to_host(t: torch.Tensor) -> np.ndarray:
    """bf16 tensors become uint16 bit arrays, everything else a numpy copy."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def weights_to_host(w: Dict[str, torch.Tensor]) -> Dict[str, np.ndarray]:
    return {k: to_host(v) for k, v in w.items()}
