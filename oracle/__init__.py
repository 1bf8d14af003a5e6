"""Plain, slow float64 CPU oracle for the ds4 DeepSeek-V4-style layer path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP path never
calls it, and it imports nothing from the HIP path.

What it follows (ds4.c 学习笔记, page 端到端推理流程):
  * layer.py   -- 阶段四 4.2 单层前向 (the per-layer pseudo-code) and
                  阶段三 逐层批处理 (layer-major prefill), 4.1 Embedding;
  * sampler.py -- 阶段四 4.3 采样 (temperature, top-p, roulette, argmax);
  * rng.py     -- the sampler's uniform draw, splitmix64 (Steele, Lea and
                  Flood, "Fast splittable pseudorandom number generators",
                  OOPSLA 2014), since the page names the call but not the
                  generator.

Readings where the page is silent are listed in each function's docstring.
Every function is pinned by CPU tests against closed forms, invariants,
brute force on tiny inputs, or published test values.
"""
from .layer import (widen, rmsnorm, silu, rope, Ring, attend, topk_desc,
                    routing_permutation, layer_forward, lm_head, embed,
                    stack_prefill, router_margin)
from .sampler import sample, argmax, nucleus, min_p_mask
from .rng import SplitMix64

__all__ = ["widen", "rmsnorm", "silu", "rope", "Ring", "attend", "topk_desc",
           "routing_permutation", "layer_forward", "lm_head", "embed",
           "stack_prefill", "router_margin", "sample", "argmax", "nucleus", "min_p_mask",
           "SplitMix64"]
