"""The sampler's uniform draw (ds4.c 学习笔记, 端到端推理流程, 阶段四 4.3 采样:
'sample_rng_f32(rng)').

TEST INFRASTRUCTURE ONLY (see the package docstring).

The page names the call but not the generator.  Reading: splitmix64 as
published by Steele, Lea and Flood ("Fast splittable pseudorandom number
generators", OOPSLA 2014) on a 64-bit state, one draw per sampled token:
    state += 0x9E3779B97F4A7C15
    z = state
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
    z = (z ^ (z >> 27)) * 0x94D049BB133111EB
    out = z ^ (z >> 31)
and the float is the top 24 bits scaled by 2^-24, a value in [0, 1) that
fp32 holds exactly.
"""
from __future__ import annotations

MASK = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


class SplitMix64:
    def __init__(self, state: int):
        self.state = state & MASK

    def next_u64(self) -> int:
        self.state = (self.state + GAMMA) & MASK
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
        return z ^ (z >> 31)

    def next_f32(self) -> float:
        return (self.next_u64() >> 40) * (1.0 / (1 << 24))
