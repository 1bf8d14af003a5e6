"""Small synthetic layers for the oracle's CPU tests (numpy only)."""
import dataclasses

import numpy as np


@dataclasses.dataclass
class Cfg:
    hidden: int = 16
    n_heads: int = 3
    head_dim: int = 4
    qkv_rank: int = 5
    window: int = 4
    n_experts: int = 6
    top_k: int = 2
    ffn_inter: int = 7
    rope_dim: int = 0
    rope_base: float = 10000.0
    rms_eps: float = 1e-6


def tiny_weights(cfg, seed=0, std=0.3):
    r = np.random.default_rng(seed)
    d, H, dh, rk, E, I = (cfg.hidden, cfg.n_heads, cfg.head_dim, cfg.qkv_rank,
                          cfg.n_experts, cfg.ffn_inter)
    n = lambda *s: r.normal(0.0, std, s)
    return {
        "attn_norm": 1.0 + n(d) * 0.1, "qkv_a": n(rk, d), "qkv_b": n(H * dh + 2 * dh, rk),
        "wo": n(d, H * dh), "ffn_norm": 1.0 + n(d) * 0.1, "router": n(E, d),
        "gate": n(E, I, d), "up": n(E, I, d), "down": n(E, d, I),
        "sh_gate": n(I, d), "sh_up": n(I, d), "sh_down": n(d, I),
    }
