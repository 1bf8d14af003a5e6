"""Float64 oracle of one DeepSeek-V4-style layer, its stack and the lm_head.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: ds4.c 学习笔记, page 端到端推理流程, section 阶段四 4.2 单层前向 (the
layer as two norm -> compute -> residual blocks), 阶段三 逐层批处理 (layer-major
prefill: every token goes through layer l before layer l+1), 4.1 Embedding
and 4.3 采样 (the lm_head projection to the vocabulary).

Conventions (readings where the page is silent; each is also stated where
it is used):
  * every weight matrix is row-major [out, in]; y = W x means
    y[i] = sum_j W[i, j] x[j];
  * the low-rank QKV is one shared bottleneck: c = A x (A [rank, hidden]),
    then [q | k | v] = B c (B [H*dh + 2*dh, rank]);
  * a dense output projection W_o [hidden, H*dh] maps the 64 heads back to
    the residual width (H*dh = 8192 differs from hidden = 4096);
  * RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gamma;
  * RoPE rotates interleaved pairs (2i, 2i+1) of the last rope_dim entries
    of each head by pos * base^(-2i/rope_dim), q and k only, before caching;
  * the window holds W keys including the token itself: [pos-W+1, pos];
  * attention scale 1/sqrt(dh), no bias, no soft-cap, no sink;
  * router: softmax over all experts, top-k chosen by logit (ties go to the
    lower index), each chosen expert weighted by its softmax probability
    (no renormalisation); expert FFNs are SwiGLU, the shared expert has
    weight 1;
  * the residual stream is carried in full precision end to end.
"""
from __future__ import annotations

import copy
import math
from typing import Dict, Optional, Sequence

import numpy as np


# ---------------------------------------------------------------- numbers

def widen(a) -> np.ndarray:
    """Stored tensor -> float64, exactly.

    bf16 arrives as uint16 bit patterns: a bf16 value is the upper half of
    the fp32 with the same bits, so shifting left by 16 and reading fp32
    gives the value exactly.  fp32 / fp64 arrays are converted directly.
    """
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rmsnorm(x: np.ndarray, gamma, eps: float) -> np.ndarray:
    """RMSNorm over the last axis (阶段四 4.2, 'x_norm = RMSNorm(x)')."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * widen(gamma)


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + e^-z), the SwiGLU gate activation."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def softmax(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


# ---------------------------------------------------------------- RoPE

def rope(x: np.ndarray, pos: int, base: float, rope_dim: Optional[int] = None) -> np.ndarray:
    """Rotary position embedding of one position (阶段四 4.2, 'Q, K = RoPE(Q, K, position)').

    The page names the routine rope_tail_ext_inplace but gives no formula.
    Reading: the last `rope_dim` entries of each head (the whole head when
    rope_dim == dh) form pairs (off+2i, off+2i+1), i < rope_dim/2; pair i
    turns by angle pos * base^(-2i/rope_dim):
        (a, b) -> (a cos t - b sin t,  a sin t + b cos t).
    No context-extension scaling.  Angles are formed in float64.
    x: [..., dh]; returns a new array.
    """
    x = np.asarray(x, dtype=np.float64)
    dh = x.shape[-1]
    rd = dh if not rope_dim else rope_dim
    off = dh - rd
    out = x.copy()
    for i in range(rd // 2):
        theta = float(pos) * base ** (-2.0 * i / rd)
        c, s = math.cos(theta), math.sin(theta)
        a = x[..., off + 2 * i]
        b = x[..., off + 2 * i + 1]
        out[..., off + 2 * i] = a * c - b * s
        out[..., off + 2 * i + 1] = a * s + b * c
    return out


# ---------------------------------------------------------------- KV ring

class Ring:
    """The per-layer KV cache, kept as a W-slot ring (阶段四 4.2 'KVCache.append(K, V)').

    Position p lives in slot p mod W.  `pos` is the number of positions
    appended so far, i.e. the position of the next token.  Keys are stored
    after RoPE.  A window of W keys includes the newest token, so a W-slot
    ring holds everything attention can still see.
    """

    def __init__(self, window: int, head_dim: int):
        self.W = window
        self.k = np.zeros((window, head_dim))
        self.v = np.zeros((window, head_dim))
        self.pos = 0

    def append(self, k: np.ndarray, v: np.ndarray) -> None:
        slot = self.pos % self.W
        self.k[slot] = k
        self.v[slot] = v
        self.pos += 1

    def window(self):
        """Keys/values of positions [max(0, pos-W), pos) in position order."""
        lo = max(0, self.pos - self.W)
        slots = [p % self.W for p in range(lo, self.pos)]
        return self.k[slots], self.v[slots], np.arange(lo, self.pos)

    def snapshot(self) -> "Ring":
        return copy.deepcopy(self)


# ---------------------------------------------------------------- attention

def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """Multi-query attention of one token (阶段四 4.2 'Attention(Q, KVCache)', 64 头 MQA).

    q: [H, dh] (all heads of the token), keys/vals: [n, dh] shared by every
    head.  o_h = sum_j softmax_j(q_h . k_j / sqrt(dh)) v_j.
    """
    dh = q.shape[-1]
    s = (q @ keys.T) / math.sqrt(dh)                # [H, n]
    return softmax(s) @ vals                        # [H, dh]


# ---------------------------------------------------------------- router

def topk_desc(s: np.ndarray, k: int) -> np.ndarray:
    """Top-k indices in descending score order (阶段四 4.2 'TopK(scores, 6)').

    s: [n] or [T, n].  Done as k rounds of 'take the largest remaining
    score' (np.argmax returns the first maximum, so among equal scores the
    lower index is taken first).
    """
    s = np.array(s, dtype=np.float64)
    one = s.ndim == 1
    if one:
        s = s[None]
    out = np.empty((s.shape[0], k), dtype=np.int64)
    rows = np.arange(s.shape[0])
    for r in range(k):
        best = np.argmax(s, axis=1)
        out[:, r] = best
        s[rows, best] = -np.inf
    return out[0] if one else out


def routing_permutation(topk_idx: np.ndarray, n_experts: int):
    """Group the (token, slot) pairs by expert.

    Entry number t*k + j stands for slot j of token t.  The permutation
    lists entries expert by expert, and within an expert in token order.
    Returns (count [E], offset [E+1], perm [T*k]) with expert e's entries
    at perm[offset[e]:offset[e+1]].  (The layout of this grouping is a
    design choice of the build; the page only says six experts are chosen.)
    """
    T, k = topk_idx.shape
    count = np.zeros(n_experts, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            count[topk_idx[t, j]] += 1
    offset = np.zeros(n_experts + 1, dtype=np.int64)
    for e in range(n_experts):
        offset[e + 1] = offset[e] + count[e]
    fill = offset[:-1].copy()
    perm = np.empty(T * k, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = topk_idx[t, j]
            perm[fill[e]] = t * k + j
            fill[e] += 1
    return count, offset, perm


def router_margin(s: np.ndarray, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest router logit of each row."""
    srt = -np.sort(-np.asarray(s, dtype=np.float64), axis=-1)
    return srt[..., k - 1] - srt[..., k]


# ---------------------------------------------------------------- experts

def swiglu_ffn(y: np.ndarray, G, U, D) -> np.ndarray:
    """SwiGLU FFN: D (silu(G y) * (U y)); y [n, hidden] -> [n, hidden]."""
    g = y @ widen(G).T
    u = y @ widen(U).T
    return (silu(g) * u) @ widen(D).T


# ---------------------------------------------------------------- layer

def layer_forward(cfg, w: Dict[str, np.ndarray], ring: Ring, h: np.ndarray,
                  rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """One layer over T tokens at positions ring.pos .. ring.pos+T-1.

    Follows 阶段四 4.2 单层前向 step by step:
      x  = RMSNorm(h) * g1
      c  = A x ;  [q | k | v] = B c                 (low-rank QKV)
      q, k <- RoPE(q, k, pos)
      ring.append(k, v)
      o  = Attention(q, ring)                       (64-head MQA, window W)
      h2 = h + W_o o                                (residual)
      y  = RMSNorm(h2) * g2
      s  = W_r y ; p = softmax(s) ; S = TopK(s, k)
      out = h2 + sum_{e in S} p_e FFN_e(y) + FFN_shared(y)
    T = 1 is a decode step; T > 1 is layer-major prefill of this layer
    (阶段三): every step runs for all T tokens before the next, and the
    attention walks the tokens in order, appending each token's key before
    it attends, exactly as T decode steps would.

    h: [T, hidden].  The ring is updated in place.  rows: if given, the
    expert FFNs (the costly part) are evaluated only for these rows and the
    other rows of 'out' are NaN; everything else is computed for all rows.
    Returns a dict with out, h2, y, logits, probs, topk_idx, topk_w,
    count, offset, perm, margin.
    """
    h = np.asarray(h, dtype=np.float64)
    T, d = h.shape
    H, dh, k_top = cfg.n_heads, cfg.head_dim, cfg.top_k
    rd = getattr(cfg, "rope_dim", 0) or dh
    eps = cfg.rms_eps

    x = rmsnorm(h, w["attn_norm"], eps)
    c = x @ widen(w["qkv_a"]).T
    qkv = c @ widen(w["qkv_b"]).T
    q = qkv[:, : H * dh].reshape(T, H, dh)
    kk = qkv[:, H * dh: H * dh + dh]
    vv = qkv[:, H * dh + dh: H * dh + 2 * dh]

    o = np.empty((T, H, dh))
    for t in range(T):
        p = ring.pos
        qt = rope(q[t], p, cfg.rope_base, rd)
        kt = rope(kk[t], p, cfg.rope_base, rd)
        ring.append(kt, vv[t])
        keys, vals, _ = ring.window()
        o[t] = attend(qt, keys, vals)
    h2 = h + o.reshape(T, H * dh) @ widen(w["wo"]).T

    y = rmsnorm(h2, w["ffn_norm"], eps)
    logits = y @ widen(w["router"]).T
    probs = softmax(logits)
    topk_idx = topk_desc(logits, k_top)
    topk_w = np.take_along_axis(probs, topk_idx, axis=1)
    count, offset, perm = routing_permutation(topk_idx, cfg.n_experts)

    want = np.arange(T) if rows is None else np.asarray(sorted(set(rows)), dtype=np.int64)
    routed = np.zeros((T, d))
    sel = np.zeros(T, dtype=bool)
    sel[want] = True
    for e in range(cfg.n_experts):
        tt, jj = np.nonzero((topk_idx == e) & sel[:, None])
        if tt.size == 0:
            continue
        f = swiglu_ffn(y[tt], w["gate"][e], w["up"][e], w["down"][e])
        for n in range(tt.size):
            routed[tt[n]] += topk_w[tt[n], jj[n]] * f[n]
    shared = swiglu_ffn(y[want], w["sh_gate"], w["sh_up"], w["sh_down"])
    out = np.full((T, d), np.nan)
    out[want] = h2[want] + routed[want] + shared

    return dict(out=out, h2=h2, y=y, logits=logits, probs=probs,
                topk_idx=topk_idx, topk_w=topk_w, count=count, offset=offset,
                perm=perm, margin=router_margin(logits, k_top), x=x, c=c,
                qkv=qkv, o=o.reshape(T, H * dh))


# ---------------------------------------------------------------- stack

def embed(ids: np.ndarray, table) -> np.ndarray:
    """Embedding lookup (阶段四 4.1): row `id` of the table, widened to float."""
    ids = np.asarray(ids, dtype=np.int64)
    return widen(np.asarray(table)[ids])


def lm_head(x: np.ndarray, final_norm, w_lm, eps: float) -> np.ndarray:
    """Final hidden -> vocabulary logits (阶段四 4.3 'lm_head 投影').

    The page does not say whether a norm precedes the projection; the
    reading is a final RMSNorm with its own gain, skipped when final_norm
    is None.  x: [..., hidden] -> [..., vocab].
    """
    x = np.asarray(x, dtype=np.float64)
    if final_norm is not None:
        x = rmsnorm(x, final_norm, eps)
    return x @ widen(w_lm).T


def stack_prefill(cfg, layers, rings, h: np.ndarray, rows=None):
    """Layer-major prefill through a stack (阶段三 逐层批处理): all tokens
    through layer 0, then all through layer 1, ...  Returns the last
    hidden [T, hidden] and the per-layer result dicts."""
    x = np.asarray(h, dtype=np.float64)
    infos = []
    for l, (w, ring) in enumerate(zip(layers, rings)):
        r = layer_forward(cfg, w, ring, x, rows=rows)
        infos.append(r)
        x = r["out"]
    return x, infos
