"""Float64 oracle of the token sampler (ds4.c 学习笔记, 端到端推理流程,
阶段四 4.3 采样, with the argmax of 阶段六 温度覆盖 and the function index).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Steps as the page orders them: divide the logits by the temperature, turn
them into probabilities, keep the most probable tokens until their total
reaches top_p (sort descending, accumulate, drop the rest), then walk the
vocabulary with r = u * (sum of kept probabilities), subtracting each
token's probability until r <= 0.  Temperature 0 means argmax.

Readings where the page is silent:
  * temperature <= 0: argmax, first index among equal maxima; no draw;
  * the probabilities are exp((l - max l) / temperature) (the same as
    exp(l / temperature) up to a common factor);
  * ties in the descending sort go to the lower index; the token whose
    probability makes the running total reach top_p is kept, at least one
    token is kept, top_p >= 1 keeps everything;
  * the roulette walks the vocabulary in index order and skips tokens the
    top-p step dropped; if rounding leaves r > 0 after the last kept token,
    that last kept token is returned;
  * min-p (named with top-p in the page's function index, not defined
    there): the usual filter, a token stays when its probability is at least
    min(min_p, 1) times the largest one (so the most probable tokens always
    stay); with top-p a token is kept when both keep it (both keep a prefix
    of the descending order, so the shorter prefix); min_p <= 0 disables it.
"""
from __future__ import annotations

import numpy as np


def argmax(logits) -> int:
    """Greedy pick: the first index of the largest logit."""
    return int(np.argmax(np.asarray(logits, dtype=np.float64)))


def nucleus(q: np.ndarray, top_p: float) -> np.ndarray:
    """Boolean mask of the tokens top-p keeps.  q: unnormalised weights."""
    n = q.shape[0]
    if top_p >= 1.0:
        return np.ones(n, dtype=bool)
    order = np.lexsort((np.arange(n), -q))        # q descending, then index
    cum = np.cumsum(q[order]) / np.sum(q)
    n_keep = int(np.searchsorted(cum, top_p, side="left")) + 1
    n_keep = min(max(n_keep, 1), n)
    keep = np.zeros(n, dtype=bool)
    keep[order[:n_keep]] = True
    return keep


def min_p_mask(q: np.ndarray, min_p: float) -> np.ndarray:
    """Boolean mask of the tokens min-p keeps: q >= min(min_p, 1) * max q."""
    if min_p <= 0.0:
        return np.ones(q.shape[0], dtype=bool)
    return q >= min(min_p, 1.0) * np.max(q)


def sample(logits, temperature: float, top_p: float, u: float, min_p: float = 0.0) -> dict:
    """Sample one token id.  u in [0, 1) is the generator's draw.

    Returns dict(token, n_kept, kept_sum, r, gap, cut_gap, min_p_gap) where
    gap is the smallest distance, relative to kept_sum, between r and a
    running-sum boundary of the roulette; cut_gap the distance between top_p
    and the nearer of the two descending cumulative shares around the top-p
    cut (inf when top_p >= 1 keeps everything); min_p_gap the smallest
    relative distance of a weight from the min-p threshold (inf without
    min-p).  A test uses them to spot draws that sit on a boundary.
    """
    l = np.asarray(logits, dtype=np.float64)
    if temperature <= 0.0:
        return dict(token=argmax(l), n_kept=1, kept_sum=1.0, r=0.0, gap=np.inf,
                    cut_gap=np.inf, min_p_gap=np.inf)
    q = np.exp((l - np.max(l)) / temperature)
    keep = nucleus(q, top_p) & min_p_mask(q, min_p)
    kept_idx = np.nonzero(keep)[0]                 # index order
    running = np.cumsum(q[kept_idx])
    S = running[-1]
    r = u * S
    pos = int(np.searchsorted(running, r, side="left"))   # first running >= r
    tok = int(kept_idx[min(pos, kept_idx.size - 1)])
    gap = float(np.min(np.abs(running - r)) / S)
    mgap = np.inf
    if min_p > 0.0:
        thr = min(min_p, 1.0) * np.max(q)
        mgap = float(np.min(np.abs(q - thr)) / thr)
    return dict(token=tok, n_kept=int(kept_idx.size), kept_sum=float(S),
                r=float(r), gap=gap, cut_gap=nucleus_cut_gap(q, top_p), min_p_gap=mgap)


def nucleus_cut_gap(q: np.ndarray, top_p: float) -> float:
    """Distance between top_p and the descending cumulative shares on either
    side of the top-p cut: the cut keeps n tokens, so the shares after n - 1
    and after n tokens straddle top_p; the smaller distance is how far the
    weights may move before the cut moves.  inf when top_p >= 1."""
    if top_p >= 1.0:
        return float("inf")
    n = q.shape[0]
    order = np.lexsort((np.arange(n), -q))
    cum = np.cumsum(q[order]) / np.sum(q)
    n_keep = min(max(int(np.searchsorted(cum, top_p, side="left")) + 1, 1), n)
    hi = cum[n_keep - 1]
    lo = cum[n_keep - 2] if n_keep >= 2 else 0.0
    return float(min(abs(hi - top_p), abs(top_p - lo)))
