"""Step-by-step (teacher-forced) parity of a prefill: every kernel of the
layer is checked on its own.  ds4g_layer_prefill_trace copies each step's
output (x_norm, c, q, k, v, o, h2, and through the routing outputs y and the
router logits); the oracle applies that one step (阶段四 4.2) to the GPU's
copy of the step's input, so each comparison sees only that kernel's
arithmetic.  Bounds follow from what the step rounds:
  * an fp16 output (bf16-weight path: x_norm, c, q, k, v, o) is within half
    an fp16 ulp (2^-11 relative) of the fp32 value, plus fp32 accumulation;
  * the attention output also carries the fp16 rounding of its
    probabilities: at most 2^-11 of sum_j p_j |v_j| per element, counted
    twice (the normaliser adds the unrounded weights);
  * fp32 outputs (h2, y, logits) differ only by fp32 accumulation;
  * every product sum carries the usual dot-product bound, (number of
    roundings) x 2^-24 x sum |terms|: the matrix cores add 16 products per
    step, then round into the accumulator, so K / 16 + 16 roundings;
  * the routed and shared experts take bf16 inputs and round z and each
    routed output to bf16, so the MoE increment is held to the layer's 1e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import GpuLayer, log, rel_l2, small_shape

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

U16 = 2.0 ** -11      # half an fp16 ulp, relative
U32 = 2.0 ** -24      # half an fp32 ulp, relative


def _dot_bound(a, b):
    """Accumulation bound of a @ b.T in fp32: (K / 16 + 16) * 2^-24 * |a| @ |b|.T."""
    K = a.shape[-1]
    return (K / 16 + 16) * U32 * (np.abs(a) @ np.abs(b).T)


def _f16(t):
    return t.view(torch.float16).float().cpu().numpy().astype(np.float64)


def _act(t, f16):
    return _f16(t) if f16 else t.cpu().numpy().astype(np.float64)


def _close(label, got, ref, rel_bound, scale=None):
    """Elementwise |got - ref| <= rel_bound |ref| + scale (the step's
    accumulation bound) + the smallest fp16 step; returns the rel-L2."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    lim = rel_bound * (np.abs(ref) + (0 if scale is None else scale)) + 2.0 ** -25
    if scale is not None:
        lim = lim + scale
    bad = np.abs(got - ref) > lim
    assert not bad.any(), (label, int(bad.sum()), float((np.abs(got - ref) / lim).max()))
    return rel_l2(got, ref)


def _run(shape, seed, T):
    import moe_dsv4_layer_amd as ds4g
    f16 = shape.wdtype == synth.BF16
    gl = GpuLayer(shape, seed=seed, max_tokens=T)
    h = synth.hidden(T, shape.hidden, seed, device="cuda")
    adt = torch.int16 if f16 else torch.float32
    qd, dh = shape.q_dim, shape.head_dim
    tr = {"x_norm": torch.empty((T, shape.hidden), dtype=adt, device="cuda"),
          "c": torch.empty((T, shape.qkv_rank), dtype=adt, device="cuda"),
          "q": torch.empty((T, qd), dtype=adt, device="cuda"),
          "k": torch.empty((T, dh), dtype=torch.int16, device="cuda"),
          "v": torch.empty((T, dh), dtype=torch.int16, device="cuda"),
          "o": torch.empty((T, qd), dtype=adt, device="cuda"),
          "h2": torch.empty((T, shape.hidden), dtype=torch.float32, device="cuda")}
    x = h.clone()
    bufs, r = gl._routing(T)
    ds4g.layer_prefill_trace(gl.cfg, gl.cw, gl.ring, x, T, gl.ws, tr, r)
    torch.cuda.synchronize()
    w = gl.host_weights()
    W = lambda n: oracle.widen(w[n])
    hh = h.cpu().numpy().astype(np.float64)
    H, rd, eps = shape.n_heads, shape.rope_width, shape.rms_eps
    qtol = U16 if f16 else 2.0 ** -22
    res = {}
    # x_norm = RMSNorm(h) g1
    xg = _act(tr["x_norm"], f16)
    res["x_norm"] = _close("x_norm", xg, oracle.rmsnorm(hh, w["attn_norm"], eps), qtol)
    # c = A x_norm (on the GPU's x_norm)
    cg = _act(tr["c"], f16)
    res["c"] = _close("c", cg, xg @ W("qkv_a").T, qtol, _dot_bound(xg, W("qkv_a")))
    # q, k, v = B c, RoPE at positions 0..T-1 (on the GPU's c)
    qkv = cg @ W("qkv_b").T
    bqkv = _dot_bound(cg, W("qkv_b"))
    # RoPE mixes a pair: its bound is the pair's larger one, plus 3 fp32 roundings
    bpair = np.maximum(bqkv, bqkv.reshape(T, -1, 2)[:, :, ::-1].reshape(T, -1)) * 2 + \
        3 * U32 * np.abs(qkv)
    qref = np.stack([oracle.rope(qkv[t, :qd].reshape(H, dh), t, shape.rope_base, rd)
                     for t in range(T)]).reshape(T, qd)
    kref = np.stack([oracle.rope(qkv[t, qd:qd + dh], t, shape.rope_base, rd) for t in range(T)])
    vref = qkv[:, qd + dh:]
    qg, kg, vg = _act(tr["q"], f16), _f16(tr["k"]), _f16(tr["v"])
    res["q"] = _close("q", qg, qref, qtol, bpair[:, :qd])
    res["k"] = _close("k", kg, kref, U16, bpair[:, qd:qd + dh])
    res["v"] = _close("v", vg, vref, U16, bqkv[:, qd + dh:])
    # o = window attention over the GPU's q, k, v
    og = _act(tr["o"], f16)
    oref = np.empty((T, H, dh))
    pscale = np.empty((T, H, dh))
    for t in range(T):
        lo = max(0, t - shape.window + 1)
        qh = qg[t].reshape(H, dh)
        s = qh @ kg[lo:t + 1].T / np.sqrt(dh)
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        oref[t] = p @ vg[lo:t + 1]
        pscale[t] = p @ np.abs(vg[lo:t + 1])
    oref = oref.reshape(T, qd)
    extra = (2 * U16 if f16 else 2.0 ** -20) * pscale.reshape(T, qd) + \
        (dh / 16 + 16) * U32 * 4 * pscale.reshape(T, qd)
    res["o"] = _close("o", og, oref, qtol, scale=extra)
    # h2 = h + W_o o (on the GPU's o)
    h2g = tr["h2"].cpu().numpy().astype(np.float64)
    res["h2"] = _close("h2", h2g - hh, og @ W("wo").T, 0.0,
                       _dot_bound(og, W("wo")) + U32 * np.abs(h2g))
    # y = RMSNorm(h2) g2, router logits (on the GPU's h2, y)
    g = {k: v.cpu().numpy() for k, v in bufs.items()}
    yg = g["router_in"].astype(np.float64)
    res["y"] = _close("y", yg, oracle.rmsnorm(h2g, w["ffn_norm"], eps), 2.0 ** -20)
    # the router adds three bf16 terms of y (the last within 2^-27 |y|)
    blg = 3 * _dot_bound(yg, W("router")) + 2.0 ** -26 * (np.abs(yg) @ np.abs(W("router")).T)
    res["logits"] = _close("logits", g["router_logits"], yg @ W("router").T, 0.0, blg)
    # experts + combine on the GPU's y and choice of experts
    idx = g["topk_idx"].astype(np.int64)
    p = oracle.layer.softmax(yg @ W("router").T)
    inc = np.zeros_like(hh)
    for e in range(shape.n_experts):
        tt, jj = np.nonzero(idx == e)
        if tt.size:
            f = oracle.layer.swiglu_ffn(yg[tt], w["gate"][e], w["up"][e], w["down"][e])
            inc[tt] += p[tt, e][:, None] * f
    inc += oracle.layer.swiglu_ffn(yg, w["sh_gate"], w["sh_up"], w["sh_down"])
    out = x.cpu().numpy().astype(np.float64)
    res["moe"] = rel_l2(out - h2g, inc)
    log(f"steps {shape.hidden}/{shape.wdtype} T={T}: " +
        " ".join(f"{k} {v:.1e}" for k, v in res.items()))
    assert res["moe"] < 1e-2
    return res


@pytest.mark.parametrize("wdtype", [synth.BF16, synth.F32])
def test_steps_small(wdtype):
    _run(small_shape(wdtype=wdtype), 61, 40)


def test_steps_full_size():
    _run(synth.WORKLOADS["layer_prefill_2048"].layer, 62, 256)
