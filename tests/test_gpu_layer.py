"""GPU parity of the layer (prefill and decode) against the float64 oracle,
through the C ABI.  Shapes: small ones that span several GEMM tiles, a
ragged tail and ring wrap-around; fp32 weights; and the full-size layer."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import GpuLayer, check_routing, log, rel_l2, small_shape, to_np

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

LAYER_TOL = 1e-2       # rel-L2 per layer output (and per increment out - h)


def _oracle_ring(shape):
    return oracle.Ring(shape.window, shape.head_dim)


def _compare_layer(label, shape, gl, h, x_gpu, bufs, orc, rows=None):
    g = to_np(bufs)
    out = x_gpu.cpu().numpy().astype(np.float64)
    hh = h.cpu().numpy().astype(np.float64)
    if rows is None:
        rows = np.arange(out.shape[0])
    e_out = rel_l2(out[rows], orc["out"][rows])
    e_inc = rel_l2(out[rows] - hh[rows], orc["out"][rows] - hh[rows])
    e_y = rel_l2(g["router_in"], orc["y"])
    st = check_routing(shape, gl.host_weights(), g, orc, label=label)
    log(f"{label}: rel_l2 out={e_out:.2e} inc={e_inc:.2e} y={e_y:.2e} routing={st}")
    assert e_y < LAYER_TOL, (label, e_y)
    assert e_out < LAYER_TOL, (label, e_out)
    assert e_inc < LAYER_TOL, (label, e_inc)
    return e_out, e_inc


@pytest.mark.parametrize("T", [1, 40, 300])
def test_prefill_small_bf16(T):
    shape = small_shape()
    log(f"prefill small bf16 T={T}")
    gl = GpuLayer(shape, seed=11, max_tokens=T)
    h = synth.hidden(T, shape.hidden, 11, device="cuda")
    x, bufs = gl.prefill(h)
    ring = _oracle_ring(shape)
    orc = oracle.layer_forward(shape, gl.host_weights(), ring, h.cpu().numpy())
    _compare_layer(f"prefill T={T}", shape, gl, h, x, bufs, orc)
    assert int(gl.pos.item()) == T
    # ring contents: the last min(T, W) positions, keys after RoPE
    rk = gl.ring_k.float().cpu().numpy()
    rv = gl.ring_v.float().cpu().numpy()
    assert rel_l2(rk, ring.k) < 1e-2 and rel_l2(rv, ring.v) < 1e-2


def test_decode_small_bf16_wraps_ring():
    shape = small_shape()
    n_pre, n_dec = 20, 25
    log("decode small bf16")
    gl = GpuLayer(shape, seed=12, max_tokens=n_pre)
    h = synth.hidden(n_pre + n_dec, shape.hidden, 12, device="cuda")
    ring = _oracle_ring(shape)
    wh = gl.host_weights()
    x, bufs = gl.prefill(h[:n_pre])
    orc = oracle.layer_forward(shape, wh, ring, h[:n_pre].cpu().numpy())
    _compare_layer("decode-prefix", shape, gl, h[:n_pre], x, bufs, orc)
    for t in range(n_pre, n_pre + n_dec):
        x, bufs = gl.decode(h[t])
        orc = oracle.layer_forward(shape, wh, ring, h[t:t + 1].cpu().numpy())
        bufs = {k: v.reshape((1,) + tuple(v.shape[1:])) if v.dim() >= 1 and k in
                ("topk_idx", "topk_w", "router_in", "router_logits") else v
                for k, v in bufs.items()}
        _compare_layer(f"decode pos={t}", shape, gl, h[t:t + 1], x.reshape(1, -1), bufs, orc)
    assert int(gl.pos.item()) == n_pre + n_dec


def test_prefill_matches_decode_on_gpu():
    # layer-major prefill and token-by-token decode compute the same layer
    shape = small_shape()
    T = 24
    h = synth.hidden(T, shape.hidden, 13, device="cuda")
    a = GpuLayer(shape, seed=13, max_tokens=T)
    b = GpuLayer(shape, seed=13, max_tokens=T)
    xa, _ = a.prefill(h)
    xb = torch.stack([b.decode(h[t])[0] for t in range(T)])
    e = rel_l2((xb - h).cpu().numpy(), (xa - h).cpu().numpy())
    log(f"prefill vs decode increment rel_l2 {e:.2e}")
    assert e < LAYER_TOL


def test_fp32_weights_tiny_stack_layer():
    # the tiny stack's layer: fp32 weights, window 128, 8 experts top-2
    shape = synth.WORKLOADS["tiny_stack"].layer
    T, n_dec = 64, 16
    gl = GpuLayer(shape, seed=1001, max_tokens=T)
    h = synth.hidden(T + n_dec, shape.hidden, 1001, device="cuda")
    ring = _oracle_ring(shape)
    wh = gl.host_weights()
    x, bufs = gl.prefill(h[:T])
    orc = oracle.layer_forward(shape, wh, ring, h[:T].cpu().numpy())
    _compare_layer("fp32 prefill", shape, gl, h[:T], x, bufs, orc)
    for t in range(T, T + n_dec):
        x, bufs = gl.decode(h[t])
        orc = oracle.layer_forward(shape, wh, ring, h[t:t + 1].cpu().numpy())
        bufs = {k: v.reshape(1, -1) if k in ("topk_idx", "topk_w", "router_in",
                                             "router_logits") else v for k, v in bufs.items()}
        _compare_layer(f"fp32 decode pos={t}", shape, gl, h[t:t + 1], x.reshape(1, -1),
                       bufs, orc)


LIMIT_SHAPES = {
    # the largest supported routing (512 experts, top-8), the longest window,
    # head_dim 128 with RoPE on its last 64 entries only
    "limits": (dict(hidden=256, n_heads=4, head_dim=128, qkv_rank=64, window=128,
                    n_experts=512, top_k=8, ffn_inter=64, rope_dim=64), 300),
    # degenerate: a window of one (each token attends to itself only) and
    # top-8 of 9 experts
    "degenerate": (dict(hidden=128, n_heads=4, head_dim=64, qkv_rank=64, window=1,
                        n_experts=9, top_k=8, ffn_inter=64), 40),
}


@pytest.mark.parametrize("name", sorted(LIMIT_SHAPES))
def test_prefill_and_decode_at_the_limits(name):
    dims, T = LIMIT_SHAPES[name]
    shape = synth.LayerShape(wdtype=synth.BF16, **dims)
    n_dec = 3
    log(f"{name}: prefill {T} + {n_dec} decode steps")
    gl = GpuLayer(shape, seed=14, max_tokens=T)
    h = synth.hidden(T + n_dec, shape.hidden, 14, device="cuda")
    ring = _oracle_ring(shape)
    wh = gl.host_weights()
    x, bufs = gl.prefill(h[:T])
    orc = oracle.layer_forward(shape, wh, ring, h[:T].cpu().numpy())
    _compare_layer(f"{name} prefill", shape, gl, h[:T], x, bufs, orc)
    for t in range(T, T + n_dec):
        x, bufs = gl.decode(h[t])
        orc = oracle.layer_forward(shape, wh, ring, h[t:t + 1].cpu().numpy())
        bufs = {k: v.reshape(1, -1) if k in ("topk_idx", "topk_w", "router_in",
                                             "router_logits") else v for k, v in bufs.items()}
        _compare_layer(f"{name} decode pos={t}", shape, gl, h[t:t + 1], x.reshape(1, -1), bufs,
                       orc)
    assert int(gl.pos.item()) == T + n_dec
    assert rel_l2(gl.ring_k.float().cpu().numpy(), ring.k) < 1e-2
