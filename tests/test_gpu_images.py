"""Prepared fp16 images (ds4g_make_f16_images): a prefill or batched decode
that reads the layer's prepared images must give exactly the results of the
same call making the images in its workspace (same bits in, same kernels)."""
import pytest
import torch

import synth
from tests.harness import GpuLayer, log

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def test_prepared_images_prefill_bit_identical():
    import moe_dsv4_layer_amd as ds4g
    shape = synth.WORKLOADS["layer_prefill_2048"].layer
    T = 300
    gl = GpuLayer(shape, seed=71, max_tokens=T)
    img = ds4g.make_f16_images(gl.cfg, gl.cw)
    cw_img = ds4g.make_weights(gl.w, img)
    h = synth.hidden(T, shape.hidden, 71, device="cuda")
    x1, x2 = h.clone(), h.clone()
    ds4g.layer_prefill(gl.cfg, gl.cw, gl.ring, x1, T, gl.ws)
    k1, v1 = gl.ring_k.clone(), gl.ring_v.clone()
    gl.pos.zero_()
    ds4g.layer_prefill(gl.cfg, cw_img, gl.ring, x2, T, gl.ws)
    torch.cuda.synchronize()
    assert torch.equal(x1, x2) and torch.equal(k1, gl.ring_k) and torch.equal(v1, gl.ring_v)
    log(f"prepared images: {img.numel()} bytes; prefill of {T} tokens bit-identical")


@pytest.mark.parametrize("B", [8, 32])
def test_prepared_images_batch_bit_identical(B):
    import moe_dsv4_layer_amd as ds4g
    shape = synth.WORKLOADS["layer_decode"].layer
    w = synth.layer_weights(shape, 72, device="cuda")
    cfg = ds4g.make_cfg(shape)
    img = ds4g.make_f16_images(cfg, ds4g.make_weights(w))
    ws = ds4g.alloc_workspace(ds4g.workspace_bytes(cfg, B))
    outs = []
    for cw in (ds4g.make_weights(w), ds4g.make_weights(w, img)):
        rk = torch.zeros((B, shape.window, shape.head_dim), dtype=torch.float16, device="cuda")
        rv = torch.zeros_like(rk)
        pos = torch.full((B,), 5, dtype=torch.int64, device="cuda")
        x = synth.hidden(B, shape.hidden, 72, device="cuda")
        ds4g.layer_decode_batch(cfg, cw, ds4g.make_ring(rk, rv, pos), x, B, ws)
        torch.cuda.synchronize()
        outs.append((x, rk, rv, pos))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
