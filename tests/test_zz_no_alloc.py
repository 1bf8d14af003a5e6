"""ds4g_layer_decode_noalloc (the decode step on the library's static
scratch, for callers that cannot allocate) against ds4g_layer_decode with a
caller workspace.  Both run the same kernels on the same inputs, so every
output must agree bit for bit: the layer output, the ring, the position and
the routing outputs.  Two calls in a row: a full-size layer, then a smaller
layer (less scratch) on the same array."""
import ctypes

import pytest
import torch

import synth
from tests.harness import GpuLayer, log, small_shape

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _decode_both(shape, seed, npre):
    import moe_dsv4_layer_amd as ds4g
    log(f"noalloc: hidden {shape.hidden}, {npre} positions prefilled, seed {seed}")
    gl = GpuLayer(shape, seed=seed, max_tokens=npre)
    h = synth.hidden(npre + 1, shape.hidden, seed, device="cuda")
    gl.prefill(h[:npre])
    rk2, rv2, pos2 = gl.ring_k.clone(), gl.ring_v.clone(), gl.pos.clone()
    ring2 = ds4g.make_ring(rk2, rv2, pos2)
    # the existing entry point, with its workspace
    x1 = h[npre].clone()
    b1, r1 = gl._routing(1)
    ds4g.layer_decode(gl.cfg, gl.cw, gl.ring, x1, gl.ws, r1)
    # the entry point without one, through the C ABI
    x2 = h[npre].clone()
    b2, r2 = gl._routing(1)
    rc = ds4g.lib.ds4g_layer_decode_noalloc(ctypes.byref(gl.cfg), ctypes.byref(gl.cw),
                                            ctypes.byref(ring2), x2.data_ptr(), ctypes.byref(r2),
                                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == ds4g.OK, ds4g.status_string(rc)
    assert torch.equal(x1, x2)
    assert torch.equal(gl.ring_k, rk2) and torch.equal(gl.ring_v, rv2)
    assert int(gl.pos.item()) == int(pos2.item()) == npre + 1
    for n in b1:
        assert torch.equal(b1[n], b2[n]), n
    log(f"  bit-identical; |x| = {float(x2.norm()):.4f}")


def test_noalloc_decode_matches_workspace_decode_twice():
    _decode_both(synth.WORKLOADS["layer_decode"].layer, 1002, 128)
    _decode_both(small_shape(), 7, 40)
