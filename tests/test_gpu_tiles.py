"""The dense-GEMM tile choices at the token counts where they change, on one
full-size layer (expert inter 512, as in the 43-layer stack).

Around 16 384 - 20 480 tokens the one-shot prefill switches between tile
shapes: QKV-A and the split-K router run a single pass of 320x256 tiles when
256x256 tiles would need one round of 256 blocks and a few more but 320-row
tiles fit one round (16 385..20 480 tokens), W_o and the shared down run
320x256 tiles over their whole rounds and 128x128 tiles past them.  A
prefill in 2048-token chunks runs every GEMM on 128x128 and 64-row tiles.
Each output element sums its K products in the same order under every
tiling (and the split-K router in the same slices), so the one-shot and the
chunked prefill must agree bit for bit: outputs, ring and routing.  The
oracle parity of these shapes is covered at 16 994 tokens by the 43-layer
stack test; this one pins the tile boundaries themselves.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from tests.harness import log

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


@pytest.fixture(scope="module")
def layer():
    import moe_dsv4_layer_amd as ds4g
    s = dataclasses.replace(synth.WORKLOADS["layer_decode"].layer, ffn_inter=512)
    cfg = ds4g.make_cfg(s)
    w = synth.layer_weights(s, 1101, layer=0, device="cuda")
    cw = ds4g.make_weights(w)
    img = ds4g.make_f16_images(cfg, cw, "cuda")
    cwi = ds4g.make_weights(w, img)
    return ds4g, s, cfg, w, img, cwi


def _prefill(ds4g, s, cfg, cwi, h, chunk, ws):
    T = h.shape[0]
    rk = torch.zeros((s.window, s.head_dim), dtype=torch.float16, device="cuda")
    rv = torch.zeros_like(rk)
    pos = torch.zeros(1, dtype=torch.int64, device="cuda")
    ring = ds4g.make_ring(rk, rv, pos)
    x = h.clone()
    tk = torch.full((T, s.top_k), -1, dtype=torch.int32, device="cuda")
    for c0 in range(0, T, chunk):
        n = min(chunk, T - c0)
        bufs = {"topk_idx": tk[c0:c0 + n]}
        ds4g.layer_prefill(cfg, cwi, ring, x[c0:c0 + n], n, ws, ds4g.make_routing(bufs))
    torch.cuda.synchronize()
    return x, rk, rv, int(pos.item()), tk


@pytest.mark.parametrize("T", [16385, 20480, 20481])
def test_one_shot_equals_chunks_at_tile_boundaries(layer, T):
    ds4g, s, cfg, w, img, cwi = layer
    log(f"tiles: T={T}")
    h = synth.hidden(T, s.hidden, 1100 + T, device="cuda")
    ws = ds4g.alloc_workspace(ds4g.workspace_bytes(cfg, T))
    one = _prefill(ds4g, s, cfg, cwi, h, T, ws)
    chk = _prefill(ds4g, s, cfg, cwi, h, 2048, ws)
    assert torch.isfinite(one[0]).all()
    assert torch.equal(one[0], chk[0]), f"T={T}: one-shot and chunked outputs differ"
    assert torch.equal(one[1], chk[1]) and torch.equal(one[2], chk[2]), f"T={T}: rings differ"
    assert one[3] == chk[3] == T
    assert torch.equal(one[4], chk[4]), f"T={T}: expert choices differ"
    tk = one[4].cpu().numpy()
    assert tk.min() >= 0 and tk.max() < s.n_experts
    assert all(len(set(r)) == s.top_k for r in tk[:: max(1, T // 512)].tolist())
    log(f"tiles: T={T} one-shot == 2048-token chunks (output, ring, routing)")
    del ws
    torch.cuda.empty_cache()
