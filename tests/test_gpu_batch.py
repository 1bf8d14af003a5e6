"""GPU parity of ds4g_layer_decode_batch: one decode token of each of B
independent sequences, each with its own ring and position, against the
float64 oracle run on every sequence separately (阶段四 4.2 for each token),
and against the single-sequence decode call."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import check_routing, log, rel_l2, small_shape, to_np

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import moe_dsv4_layer_amd as ds4g

LAYER_TOL = 1e-2


def _routing_bufs(shape, B):
    return {
        "topk_idx": torch.full((B, shape.top_k), -1, dtype=torch.int32, device="cuda"),
        "topk_w": torch.zeros((B, shape.top_k), dtype=torch.float32, device="cuda"),
        "expert_count": torch.full((shape.n_experts,), -1, dtype=torch.int32, device="cuda"),
        "expert_offset": torch.full((shape.n_experts + 1,), -1, dtype=torch.int32, device="cuda"),
        "perm": torch.full((B * shape.top_k,), -1, dtype=torch.int32, device="cuda"),
        "router_in": torch.zeros((B, shape.hidden), dtype=torch.float32, device="cuda"),
        "router_logits": torch.zeros((B, shape.n_experts), dtype=torch.float32, device="cuda"),
    }


class Batch:
    """B sequences sharing one layer's weights; rings [B, W, dh], pos [B]."""

    def __init__(self, shape, seed, hist):
        self.shape, self.hist, self.B = shape, hist, len(hist)
        self.w = synth.layer_weights(shape, seed, layer=0, device="cuda")
        self.cfg, self.cw = ds4g.make_cfg(shape), ds4g.make_weights(self.w)
        dh, W = shape.head_dim, shape.window
        self.rk = torch.zeros((self.B, W, dh), dtype=torch.float16, device="cuda")
        self.rv = torch.zeros_like(self.rk)
        self.pos = torch.zeros(self.B, dtype=torch.int64, device="cuda")
        self.rings = ds4g.make_ring(self.rk, self.rv, self.pos)
        self.ws = ds4g.alloc_workspace(ds4g.workspace_bytes(self.cfg, max(max(hist), self.B)))
        self.wh = synth.weights_to_host(self.w)
        self.orc = [oracle.Ring(W, dh) for _ in hist]
        self.h = [synth.hidden(n + 4, shape.hidden, seed, stream=b, device="cuda")
                  for b, n in enumerate(hist)]
        # each sequence's history: GPU prefill into its own ring, oracle alike
        for b, n in enumerate(hist):
            if n == 0:
                continue
            ring_b = ds4g.make_ring(self.rk[b], self.rv[b], self.pos[b:b + 1])
            x = self.h[b][:n].clone()
            ds4g.layer_prefill(self.cfg, self.cw, ring_b, x, n, self.ws)
            oracle.layer_forward(shape, self.wh, self.orc[b], self.h[b][:n].cpu().numpy())
        torch.cuda.synchronize()

    def step(self, j):
        """Decode token j of every sequence (input h[b][hist[b] + j])."""
        B = self.B
        xin = torch.stack([self.h[b][self.hist[b] + j] for b in range(B)]).contiguous()
        x = xin.clone()
        bufs = _routing_bufs(self.shape, B)
        ds4g.layer_decode_batch(self.cfg, self.cw, self.rings, x, B, self.ws,
                                ds4g.make_routing(bufs))
        torch.cuda.synchronize()
        outs = [oracle.layer_forward(self.shape, self.wh, self.orc[b],
                                     xin[b:b + 1].cpu().numpy()) for b in range(B)]
        return xin, x, bufs, outs


def _check_step(label, bt, xin, x, bufs, outs):
    g = to_np(bufs)
    out = x.cpu().numpy().astype(np.float64)
    hh = xin.cpu().numpy().astype(np.float64)
    for b in range(bt.B):
        o = outs[b]
        e_out = rel_l2(out[b], o["out"][0])
        e_inc = rel_l2(out[b] - hh[b], o["out"][0] - hh[b])
        assert e_out < LAYER_TOL and e_inc < LAYER_TOL, (label, b, e_out, e_inc)
    # routing of all rows at once: the oracle's y/logits stacked row by row
    orc = {k: np.concatenate([o[k] for o in outs]) for k in outs[0] if k in
           ("y", "logits", "topk_idx", "topk_w", "out", "margin")}
    st = check_routing(bt.shape, bt.wh, g, orc, label=label)
    log(f"{label}: rows within {LAYER_TOL} of the oracle; routing {st}")


def test_batch_small_bf16_mixed_histories():
    # empty ring, short, exactly one window, and wrapped histories
    bt = Batch(small_shape(), 31, hist=[0, 3, 15, 16, 40])
    pos0 = bt.pos.cpu().numpy().copy()
    for j in range(3):
        xin, x, bufs, outs = bt.step(j)
        _check_step(f"batch step {j}", bt, xin, x, bufs, outs)
    assert (bt.pos.cpu().numpy() == pos0 + 3).all()
    # ring contents: every sequence's ring equals its oracle ring
    for b in range(bt.B):
        assert rel_l2(bt.rk[b].float().cpu().numpy(), bt.orc[b].k) < 1e-2
        assert rel_l2(bt.rv[b].float().cpu().numpy(), bt.orc[b].v) < 1e-2


@pytest.mark.parametrize("hist", [[9], [7, 0], [3, 0, 17, 1, 16, 5, 0, 2, 30, 8, 12, 4]],
                         ids=["B1", "B2", "B12"])
def test_batch_sizes_bf16(hist):
    # B = 1 and 2: the multi-row GEMV with rows masked; B = 12: past its
    # 8-row limit, the split-K GEMM path
    bt = Batch(small_shape(), 33, hist=hist)
    for j in range(2):
        xin, x, bufs, outs = bt.step(j)
        _check_step(f"batch of {len(hist)}, step {j}", bt, xin, x, bufs, outs)


def test_batch_fp32_weights():
    bt = Batch(small_shape(wdtype=synth.F32), 32, hist=[5, 0, 21])
    xin, x, bufs, outs = bt.step(0)
    _check_step("batch fp32", bt, xin, x, bufs, outs)


def test_batch_matches_single_decode_full_size():
    # the full-size layer: B sequences at position 128 (ring full); the
    # batched call against the single-sequence decode of the same inputs,
    # and against the oracle for one of them
    wl = synth.WORKLOADS["layer_decode"]
    s = wl.layer
    B = 6
    cfg = ds4g.make_cfg(s)
    w = synth.layer_weights(s, wl.seed, layer=0, device="cuda")
    cw = ds4g.make_weights(w)
    W, dh = s.window, s.head_dim
    rk = torch.zeros((B, W, dh), dtype=torch.float16, device="cuda")
    rv = torch.zeros_like(rk)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    ws = ds4g.alloc_workspace(ds4g.workspace_bytes(cfg, W))
    hs = [synth.hidden(W + 1, s.hidden, wl.seed, stream=b, device="cuda") for b in range(B)]
    for b in range(B):
        x = hs[b][:W].clone()
        ds4g.layer_prefill(cfg, cw, ds4g.make_ring(rk[b], rv[b], pos[b:b + 1]), x, W, ws)
    torch.cuda.synchronize()
    # single decodes on copies of the rings
    rk1, rv1, pos1 = rk.clone(), rv.clone(), pos.clone()
    single = []
    for b in range(B):
        x = hs[b][W].clone()
        ds4g.layer_decode(cfg, cw, ds4g.make_ring(rk1[b], rv1[b], pos1[b:b + 1]), x, ws)
        single.append(x)
    xin = torch.stack([hs[b][W] for b in range(B)]).contiguous()
    xb = xin.clone()
    ds4g.layer_decode_batch(cfg, cw, ds4g.make_ring(rk, rv, pos), xb, B, ws)
    torch.cuda.synchronize()
    xs = torch.stack(single)
    e = rel_l2((xb - xin).cpu().numpy(), (xs - xin).cpu().numpy())
    log(f"full-size batch B={B} vs single decode: increment rel_l2 {e:.2e}")
    assert e < LAYER_TOL
    assert (pos.cpu().numpy() == W + 1).all() and torch.equal(pos, pos1)
    assert rel_l2(rk.float().cpu().numpy(), rk1.float().cpu().numpy()) < 1e-2
    # one sequence against the oracle
    wh = synth.weights_to_host(w)
    ring = oracle.Ring(W, dh)
    oracle.layer_forward(s, wh, ring, hs[0][:W].cpu().numpy())
    o = oracle.layer_forward(s, wh, ring, hs[0][W:W + 1].cpu().numpy())
    e0 = rel_l2(xb[0].cpu().numpy(), o["out"][0])
    log(f"full-size batch row 0 vs oracle: rel_l2 {e0:.2e}")
    assert e0 < LAYER_TOL
