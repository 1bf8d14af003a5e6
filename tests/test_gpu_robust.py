"""Non-finite inputs must never turn into out-of-range indices.

Routing (prefill top-k, decode per-wave top-k) and the sampler derive array
indices from floating-point scores.  With NaN or infinite activations every
expert index must still lie in [0, E), the grouping must still cover T*k
entries, and the sampled token must still be a vocabulary id.  The values
themselves are not checked: NaN in, NaN out."""
import numpy as np
import pytest
import torch

import synth
from tests.harness import GpuLayer, log, small_shape

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import moe_dsv4_layer_amd as ds4g


def _poison(h: torch.Tensor) -> torch.Tensor:
    h = h.clone()
    h[3] = float("nan")
    h[7, ::5] = float("inf")
    h[11, 1::3] = float("-inf")
    return h


def _check_routing(bufs, T, k, E):
    idx = bufs["topk_idx"].cpu().numpy()
    assert idx.shape == (T, k)
    assert idx.min() >= 0 and idx.max() < E, idx
    for t in range(T):
        assert len(set(idx[t].tolist())) == k, (t, idx[t])
    cnt = bufs["expert_count"].cpu().numpy()
    off = bufs["expert_offset"].cpu().numpy()
    assert cnt.min() >= 0 and int(cnt.sum()) == T * k
    assert off[0] == 0 and int(off[-1]) == T * k
    perm = bufs["perm"].cpu().numpy()
    assert sorted(perm.tolist()) == list(range(T * k))


def test_nonfinite_prefill_and_decode_keep_indices_in_range():
    shape = small_shape()
    T = 40
    gl = GpuLayer(shape, seed=21, max_tokens=T)
    h = _poison(synth.hidden(T, shape.hidden, 21, device="cuda"))
    log(f"non-finite prefill T={T}")
    x, bufs = gl.prefill(h)
    _check_routing(bufs, T, shape.top_k, shape.n_experts)
    log("non-finite decode")
    xd, bd = gl.decode(torch.full((shape.hidden,), float("nan"), device="cuda"))
    _check_routing(bd, 1, shape.top_k, shape.n_experts)
    assert int(gl.pos.item()) == T + 1


@pytest.mark.parametrize("temperature", [0.0, 0.7])
def test_nonfinite_logits_sample_a_vocabulary_id(temperature):
    hidden, vocab = 256, 5000
    shape = synth.LayerShape(hidden=hidden, n_heads=1, head_dim=64, qkv_rank=64, window=1,
                             n_experts=2, top_k=1, ffn_inter=64, wdtype=synth.BF16)
    hw = synth.head_weights(shape, vocab, 5, device="cuda")
    ws = ds4g.alloc_workspace(ds4g.workspace_bytes(None, 0, vocab))
    logits = torch.empty(vocab, dtype=torch.float32, device="cuda")
    token = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rng = torch.tensor([12345], dtype=torch.int64, device="cuda")
    for x in (torch.full((hidden,), float("nan"), device="cuda"),
              torch.full((hidden,), float("inf"), device="cuda")):
        log(f"non-finite lm_head x={float(x[0])} T={temperature}")
        ds4g.lmhead_sample(hidden, vocab, ds4g.BF16, hw["final_norm"], shape.rms_eps,
                           hw["lm_head"], x, temperature, 0.9, rng, logits, token, ws)
        torch.cuda.synchronize()
        tok = int(token.item())
        assert 0 <= tok < vocab, tok
