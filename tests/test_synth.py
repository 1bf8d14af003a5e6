"""The seeded input generators: determinism, shapes, value distribution."""
import numpy as np
import torch

import synth


def test_layer_weights_deterministic_and_shaped():
    s = synth.WORKLOADS["tiny_stack"].layer
    a = synth.layer_weights(s, 1001, layer=0)
    b = synth.layer_weights(s, 1001, layer=0)
    c = synth.layer_weights(s, 1001, layer=1)
    for k, shp in synth.layer_tensor_shapes(s).items():
        assert tuple(a[k].shape) == shp and a[k].dtype == torch.float32
        assert torch.equal(a[k], b[k])
        assert not torch.equal(a[k], c[k])
    assert abs(a["router"].std().item() - 0.02) < 1e-3
    assert abs(a["attn_norm"].mean().item() - 1.0) < 5e-3


def test_bf16_storage_is_round_to_nearest_even():
    s = synth.LayerShape(hidden=64, n_heads=2, head_dim=16, qkv_rank=16, window=8,
                         n_experts=4, top_k=2, ffn_inter=32)
    w = synth.layer_weights(s, 5)
    assert w["wo"].dtype == torch.bfloat16
    bits = synth.to_host(w["wo"])
    assert bits.dtype == np.uint16
    # redraw in fp32 and round by hand (RNE on the low 16 bits)
    f = synth.normal((64, 32), (5, 0, 3), "cpu", 0.0, 0.02, torch.float32).numpy()
    u = f.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(bits, rne)


def test_hidden_attempts_replace_rows():
    base = synth.hidden(6, 8, 3)
    att = np.array([0, 2, 0, 1, 0, 2])
    h = synth.hidden(6, 8, 3, attempts=att)
    assert torch.equal(h[[0, 2, 4]], base[[0, 2, 4]])
    assert not torch.equal(h[1], base[1])
    assert torch.equal(h[1], synth.normal((6, 8), (3, 7001, 0, 2))[1])
    assert torch.equal(h[3], synth.normal((6, 8), (3, 7001, 0, 1))[3])


def test_token_ids_range():
    ids = synth.token_ids(1000, 129280, 1004)
    assert ids.dtype == np.int32 and ids.min() >= 0 and ids.max() < 129280
    assert np.array_equal(ids, synth.token_ids(1000, 129280, 1004))


def test_workloads_match_rebuild_log():
    import os
    g = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "rebuild_log_tokens.txt")):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            g[k] = int(v)
    w = synth.WORKLOADS["stack43_resume"]
    assert w.prompt == g["live"] and w.snapshot_at == g["common"]
    assert w.prompt - w.snapshot_at == 148
