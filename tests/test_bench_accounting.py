"""The byte and flop accounting behind bench.py's roofline, checked on the CPU:
the formulas against the sizes of the tensors the seeded generator actually
builds, the full-size decode figure, and the stored HBM-traffic measurement
against the decode sources it was taken on."""
import importlib.util
import os

import pytest

import synth
from tests.harness import small_shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _bytes(t):
    return t.numel() * t.element_size()


def test_prefill_weight_bytes_is_every_weight_of_the_layer():
    b = _bench()
    sh = small_shape()
    w = synth.layer_weights(sh, 3, layer=0, device="cpu")
    assert b.prefill_weight_bytes(sh) == sum(_bytes(t) for t in w.values())


def test_layer_decode_bytes_is_what_one_token_touches():
    # one token reads every dense weight, the router, k routed experts and the
    # shared expert (gate, up, down each), the two norm gains, the K/V window
    # (bf16) and its fp32 activation vector in and out
    b = _bench()
    sh = small_shape()
    w = synth.layer_weights(sh, 3, layer=0, device="cpu")
    dense = sum(_bytes(w[n]) for n in ("attn_norm", "qkv_a", "qkv_b", "wo", "ffn_norm", "router",
                                       "sh_gate", "sh_up", "sh_down"))
    per_expert = sum(_bytes(w[n][0]) for n in ("gate", "up", "down"))
    kv = 2 * sh.window * sh.head_dim * 2
    act = 2 * 4 * sh.hidden
    assert b.layer_decode_bytes(sh) == dense + sh.top_k * per_expert + kv + act


def test_full_size_decode_bytes():
    b = _bench()
    assert b.layer_decode_bytes(synth.WORKLOADS["layer_decode"].layer) == 271_171_584


def test_stored_decode_traffic_matches_the_sources():
    # the counter measurement in bench.py is tied to a hash of the decode
    # sources (bench.py then reports traffic as null); a change to them
    # without a new measurement shows up here as a skip
    b = _bench()
    if b.decode_traffic() is None:
        pytest.skip("decode sources changed since the HBM traffic was measured")
    assert b.decode_traffic() == b.DECODE_TRAFFIC_BYTES
    assert abs(b.DECODE_TRAFFIC_BYTES / b.layer_decode_bytes(synth.WORKLOADS["layer_decode"].layer)
               - 1.0) < 0.05   # the measured bytes stay within 5% of the algorithmic ones
