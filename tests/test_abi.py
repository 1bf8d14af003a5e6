"""The C-ABI library loads, exports every function include/ds4g.h declares,
and rejects bad arguments on the host before touching the device (these
calls return before any HIP call, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ds4g.h")

ds4g = pytest.importorskip("moe_dsv4_layer_amd")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(ds4g_[a-z_0-9]+)\s*\(", txt)))


def test_header_and_binding_agree():
    assert _declared() == sorted(ds4g.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ds4g.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def _cfg(**kw):
    import synth
    s = synth.WORKLOADS["layer_decode"].layer
    c = ds4g.make_cfg(s)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_status_strings():
    assert ds4g.status_string(0) == "ok"
    assert "workspace" in ds4g.status_string(-3)
    assert ds4g.status_string(99) == "unknown status"


def test_workspace_bytes():
    c = _cfg()
    n1 = ds4g.workspace_bytes(c, 1)
    n2 = ds4g.workspace_bytes(c, 2048)
    assert 0 < n1 < n2
    assert ds4g.workspace_bytes(c, 0) == 0
    assert ds4g.workspace_bytes(None, 0, 129280) > 129280 * 4
    assert ds4g.workspace_bytes(_cfg(head_dim=96), 16) == 0


P = ctypes.c_void_p


def _weights(nonnull=True):
    return ds4g.LayerWeights(*[(0x1000 if nonnull else 0) for _ in ds4g.WEIGHT_NAMES])


def _prefill(cfg, w, ring, x, T, ws, nbytes):
    return ds4g.lib.ds4g_layer_prefill(ctypes.byref(cfg) if cfg is not None else None,
                                       ctypes.byref(w) if w is not None else None,
                                       ctypes.byref(ring) if ring is not None else None,
                                       x, T, None, ws, nbytes, None)


def test_prefill_rejects_before_launch():
    c = _cfg()
    w = _weights()
    ring = ds4g.KvRing(0x1000, 0x1000, 0x1000)
    ok_ws = ds4g.workspace_bytes(c, 8)
    assert _prefill(None, w, ring, 0x1000, 8, 0x1000, ok_ws) == ds4g.ERR_INVALID_ARG
    assert _prefill(c, None, ring, 0x1000, 8, 0x1000, ok_ws) == ds4g.ERR_INVALID_ARG
    assert _prefill(c, _weights(False), ring, 0x1000, 8, 0x1000, ok_ws) == ds4g.ERR_INVALID_ARG
    assert _prefill(c, w, ds4g.KvRing(0, 0x1000, 0x1000), 0x1000, 8, 0x1000, ok_ws) == ds4g.ERR_INVALID_ARG
    assert _prefill(c, w, ring, None, 8, 0x1000, ok_ws) == ds4g.ERR_INVALID_ARG
    assert _prefill(c, w, ring, 0x1000, 0, 0x1000, ok_ws) == ds4g.ERR_INVALID_ARG
    assert _prefill(c, w, ring, 0x1000, -5, 0x1000, ok_ws) == ds4g.ERR_INVALID_ARG
    assert _prefill(c, w, ring, 0x1000, 8, 0x1004, ok_ws) == ds4g.ERR_INVALID_ARG   # misaligned ws
    assert _prefill(c, w, ring, 0x1000, 8, 0x1000, ok_ws - 1) == ds4g.ERR_WORKSPACE
    assert _prefill(c, w, ring, 0x1000, 9, 0x1000, ok_ws) == ds4g.ERR_WORKSPACE
    assert _prefill(_cfg(head_dim=96), w, ring, 0x1000, 8, 0x1000, ok_ws) == ds4g.ERR_UNSUPPORTED
    assert _prefill(_cfg(window=129), w, ring, 0x1000, 8, 0x1000, ok_ws) == ds4g.ERR_UNSUPPORTED
    assert _prefill(_cfg(top_k=9), w, ring, 0x1000, 8, 0x1000, ok_ws) == ds4g.ERR_UNSUPPORTED
    assert _prefill(_cfg(top_k=256), w, ring, 0x1000, 8, 0x1000, ok_ws) == ds4g.ERR_INVALID_ARG
    assert _prefill(_cfg(hidden=100), w, ring, 0x1000, 8, 0x1000, ok_ws) == ds4g.ERR_UNSUPPORTED
    assert _prefill(_cfg(wdtype=7), w, ring, 0x1000, 8, 0x1000, ok_ws) == ds4g.ERR_INVALID_ARG
    assert _prefill(_cfg(rope_dim=3), w, ring, 0x1000, 8, 0x1000, ok_ws) == ds4g.ERR_INVALID_ARG
    assert _prefill(_cfg(n_experts=600), w, ring, 0x1000, 8, 0x1000, ok_ws) == ds4g.ERR_UNSUPPORTED
    assert _prefill(_cfg(n_heads=6), w, ring, 0x1000, 8, 0x1000, ok_ws) == ds4g.ERR_UNSUPPORTED


def test_decode_and_sample_reject_before_launch():
    c = _cfg()
    w = _weights()
    ring = ds4g.KvRing(0x1000, 0x1000, 0x1000)
    n = ds4g.workspace_bytes(c, 1)
    L = ds4g.lib
    assert L.ds4g_layer_decode(ctypes.byref(c), ctypes.byref(w), ctypes.byref(ring), None, None,
                               0x1000, n, None) == ds4g.ERR_INVALID_ARG
    assert L.ds4g_layer_decode(ctypes.byref(c), ctypes.byref(w), ctypes.byref(ring), 0x1000,
                               None, 0x1000, n - 1, None) == ds4g.ERR_WORKSPACE
    ns = ds4g.workspace_bytes(None, 0, 129280)
    args = dict(hidden=4096, vocab=129280, wd=ds4g.BF16, norm=0x1000, eps=1e-6, w=0x1000, x=0x1000,
                T=0.7, p=0.95, rng=0x1000, logits=0x1000, tok=0x1000, ws=0x1000, n=ns)

    def call(**kw):
        a = dict(args, **kw)
        return L.ds4g_lmhead_sample(a["hidden"], a["vocab"], a["wd"], a["norm"], a["eps"], a["w"],
                                    a["x"], a["T"], a["p"], a["rng"], a["logits"], a["tok"],
                                    a.get("etab"), a.get("xnext"), a["ws"], a["n"], None)
    assert call(rng=None) == ds4g.ERR_INVALID_ARG          # sampling needs the generator
    assert call(vocab=0) == ds4g.ERR_INVALID_ARG
    assert call(wd=5) == ds4g.ERR_INVALID_ARG
    assert call(n=ns - 1) == ds4g.ERR_WORKSPACE
    assert call(hidden=100) == ds4g.ERR_UNSUPPORTED
    assert call(vocab=300000) == ds4g.ERR_UNSUPPORTED
    assert call(T=float("nan")) == ds4g.ERR_INVALID_ARG
    assert call(ws=0x1001) == ds4g.ERR_INVALID_ARG
    assert call(etab=0x1000) == ds4g.ERR_INVALID_ARG        # table without x_next
    assert call(xnext=0x1000) == ds4g.ERR_INVALID_ARG
    E = L.ds4g_embed
    assert E(0, 64, ds4g.BF16, 0x1000, 0x1000, 4, 0x1000, None) == ds4g.ERR_INVALID_ARG
    assert E(10, 64, ds4g.BF16, None, 0x1000, 4, 0x1000, None) == ds4g.ERR_INVALID_ARG
    assert E(10, 64, ds4g.BF16, 0x1000, 0x1000, 0, 0x1000, None) == ds4g.ERR_INVALID_ARG
    assert E(10, 60, ds4g.BF16, 0x1000, 0x1000, 4, 0x1000, None) == ds4g.ERR_UNSUPPORTED
    assert E(10, 64, 3, 0x1000, 0x1000, 4, 0x1000, None) == ds4g.ERR_INVALID_ARG


def test_sample_ex_rejects_before_launch():
    L = ds4g.lib
    ns = ds4g.workspace_bytes(None, 0, 129280)

    def call(params, rng=0x1000):
        return L.ds4g_lmhead_sample_ex(4096, 129280, ds4g.BF16, 0x1000, 1e-6, 0x1000, 0x1000,
                                       ctypes.byref(params) if params is not None else None,
                                       rng, 0x1000, 0x1000, None, None, 0x1000, ns, None)
    P = ds4g.SampleParams
    assert call(None) == ds4g.ERR_INVALID_ARG                            # no params
    assert call(P(0.7, 0.95, float("nan"), None)) == ds4g.ERR_INVALID_ARG
    assert call(P(0.7, 0.95, 0.05, None), rng=None) == ds4g.ERR_INVALID_ARG
    # a device temperature may ask for sampling at run time: the generator is required
    assert call(P(0.0, 0.95, 0.0, 0x1000), rng=None) == ds4g.ERR_INVALID_ARG
    assert call(P(0.7, float("nan"), 0.0, None)) == ds4g.ERR_INVALID_ARG
