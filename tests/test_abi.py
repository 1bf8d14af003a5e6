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
    # ds4g_workspace_bytes is the largest need of any layer call (a prefill
    # of that many tokens, with its fp16 weight images); the decode step
    # needs far less, and refuses a workspace below its own need
    assert L.ds4g_layer_decode(ctypes.byref(c), ctypes.byref(w), ctypes.byref(ring), 0x1000,
                               None, 0x1000, 4096, None) == ds4g.ERR_WORKSPACE
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


def _decode(cfg, nbytes):
    w = _weights()
    ring = ds4g.KvRing(0x1000, 0x1000, 0x1000)
    return ds4g.lib.ds4g_layer_decode(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ring),
                                      0x1000, None, 0x1000, nbytes, None)


def _batch(cfg, B, nbytes):
    w = _weights()
    ring = ds4g.KvRing(0x1000, 0x1000, 0x1000)
    return ds4g.lib.ds4g_layer_decode_batch(ctypes.byref(cfg), ctypes.byref(w),
                                            ctypes.byref(ring), 0x1000, B, None, 0x1000, nbytes,
                                            None)


def test_decode_rejects_hidden_past_its_kernels():
    # the decode MoE kernels hold a wave's K slice of y in registers: hidden
    # <= 8192.  A wider layer passes the dimension checks (prefill takes it)
    # and must be refused before the first launch, not after QKV and W_o ran.
    c = _cfg(hidden=16384)
    assert ds4g.layer_supported(c, 1, ds4g.MODE_DECODE) == ds4g.ERR_UNSUPPORTED
    assert ds4g.layer_supported(c, 64, ds4g.MODE_PREFILL) == ds4g.OK
    assert _decode(c, 1 << 62) == ds4g.ERR_UNSUPPORTED
    assert ds4g.layer_supported(_cfg(hidden=8192), 1, ds4g.MODE_DECODE) == ds4g.OK


def test_batch_rejects_past_32bit_operand_offsets():
    # the MFMA GEMMs address 16-bit operands with 32-bit byte offsets; the
    # router operand of B rows is B x 3*hidden bf16 (4.9 GB at B = 50000)
    c = _cfg(hidden=16384)
    assert ds4g.layer_supported(c, 50000, ds4g.MODE_DECODE_BATCH) == ds4g.ERR_UNSUPPORTED
    assert _batch(c, 50000, 1 << 62) == ds4g.ERR_UNSUPPORTED
    assert ds4g.layer_supported(c, 40000, ds4g.MODE_DECODE_BATCH) == ds4g.OK
    assert ds4g.layer_supported(_cfg(), 65536, ds4g.MODE_DECODE_BATCH) == ds4g.ERR_UNSUPPORTED


def _documented(c, T, mode):
    """The support matrix the header states (ds4g_layer_cfg's comment)."""
    rd = c.rope_dim or c.head_dim
    qd = c.n_heads * c.head_dim
    ok = (c.head_dim in (64, 128) and rd % 2 == 0 and rd <= c.head_dim and 1 <= c.window <= 128
          and c.top_k + 1 <= c.n_experts <= 512 and 1 <= c.top_k <= 8 and c.n_heads % 4 == 0
          and all(v % 64 == 0 for v in (c.hidden, c.qkv_rank, c.ffn_inter, c.shared_inter, qd))
          and max(c.hidden, c.qkv_rank, qd) <= 16384 and max(c.ffn_inter, c.shared_inter) <= 2048
          and c.top_k * c.ffn_inter + c.shared_inter <= 12288)
    if mode == ds4g.MODE_DECODE:
        ok = ok and c.hidden <= 8192
    if mode == ds4g.MODE_DECODE_BATCH:
        ok = ok and T <= 65535
    if c.wdtype == ds4g.BF16:
        widest = max(3 * c.hidden, qd, c.qkv_rank, c.shared_inter, c.top_k * c.ffn_inter)
        ok = ok and T * widest * 2 < 2 ** 32
    return ok and T * c.top_k < 2 ** 24 and T <= 2 ** 20


def test_support_matrix_sweep():
    """Every configuration inside the documented limits is accepted by the
    launch sequence of each call (no kernel launcher refuses it), every one
    outside is refused, and a refused shape is refused by the call itself
    before anything is launched (these calls run without a GPU: a call that
    got as far as a launch would report a HIP error instead)."""
    import itertools
    n = 0
    for hidden, dh, window, E, k, inter, wd, rope, heads in itertools.product(
            (256, 4096, 8192, 16384), (64, 96, 128), (1, 128, 129), (8, 256, 512, 600),
            (1, 6, 8, 9), (64, 512, 2048, 4096), (ds4g.F32, ds4g.BF16), (0, 32, 33), (4, 64, 6)):
        c = _cfg(hidden=hidden, head_dim=dh, window=window, n_experts=E, top_k=k,
                 ffn_inter=inter, shared_inter=inter, wdtype=wd, rope_dim=rope, n_heads=heads)
        for T, mode in ((1, ds4g.MODE_DECODE), (1, ds4g.MODE_PREFILL), (300, ds4g.MODE_PREFILL),
                        (16994, ds4g.MODE_PREFILL), (20480, ds4g.MODE_PREFILL),
                        (8, ds4g.MODE_DECODE_BATCH),
                        (128, ds4g.MODE_DECODE_BATCH)):
            st = ds4g.layer_supported(c, T, mode)
            want = _documented(c, T, mode)
            assert (st == ds4g.OK) == want, (hidden, dh, window, E, k, inter, wd, rope, heads, T,
                                             mode, st)
            if st != ds4g.OK and n % 7 == 0:    # a sample of refusals through the calls
                if mode == ds4g.MODE_DECODE:
                    assert _decode(c, 1 << 62) == st
                elif mode == ds4g.MODE_PREFILL:
                    ring = ds4g.KvRing(0x1000, 0x1000, 0x1000)
                    assert _prefill(c, _weights(), ring, 0x1000, T, 0x1000, 1 << 62) == st
                else:
                    assert _batch(c, T, 1 << 62) == st
            n += 1
    assert n > 10000


def test_binding_refuses_two_hip_runtimes():
    """The binding imports torch (and its HIP runtime) before the library, and
    refuses to load when a second runtime has been mapped: a fresh process
    that maps /opt/rocm's runtime first must get an ImportError naming both."""
    import subprocess
    import sys
    rocm = "/opt/rocm/lib/libamdhip64.so"
    if not os.path.exists(rocm):
        pytest.skip("no /opt/rocm runtime in this image")
    code = ("import ctypes, sys; ctypes.CDLL(%r, mode=ctypes.RTLD_GLOBAL)\n"
            "sys.path.insert(0, %r)\n"
            "try:\n    import moe_dsv4_layer_amd\nexcept ImportError as e:\n"
            "    print('REFUSED', e); sys.exit(0)\n"
            "print('LOADED', moe_dsv4_layer_amd._hip_runtimes())\n") % (rocm, ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    # either the two runtimes are distinct files (refused) or they are the
    # same file (one runtime: loading is fine)
    if r.stdout.startswith("LOADED"):
        assert len(eval(r.stdout.split(" ", 1)[1])) == 1, r.stdout
    else:
        assert "two HIP runtimes" in r.stdout, r.stdout


def test_decode_noalloc_rejects_before_touching_the_device():
    # every check and the dry launch sequence run before the scratch address
    # is looked up: these refusals need no device
    L = ds4g.lib
    w = _weights()
    ring = ds4g.KvRing(0x1000, 0x1000, 0x1000)

    def call(cfg, x=0x1000, wts=w, rg=ring):
        return L.ds4g_layer_decode_noalloc(ctypes.byref(cfg) if cfg is not None else None,
                                           ctypes.byref(wts) if wts is not None else None,
                                           ctypes.byref(rg) if rg is not None else None,
                                           x, None, None)
    assert call(None) == ds4g.ERR_INVALID_ARG
    assert call(_cfg(), x=None) == ds4g.ERR_INVALID_ARG
    assert call(_cfg(), wts=_weights(False)) == ds4g.ERR_INVALID_ARG
    assert call(_cfg(), rg=ds4g.KvRing(0x1000, 0, 0x1000)) == ds4g.ERR_INVALID_ARG
    assert call(_cfg(head_dim=96)) == ds4g.ERR_UNSUPPORTED
    assert call(_cfg(hidden=16384)) == ds4g.ERR_UNSUPPORTED     # refused by the dry run


def test_probes_reject_before_launch():
    L = ds4g.lib
    GiB = 1 << 30
    src, out = 0x10000, 0x20000

    def read(step_rows=128, stride=8192, nbytes=GiB, src_bytes=GiB, blocks=512, s=src, o=out):
        return L.ds4g_probe_read(s, src_bytes, step_rows, stride, nbytes, blocks, o, None)
    assert read(s=None) == ds4g.ERR_INVALID_ARG
    assert read(o=None) == ds4g.ERR_INVALID_ARG
    assert read(blocks=0) == ds4g.ERR_INVALID_ARG
    for bad_rows in (0, 2, 3, 96, 4096):
        assert read(step_rows=bad_rows) == ds4g.ERR_INVALID_ARG, bad_rows
    assert read(stride=8000) == ds4g.ERR_INVALID_ARG            # narrower than a row
    assert read(stride=8200) == ds4g.ERR_INVALID_ARG            # not a multiple of 16
    assert read(nbytes=128 * 8192 + 16) == ds4g.ERR_INVALID_ARG  # not whole units
    assert read(s=src + 8) == ds4g.ERR_INVALID_ARG               # misaligned
    # the padded walk needs (rows - 1) * stride + 8192 bytes of source
    rows = GiB // 8192
    need = (rows - 1) * 8320 + 8192
    assert read(stride=8320, src_bytes=need - 1) == ds4g.ERR_INVALID_ARG
    assert L.ds4g_probe_chain(0, 4, 1, out, None) == ds4g.ERR_INVALID_ARG
    assert L.ds4g_probe_chain(64, 0, 1, out, None) == ds4g.ERR_INVALID_ARG
    assert L.ds4g_probe_chain(64, 4, 1, None, None) == ds4g.ERR_INVALID_ARG
    assert L.ds4g_probe_mfma_random(0, 4, 1, out, None) == ds4g.ERR_INVALID_ARG
    assert L.ds4g_probe_mfma_random(64, 0, 1, out, None) == ds4g.ERR_INVALID_ARG
    assert L.ds4g_probe_mfma_random(64, 4, 1, None, None) == ds4g.ERR_INVALID_ARG
