"""Python binding of libds4g (include/ds4g.h): argument marshalling only.

Every step of the layer, the lm_head and the sampler runs in the HIP kernels
of libds4g.so.  torch is used for device memory and streams; this module only
turns tensors into pointers and sizes and calls the C ABI.  There is no
fallback: if the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("DS4G_LIB") or os.path.join(HERE, "libds4g.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
MODE_PREFILL, MODE_DECODE, MODE_DECODE_BATCH = 0, 1, 2

# ds4g.h declares these functions; the ABI test checks the header agrees.
EXPORTS = ("ds4g_workspace_bytes", "ds4g_f16_images_bytes", "ds4g_make_f16_images",
           "ds4g_layer_supported", "ds4g_layer_prefill",
           "ds4g_layer_prefill_trace",
           "ds4g_layer_decode", "ds4g_layer_decode_noalloc", "ds4g_layer_decode_batch",
           "ds4g_lmhead_sample", "ds4g_lmhead_sample_ex", "ds4g_embed", "ds4g_probe_mfma", "ds4g_probe_mfma_random", "ds4g_probe_read", "ds4g_probe_chain",
           "ds4g_status_string")


class LayerCfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("qkv_rank", ctypes.c_int32),
                ("window", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("ffn_inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("wdtype", ctypes.c_int32)]


WEIGHT_NAMES = ("attn_norm", "qkv_a", "qkv_b", "wo", "ffn_norm", "router", "gate", "up",
                "down", "sh_gate", "sh_up", "sh_down")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_NAMES] + [("f16_images", ctypes.c_void_p)]


class SampleParams(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_p", ctypes.c_float),
                ("min_p", ctypes.c_float), ("temperature_dev", ctypes.c_void_p)]


class KvRing(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pos", ctypes.c_void_p)]


ROUTING_NAMES = ("topk_idx", "topk_w", "expert_count", "expert_offset", "perm", "router_in",
                 "router_logits")


class Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ROUTING_NAMES]


TRACE_NAMES = ("x_norm", "c", "q", "k", "v", "o", "h2")


class Trace(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in TRACE_NAMES]


class Ds4gError(RuntimeError):
    pass


def _hip_runtimes():
    """Distinct HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run moe_dsv4_layer_amd/build.py "
                          "(or __graft_entry__.build()) first")
    # torch brings its own HIP runtime.  Load it first so that the library's
    # libamdhip64.so.7 dependency binds to that same runtime (same soname);
    # loading the library first would map a second HIP/HSA runtime into the
    # process, and two runtimes cannot share the device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    rts = _hip_runtimes()
    if len(rts) > 1:
        raise ImportError(f"two HIP runtimes are loaded ({rts}); import torch before "
                          "anything that loads /opt/rocm's libamdhip64")
    P = ctypes.c_void_p
    lib.ds4g_workspace_bytes.restype = ctypes.c_size_t
    lib.ds4g_workspace_bytes.argtypes = [ctypes.POINTER(LayerCfg), ctypes.c_int32, ctypes.c_int32]
    lib.ds4g_f16_images_bytes.restype = ctypes.c_size_t
    lib.ds4g_f16_images_bytes.argtypes = [ctypes.POINTER(LayerCfg)]
    lib.ds4g_make_f16_images.restype = ctypes.c_int
    lib.ds4g_make_f16_images.argtypes = [ctypes.POINTER(LayerCfg), ctypes.POINTER(LayerWeights), P,
                                         ctypes.c_size_t, P]
    lib.ds4g_layer_supported.restype = ctypes.c_int
    lib.ds4g_layer_supported.argtypes = [ctypes.POINTER(LayerCfg), ctypes.c_int32, ctypes.c_int32]
    lib.ds4g_layer_prefill.restype = ctypes.c_int
    lib.ds4g_layer_prefill.argtypes = [ctypes.POINTER(LayerCfg), ctypes.POINTER(LayerWeights),
                                       ctypes.POINTER(KvRing), P, ctypes.c_int32,
                                       ctypes.POINTER(Routing), P, ctypes.c_size_t, P]
    lib.ds4g_layer_prefill_trace.restype = ctypes.c_int
    lib.ds4g_layer_prefill_trace.argtypes = [ctypes.POINTER(LayerCfg),
                                             ctypes.POINTER(LayerWeights),
                                             ctypes.POINTER(KvRing), P, ctypes.c_int32,
                                             ctypes.POINTER(Routing), ctypes.POINTER(Trace), P,
                                             ctypes.c_size_t, P]
    lib.ds4g_layer_decode.restype = ctypes.c_int
    lib.ds4g_layer_decode.argtypes = [ctypes.POINTER(LayerCfg), ctypes.POINTER(LayerWeights),
                                      ctypes.POINTER(KvRing), P, ctypes.POINTER(Routing), P,
                                      ctypes.c_size_t, P]
    lib.ds4g_layer_decode_noalloc.restype = ctypes.c_int
    lib.ds4g_layer_decode_noalloc.argtypes = [ctypes.POINTER(LayerCfg),
                                              ctypes.POINTER(LayerWeights),
                                              ctypes.POINTER(KvRing), P, ctypes.POINTER(Routing),
                                              P]
    lib.ds4g_layer_decode_batch.restype = ctypes.c_int
    lib.ds4g_layer_decode_batch.argtypes = [ctypes.POINTER(LayerCfg), ctypes.POINTER(LayerWeights),
                                            ctypes.POINTER(KvRing), P, ctypes.c_int32,
                                            ctypes.POINTER(Routing), P, ctypes.c_size_t, P]
    lib.ds4g_lmhead_sample.restype = ctypes.c_int
    lib.ds4g_lmhead_sample.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P,
                                       ctypes.c_float, P, P, ctypes.c_float, ctypes.c_float, P,
                                       P, P, P, P, P, ctypes.c_size_t, P]
    lib.ds4g_lmhead_sample_ex.restype = ctypes.c_int
    lib.ds4g_lmhead_sample_ex.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P,
                                          ctypes.c_float, P, P, ctypes.POINTER(SampleParams), P,
                                          P, P, P, P, P, ctypes.c_size_t, P]
    lib.ds4g_embed.restype = ctypes.c_int
    lib.ds4g_embed.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P,
                               ctypes.c_int32, P, P]
    lib.ds4g_probe_mfma.restype = ctypes.c_int
    lib.ds4g_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P]
    lib.ds4g_probe_mfma_random.restype = ctypes.c_int
    lib.ds4g_probe_mfma_random.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32, P, P]
    lib.ds4g_probe_read.restype = ctypes.c_int
    lib.ds4g_probe_read.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int32, P, P]
    lib.ds4g_probe_chain.restype = ctypes.c_int
    lib.ds4g_probe_chain.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P]
    lib.ds4g_status_string.restype = ctypes.c_char_p
    lib.ds4g_status_string.argtypes = [ctypes.c_int]
    return lib


lib = _load()


def status_string(rc: int) -> str:
    return lib.ds4g_status_string(rc).decode()


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise Ds4gError(f"{what}: {status_string(rc)} ({rc})")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_cfg(shape) -> LayerCfg:
    """ds4g_layer_cfg from any object with the layer's size attributes."""
    wd = getattr(shape, "wdtype", "bf16")
    return LayerCfg(shape.hidden, shape.n_heads, shape.head_dim, shape.qkv_rank, shape.window,
                    shape.n_experts, shape.top_k, shape.ffn_inter,
                    getattr(shape, "shared_inter", 0) or shape.ffn_inter * getattr(shape, "n_shared", 1),
                    getattr(shape, "rope_dim", 0) or 0, float(shape.rope_base),
                    float(shape.rms_eps), BF16 if wd in ("bf16", BF16) else F32)


def make_weights(w: Dict[str, "torch.Tensor"], f16_images=None) -> LayerWeights:
    """ds4g_layer_weights of a dict of contiguous weight tensors; f16_images:
    an optional buffer filled by make_f16_images (kept alive by the caller)."""
    for n in WEIGHT_NAMES:
        t = w[n]
        if not t.is_contiguous():
            raise ValueError(f"weight {n} must be contiguous")
    return LayerWeights(*[w[n].data_ptr() for n in WEIGHT_NAMES], _ptr(f16_images))


def f16_images_bytes(cfg: LayerCfg) -> int:
    return int(lib.ds4g_f16_images_bytes(ctypes.byref(cfg)))


def make_f16_images(cfg: LayerCfg, w: LayerWeights, device="cuda", stream=None):
    """A device buffer holding the layer's fp16 attention-path images
    (ds4g_make_f16_images); set it as f16_images of the layer's weights."""
    import torch
    n = f16_images_bytes(cfg)
    if n == 0:
        raise Ds4gError("this layer has no fp16 images (fp32 weights)")
    buf = torch.empty(n, dtype=torch.uint8, device=device)
    _check(lib.ds4g_make_f16_images(ctypes.byref(cfg), ctypes.byref(w), buf.data_ptr(), n,
                                    _stream(stream)), "ds4g_make_f16_images")
    return buf


def make_ring(k, v, pos) -> KvRing:
    return KvRing(k.data_ptr(), v.data_ptr(), pos.data_ptr())


def make_routing(bufs: Optional[Dict[str, "torch.Tensor"]]) -> Optional[Routing]:
    if not bufs:
        return None
    return Routing(*[_ptr(bufs.get(n)) for n in ROUTING_NAMES])


def workspace_bytes(cfg: Optional[LayerCfg], max_tokens: int, vocab: int = 0) -> int:
    return int(lib.ds4g_workspace_bytes(ctypes.byref(cfg) if cfg is not None else None,
                                        max_tokens, vocab))


def layer_supported(cfg: Optional[LayerCfg], T: int, mode: int) -> int:
    """Status a layer call of `mode` over T tokens / sequences would return
    for its shape (0 = accepted); needs no device."""
    return int(lib.ds4g_layer_supported(ctypes.byref(cfg) if cfg is not None else None, T, mode))


def layer_prefill(cfg: LayerCfg, w: LayerWeights, ring: KvRing, x, T: int, ws,
                  routing: Optional[Routing] = None, stream=None) -> None:
    rc = lib.ds4g_layer_prefill(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ring),
                                x.data_ptr(), T,
                                ctypes.byref(routing) if routing is not None else None,
                                ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "ds4g_layer_prefill")


def layer_prefill_trace(cfg: LayerCfg, w: LayerWeights, ring: KvRing, x, T: int, ws,
                        trace: Dict[str, "torch.Tensor"], routing: Optional[Routing] = None,
                        stream=None) -> None:
    """ds4g_layer_prefill_trace: the prefill, plus copies of its intermediate
    activations into the tensors named in `trace` (keys of TRACE_NAMES)."""
    tr = Trace(*[_ptr(trace.get(n)) for n in TRACE_NAMES])
    rc = lib.ds4g_layer_prefill_trace(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ring),
                                      x.data_ptr(), T,
                                      ctypes.byref(routing) if routing is not None else None,
                                      ctypes.byref(tr), ws.data_ptr(),
                                      ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "ds4g_layer_prefill_trace")


def layer_decode(cfg: LayerCfg, w: LayerWeights, ring: KvRing, x, ws,
                 routing: Optional[Routing] = None, stream=None) -> None:
    rc = lib.ds4g_layer_decode(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ring),
                               x.data_ptr(),
                               ctypes.byref(routing) if routing is not None else None,
                               ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "ds4g_layer_decode")


def layer_decode_noalloc(cfg: LayerCfg, w: LayerWeights, ring: KvRing, x,
                         routing: Optional[Routing] = None, stream=None) -> None:
    """ds4g_layer_decode with the library's static scratch (no workspace)."""
    rc = lib.ds4g_layer_decode_noalloc(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ring),
                                       x.data_ptr(),
                                       ctypes.byref(routing) if routing is not None else None,
                                       _stream(stream))
    _check(rc, "ds4g_layer_decode_noalloc")


def layer_decode_batch(cfg: LayerCfg, w: LayerWeights, rings: KvRing, x, B: int, ws,
                       routing: Optional[Routing] = None, stream=None) -> None:
    """One decode token of each of B sequences; rings: k, v [B, W, dh], pos [B]."""
    rc = lib.ds4g_layer_decode_batch(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(rings),
                                     x.data_ptr(), B,
                                     ctypes.byref(routing) if routing is not None else None,
                                     ws.data_ptr(), ws.numel() * ws.element_size(),
                                     _stream(stream))
    _check(rc, "ds4g_layer_decode_batch")


def lmhead_sample(hidden: int, vocab: int, wdtype: int, final_norm, rms_eps: float, w_lm, x,
                  temperature: float, top_p: float, rng_state, logits, token, ws,
                  stream=None, embed_table=None, x_next=None) -> None:
    rc = lib.ds4g_lmhead_sample(hidden, vocab, wdtype, _ptr(final_norm), rms_eps,
                                w_lm.data_ptr(), x.data_ptr(), temperature, top_p,
                                _ptr(rng_state), logits.data_ptr(), token.data_ptr(),
                                _ptr(embed_table), _ptr(x_next),
                                ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "ds4g_lmhead_sample")


def lmhead_sample_ex(hidden: int, vocab: int, wdtype: int, final_norm, rms_eps: float, w_lm, x,
                     temperature: float, top_p: float, min_p: float, rng_state, logits, token,
                     ws, stream=None, temperature_dev=None, embed_table=None,
                     x_next=None) -> None:
    """ds4g_lmhead_sample_ex: min-p, and an optional device temperature
    (float32 tensor of one element) read by the call in place of temperature."""
    p = SampleParams(temperature, top_p, min_p, _ptr(temperature_dev))
    rc = lib.ds4g_lmhead_sample_ex(hidden, vocab, wdtype, _ptr(final_norm), rms_eps,
                                   w_lm.data_ptr(), x.data_ptr(), ctypes.byref(p),
                                   _ptr(rng_state), logits.data_ptr(), token.data_ptr(),
                                   _ptr(embed_table), _ptr(x_next),
                                   ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "ds4g_lmhead_sample_ex")


def embed(vocab: int, hidden: int, wdtype: int, table, ids, x, stream=None) -> None:
    """x[t] = table[ids[t]] widened to fp32 (ids: device int32 [T])."""
    rc = lib.ds4g_embed(vocab, hidden, wdtype, table.data_ptr(), ids.data_ptr(), ids.numel(),
                        x.data_ptr(), _stream(stream))
    _check(rc, "ds4g_embed")


def probe_mfma(blocks: int, iters: int, out, stream=None) -> None:
    """ds4g_probe_mfma: blocks x 4 waves of iters x 8 bf16 32x32x16 MFMAs."""
    _check(lib.ds4g_probe_mfma(blocks, iters, out.data_ptr(), _stream(stream)),
           "ds4g_probe_mfma")


def probe_mfma_random(blocks: int, iters: int, seed: int, out, stream=None) -> None:
    """ds4g_probe_mfma_random: blocks x 4 waves of iters x 64 bf16 32x32x16
    MFMAs on random operands."""
    _check(lib.ds4g_probe_mfma_random(blocks, iters, seed, out.data_ptr(), _stream(stream)),
           "ds4g_probe_mfma_random")


def probe_read(src, step_rows: int, row_stride: int, read_bytes: int, blocks: int, out,
               stream=None) -> None:
    """ds4g_probe_read: read read_bytes of src (a device tensor) as units of
    step_rows rows of row_stride bytes, in 32 KB steps; out: uint32-sized
    device tensor of blocks * 256 elements."""
    _check(lib.ds4g_probe_read(src.data_ptr(), src.numel() * src.element_size(), step_rows,
                               row_stride, read_bytes, blocks, out.data_ptr(), _stream(stream)),
           "ds4g_probe_read")


def probe_chain(blocks: int, n_kernels: int, chained: bool, buf, stream=None) -> None:
    """ds4g_probe_chain: n_kernels launches, each reading the previous one's
    word when chained (buf: device tensor of at least 2 int32)."""
    _check(lib.ds4g_probe_chain(blocks, n_kernels, int(chained), buf.data_ptr(),
                                _stream(stream)), "ds4g_probe_chain")


def alloc_workspace(nbytes: int, device="cuda"):
    """A 256-byte aligned device byte buffer (torch allocations are)."""
    import torch
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
