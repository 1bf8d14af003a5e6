"""Throughput of the ds4g hot path on one MI355X.

Workload (synthetic, seeded, random-init weights of the full-size layer:
hidden 4096, 64-head MQA head_dim 128, QKV rank 1024, window 128, 256
experts top-6 + 1 shared, SwiGLU inter 1024, bf16 weights, fp32 accumulate):

  decode   one token through the full-size layer at position >= 128 (full
           window).  This is the headline `value` (tokens/s).  Four distinct
           layers' weights rotate so successive steps do not find the
           previous step's weights in the 256 MB Infinity Cache.
  prefill  layer-major prefill of 2048 tokens through the same layer
           (reported as prefill_tok_s).
  lm_head  final norm + 129280 x 4096 lm_head + temperature 0.7 / top-p
           0.95 sampler (reported as lmhead_sample_us).
  stack43  43 full-size layers (expert inter 512) + embedding + lm_head:
           prefill of 512 tokens, then decode steps (43 layers + lm_head +
           sampler + next-token embedding, one graph replay per token) at
           temperature 0.7 / top-p 0.95; and a 16994-token layer-major
           prefill, plus the 148-token suffix resumed from a ring snapshot
           taken at 16846 (reported under "stack43").

Every input lives in HBM before the timed region starts.  Times come from
HIP events on the stream the library launches on.  The CPU baseline is the
float64 oracle on a bounded sample (a few decode tokens), on the host cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s

# HBM bytes of one decode step as read by the hardware counters (rocprofv3
# --pmc FETCH_SIZE, then WRITE_SIZE, summed over the step's 7 kernels, mean of
# 12 steps; FETCH_SIZE scaled x2.0 and WRITE_SIZE x1.0, the factors that make a
# 1 GiB device copy read 1 GiB and write 1 GiB).  Valid only for the decode
# sources it was measured on: any change to them reports traffic as null.
DECODE_TRAFFIC_BYTES = 274010879
DECODE_TRAFFIC_SOURCES = ("api.hip", "attn.hip", "decode.hip", "dev.h", "kernels.h")
DECODE_TRAFFIC_SHA1 = "1e70354a962e40d8443d93259f381d8069a2a69c"


def progress(msg: str) -> None:
    """One line on stderr per section, so a long run shows its steps."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def decode_traffic():
    import hashlib
    h = hashlib.sha1()
    for f in DECODE_TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "moe_dsv4_layer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return DECODE_TRAFFIC_BYTES if h.hexdigest() == DECODE_TRAFFIC_SHA1 else None
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def layer_decode_bytes(s) -> int:
    """Algorithmic HBM bytes of one decode token through one layer: every
    weight the token needs, read once (6 routed + 1 shared expert), the KV
    window, and the fp32 activation vector in and out."""
    d, r, H, dh, I = s.hidden, s.qkv_rank, s.n_heads, s.head_dim, s.ffn_inter
    w = 2 * (r * d + (H * dh + 2 * dh) * r + d * H * dh + s.n_experts * d
             + (s.top_k + 1) * 3 * I * d + 2 * d)
    kv = 2 * 2 * s.window * dh
    return w + kv + 2 * 4 * d


def layer_flops(s, T: int) -> float:
    """Algorithmic flops of T tokens through one layer (2 per multiply-add)."""
    d, r, H, dh, I, W = s.hidden, s.qkv_rank, s.n_heads, s.head_dim, s.ffn_inter, s.window
    dense = r * d + (H * dh + 2 * dh) * r + d * H * dh + s.n_experts * d
    experts = (s.top_k + 1) * 3 * I * d
    attn = 2 * H * dh * min(W, T)     # q.k and p.v per key (upper bound)
    return 2.0 * T * (dense + experts + attn)


def dense_gemm_flops(s, T: int) -> float:
    d, r, H, dh, I = s.hidden, s.qkv_rank, s.n_heads, s.head_dim, s.ffn_inter
    return 2.0 * T * (r * d + (H * dh + 2 * dh) * r + d * H * dh + 3 * I * d)


def prefill_weight_bytes(s) -> int:
    d, r, H, dh, I = s.hidden, s.qkv_rank, s.n_heads, s.head_dim, s.ffn_inter
    return 2 * (r * d + (H * dh + 2 * dh) * r + d * H * dh + s.n_experts * d
                + (s.n_experts + 1) * 3 * I * d + 2 * d)


def cpu_baseline(shape, w_dev, h_dev, n_tokens: int):
    """The float64 oracle decoding `n_tokens` tokens through one full-size
    layer (ring pre-filled with 128 positions), timed on the host."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    wh = synth.weights_to_host(w_dev)
    h = h_dev.cpu().numpy()
    ring = oracle.Ring(shape.window, shape.head_dim)
    # fill the window (not timed): keys/values of 128 positions
    oracle.layer_forward(shape, wh, ring, h[:shape.window], rows=[])
    t0 = time.perf_counter()
    for i in range(n_tokens):
        oracle.layer_forward(shape, wh, ring, h[shape.window + i:shape.window + i + 1])
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tok/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_tokens} decode tokens through one full-size layer (float64 numpy, "
                      f"window pre-filled with {shape.window} positions), {dt:.1f} s"}


def cpu_baseline_prefill(shape, w_dev, n_tokens: int, seed: int):
    """The float64 oracle prefilling `n_tokens` fresh N(0, 1) rows through one
    full-size layer from an empty ring (layer-major, every expert each token
    routes to), timed on the host."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    wh = synth.weights_to_host(w_dev)
    h = synth.hidden(n_tokens, shape.hidden, seed).numpy()
    ring = oracle.Ring(shape.window, shape.head_dim)
    t0 = time.perf_counter()
    oracle.layer_forward(shape, wh, ring, h)
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tok/s", "cores": int(threads), "kind": "oracle",
            "sample": f"layer-major prefill of {n_tokens} tokens through one full-size layer "
                      f"(float64 numpy, empty ring), {dt:.1f} s"}


def measured_peaks(dev) -> dict:
    """What the chip sustains right now: a 1 GiB device copy (read + write)
    and the bf16 MFMA loop of ds4g_probe_mfma (4 blocks per CU)."""
    import torch
    import moe_dsv4_layer_amd as ds4g
    out = {}
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    out["hbm_copy_gbs"] = round(5 * 2 * 4 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del src, dst
    blocks, iters = 1024, 400
    buf = torch.empty(blocks * 4, dtype=torch.float32, device=dev)
    ds4g.probe_mfma(blocks, iters, buf)
    torch.cuda.synchronize()
    e0.record(stream)
    ds4g.probe_mfma(blocks, iters, buf)
    e1.record(stream)
    torch.cuda.synchronize()
    fl = blocks * 4 * iters * 8 * 2.0 * 32 * 32 * 16
    out["mfma_bf16_tflops"] = round(fl / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    return out


def calibration_probes(dev) -> dict:
    """What the chip does with launches and access shapes, from the library's
    calibration kernels (ds4g_probe_chain, ds4g_probe_read) and, for
    comparison, the vendor GEMM behind torch.matmul.  Times are HIP events on
    the launch stream; graph figures replay a captured graph."""
    import numpy as np
    import torch
    import moe_dsv4_layer_amd as ds4g
    st = torch.cuda.current_stream()

    def timed_us(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def graph_of(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        return g

    res = {}
    # launch cost: 64 launches per call, eager and graph-replayed
    buf = torch.zeros(2, dtype=torch.int32, device=dev)
    n = 64
    launch = {}
    for chained in (False, True):
        for blocks in (256, 2048):
            def call(b=blocks, c=chained):
                ds4g.probe_chain(b, n, c, buf)
            call()
            eager = timed_us(call, 10) / n
            g = graph_of(call)
            graph = timed_us(g.replay, 20) / n
            launch[f"{'chained' if chained else 'independent'}_{blocks}_blocks"] = {
                "eager_us": round(eager, 2), "graph_us": round(graph, 2)}
    res["launch_cost_per_kernel"] = launch

    # HBM read rate by access shape over 1 GiB (512 blocks, 96 KB in flight each)
    GiB = 1 << 30
    rows = GiB // 8192
    src = torch.ones((rows - 1) * 8320 + 8192, dtype=torch.uint8, device=dev)
    out = torch.empty(2048 * 256, dtype=torch.int32, device=dev)
    shapes = {}
    for name, step_rows, stride in (("contiguous, 32 KB per step", 4, 8192),
                                    ("128 rows x 256 B per step", 128, 8192),
                                    ("256 rows x 128 B per step", 256, 8192),
                                    ("256 rows x 128 B per step, row stride 8 KB + 128 B", 256,
                                     8320)):
        def rd(sr=step_rows, sd=stride):
            ds4g.probe_read(src, sr, sd, GiB, 512, out)
        rd()
        us = timed_us(rd, 5)
        shapes[name] = round(GiB / (us * 1e-6) / 1e12, 2)
    res["read_tbs_by_shape_1GiB"] = shapes

    # one contiguous read per launch, graph-replayed, four regions 256 MB
    # apart rotated so the 256 MB Infinity Cache does not hold the next one
    sizes = [8_388_608, 17_301_504, 67_108_864, 117_440_512]
    region = 256 << 20
    per_launch = []
    for nbytes in sizes:
        def four(nb=nbytes):
            for r in range(4):
                ds4g.probe_read(src[r * region: r * region + nb], 4, 8192, nb, 1024, out)
        g = graph_of(lambda: [four() for _ in range(10)])
        per_launch.append(timed_us(g.replay, 5) / 40)
    slope, icpt = np.polyfit(np.array(sizes, dtype=np.float64), np.array(per_launch), 1)
    res["contiguous_read_per_launch"] = {
        "bytes": sizes, "us": [round(u, 2) for u in per_launch],
        "fit_fixed_us": round(float(icpt), 2),
        "fit_marginal_tbs": round(1e-6 / float(slope), 2)}

    # does a read leave its bytes in the Infinity Cache for the next launch?
    def read_at(off, nb):
        v = src[off: off + nb]
        return timed_us(lambda: ds4g.probe_read(v, 4, 8192, nb, 512, out), 1)

    def flush():
        ds4g.probe_read(src, 4, 8192, GiB, 512, out)

    MB = 1 << 20
    trials = []
    for _ in range(3):
        flush()
        cold = read_at(0, 64 * MB)
        again = read_at(0, 64 * MB)
        read_at(128 * MB, 64 * MB)
        after_other = read_at(0, 64 * MB)
        flush()
        cold32 = read_at(256 * MB, 32 * MB)
        again32 = read_at(256 * MB, 32 * MB)
        trials.append((cold, again, after_other, cold32, again32))
    med = np.median(np.array(trials), axis=0)
    res["reread_us"] = {"64MB_cold": round(float(med[0]), 2),
                        "64MB_again": round(float(med[1]), 2),
                        "64MB_after_another_64MB": round(float(med[2]), 2),
                        "32MB_cold": round(float(med[3]), 2),
                        "32MB_again": round(float(med[4]), 2)}
    del src

    # the matrix cores on register operands: near-constant and random data
    blocks, iters = 1024, 400
    buf = torch.empty(blocks * 4, dtype=torch.float32, device=dev)
    ds4g.probe_mfma(blocks, iters, buf)
    us_c = timed_us(lambda: ds4g.probe_mfma(blocks, iters, buf), 3)
    ds4g.probe_mfma_random(blocks, iters // 8, 12345, buf)
    us_r = timed_us(lambda: ds4g.probe_mfma_random(blocks, iters // 8, 12345, buf), 3)
    fl = blocks * 4 * iters * 8 * 2.0 * 32 * 32 * 16
    res["mfma_loop_bf16_pflops"] = {"near_constant_operands": round(fl / (us_c * 1e-6) / 1e15, 3),
                                    "random_operands": round(fl / (us_r * 1e-6) / 1e15, 3)}

    # the vendor GEMM on two shapes (bf16, fp32 accumulate), random operands
    vendor = {}
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    for name, (M, N, K) in (("8192^3", (8192, 8192, 8192)),
                            ("W_o of a 16994-token prefill", (16994, 4096, 8192))):
        a = torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16)
        b = torch.randn((K, N), generator=gen, device=dev).to(torch.bfloat16).contiguous()
        torch.matmul(a, b)
        us = timed_us(lambda: torch.matmul(a, b), 10)
        vendor[name] = {"us": round(us, 1), "pflops": round(2.0 * M * N * K / (us * 1e-6) / 1e15, 3)}
        del a, b
    res["vendor_matmul_bf16"] = vendor
    return res


def gpu_clocks() -> dict:
    """Current clocks from rocm-smi (best effort; text as rocm-smi prints it)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                           timeout=20)
        lines = [ln.strip() for ln in r.stdout.splitlines()
                 if "clock level" in ln or "sclk" in ln or "mclk" in ln or "fclk" in ln]
        return {"rocm_smi_showclocks": lines[:12]}
    except Exception as e:   # rocm-smi missing or refused
        return {"rocm_smi_showclocks": f"unavailable ({type(e).__name__})"}


def expert_loads(counts) -> dict:
    """Per-layer routing summary from each layer's expert_count: experts
    that received a token, and the largest load."""
    import numpy as np
    touched = [int((c > 0).sum()) for c in counts]
    mx = [int(c.max()) for c in counts]
    return {"touched_experts_by_layer": touched, "max_load_by_layer": mx,
            "touched_min": min(touched), "touched_mean": round(float(np.mean(touched)), 1)}


def touched_weight_bytes(s, touched) -> int:
    """Weight bytes a prefill must read when layer l's tokens reach only
    touched[l] routed experts: every dense weight plus those experts."""
    d, r, H, dh, I = s.hidden, s.qkv_rank, s.n_heads, s.head_dim, s.ffn_inter
    dense = 2 * (r * d + (H * dh + 2 * dh) * r + d * H * dh + s.n_experts * d + 3 * I * d + 2 * d)
    return int(sum(dense + 2 * 3 * I * d * t for t in touched))


def stack_decode_bytes(s, n_layers: int, vocab: int) -> int:
    """Per token: every layer's decode bytes, then the final norm and lm_head
    rows, and the next token's embedding row."""
    return n_layers * layer_decode_bytes(s) + 2 * vocab * s.hidden + 2 * s.hidden \
        + 4 * vocab + 2 * s.hidden


def bench_stack43(decode_steps: int) -> dict:
    import torch
    import numpy as np
    import synth
    from moe_dsv4_layer_amd.stack import Stack
    wl = synth.WORKLOADS["stack43_decode"]
    wr = synth.WORKLOADS["stack43_resume"]
    s = wl.layer
    layers = [synth.layer_weights(s, wl.seed, layer=l, device="cuda") for l in range(wl.n_layers)]
    head = synth.head_weights(s, wl.vocab, wl.seed, device="cuda")
    st = Stack(s, layers, head, max_tokens=wr.prompt)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {"workload": "43 full-size layers (expert inter 512) + embedding + lm_head 129280",
           "weight_bytes": int(sum(t.numel() * t.element_size() for w in layers for t in w.values())
                               + sum(t.numel() * t.element_size() for t in head.values()))}
    # ---- prefill of 512 tokens, then graph-replayed decode steps
    progress("43-layer stack: prefill 512, decode")
    ids = torch.as_tensor(synth.token_ids(wl.prompt, wl.vocab, wl.seed), device="cuda")
    for rep in range(2):
        st.reset()
        torch.cuda.synchronize()
        e0.record(stream)
        x = st.embed(ids)
        st.prefill(x)
        e1.record(stream)
        torch.cuda.synchronize()
    ms_pre = e0.elapsed_time(e1)
    out["prefill_512_ms"] = round(ms_pre, 3)
    out["prefill_512_tok_s"] = round(wl.prompt / (ms_pre * 1e-3), 1)

    def routed_counts(run):
        """Each layer's expert_count from an untimed repeat of a prefill."""
        bufs = [{"expert_count": torch.zeros(s.n_experts, dtype=torch.int32, device="cuda")}
                for _ in range(wl.n_layers)]
        run(bufs)
        torch.cuda.synchronize()
        return [b["expert_count"].cpu().numpy() for b in bufs]

    def run512(bufs):
        st.reset()
        st.prefill(st.embed(ids), routing=bufs)
    loads = expert_loads(routed_counts(run512))
    tb = touched_weight_bytes(s, loads["touched_experts_by_layer"])
    out["prefill_512_routing"] = loads
    out["prefill_512_touched_weight_bytes"] = tb
    out["prefill_512_hbm_frac_touched"] = round(tb / (ms_pre * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    st.reset()
    x = st.embed(ids)
    st.prefill(x)
    torch.cuda.synchronize()
    rng = torch.tensor([synth.rng_seed(wl.seed) & 0x7FFFFFFFFFFFFFFF], dtype=torch.int64,
                       device="cuda")
    xl = x[-1].clone()
    st.sample(xl, wl.temperature, wl.top_p, rng, x_next=xl)     # first token from the prompt
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)
    torch.cuda.synchronize()

    def step():
        st.decode(xl)
        st.sample(xl, wl.temperature, wl.top_p, rng, x_next=xl)
    with torch.cuda.stream(cs):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        step()
    torch.cuda.synchronize()
    n = max(1, decode_steps - 2)
    e0.record(stream)
    for _ in range(n):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_tok = e0.elapsed_time(e1) / n
    b = stack_decode_bytes(s, wl.n_layers, wl.vocab)
    out["decode_ms_per_token"] = round(ms_tok, 4)
    out["decode_tok_s"] = round(1e3 / ms_tok, 2)
    out["decode_bytes_per_token"] = b
    out["decode_hbm_frac"] = round(b / (ms_tok * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    out["positions_after"] = int(st.pos[0].item())
    # ---- 16994-token prefill, and the 148-token suffix from a snapshot at 16846
    progress("43-layer stack: prefill 16994, resume 148")
    ids = torch.as_tensor(synth.token_ids(wr.prompt, wl.vocab, wr.seed), device="cuda")
    P = wr.snapshot_at
    st.reset()
    x = st.embed(ids[:P])
    st.prefill(x)
    snap = st.snapshot()
    st.reset()
    torch.cuda.synchronize()
    e0.record(stream)
    x = st.embed(ids)
    st.prefill(x)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_full = e0.elapsed_time(e1)
    st.restore(snap)
    torch.cuda.synchronize()
    e0.record(stream)
    xs = st.embed(ids[P:])
    st.prefill(xs)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_suf = e0.elapsed_time(e1)
    fl = wr.n_layers * layer_flops(s, wr.prompt)
    out["prefill_16994_ms"] = round(ms_full, 2)
    out["prefill_16994_tok_s"] = round(wr.prompt / (ms_full * 1e-3), 1)
    out["prefill_16994_tflops"] = round(fl / (ms_full * 1e-3) / 1e12, 1)
    out["prefill_16994_mfma_frac"] = round(fl / (ms_full * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    out["resume_suffix_148_ms"] = round(ms_suf, 3)
    out["resume_suffix_matches_full"] = bool(torch.equal(xs, x[P:]))

    def run_full(bufs):
        st.reset()
        st.prefill(st.embed(ids), routing=bufs)

    def run_suffix(bufs):
        st.restore(snap)
        st.prefill(st.embed(ids[P:]), routing=bufs)
    loads = expert_loads(routed_counts(run_full))
    out["prefill_16994_routing"] = loads
    loads = expert_loads(routed_counts(run_suffix))
    tb = touched_weight_bytes(s, loads["touched_experts_by_layer"])
    out["resume_suffix_148_routing"] = loads
    out["resume_suffix_148_touched_weight_bytes"] = tb
    out["resume_suffix_148_hbm_frac_touched"] = round(tb / (ms_suf * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                                      4)
    del st, layers, head
    torch.cuda.empty_cache()
    return out


def ab_prefill(ds4g, synth, torch, other: str, reps: int, tokens) -> dict:
    """Two builds of the library in one process: the in-tree one (A) and
    `other` (B, e.g. built with different launch-shape macros through
    moe_dsv4_layer_amd/build.py's build(out=..., defines=[...])).  One
    full-size layer prefill per token count (expert inter 512 for counts
    above 2048, as in the 43-layer stack, else 1024), calls alternating
    A B B A ..., medians of `reps` calls each, outputs compared bit for bit.
    Separate processes on one box differ by 1-3% from run to run; this
    resolves differences down to about 0.3-1%."""
    import ctypes, dataclasses, shutil, tempfile
    la = ds4g.lib
    cp = os.path.join(tempfile.mkdtemp(), "libds4g_b.so")   # its own copy: its own handle
    shutil.copy(other, cp)
    lb = ctypes.CDLL(cp)
    for fn in ("ds4g_workspace_bytes", "ds4g_layer_prefill"):
        fa, fb = getattr(la, fn), getattr(lb, fn)
        fb.restype, fb.argtypes = fa.restype, fa.argtypes
    out = {}
    try:
        for T in tokens:
            inter = 512 if T > 2048 else 1024
            s = dataclasses.replace(synth.WORKLOADS["layer_decode"].layer, ffn_inter=inter)
            cfg = ds4g.make_cfg(s)
            w = synth.layer_weights(s, 1005, layer=0, device="cuda")
            cw = ds4g.make_weights(w)
            img = ds4g.make_f16_images(cfg, cw, "cuda")
            cwi = ds4g.make_weights(w, img)
            rk = torch.zeros((s.window, s.head_dim), dtype=torch.float16, device="cuda")
            rv = torch.zeros_like(rk)
            pos = torch.zeros(1, dtype=torch.int64, device="cuda")
            ring = ds4g.make_ring(rk, rv, pos)
            nb = max(la.ds4g_workspace_bytes(ctypes.byref(cfg), T, 0),
                     lb.ds4g_workspace_bytes(ctypes.byref(cfg), T, 0))
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
            h = synth.hidden(T, s.hidden, 1005, device="cuda")
            x = torch.empty_like(h)
            st = torch.cuda.current_stream()
            res, last = {"A": [], "B": []}, {}
            order = ["A", "B"]
            for r in range(reps):
                order += ["A", "B"] if r % 2 == 0 else ["B", "A"]
            for i, who in enumerate(order):
                ds4g.lib = la if who == "A" else lb
                pos.zero_()
                x.copy_(h)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                ds4g.layer_prefill(cfg, cwi, ring, x, T, ws)
                e1.record(st)
                torch.cuda.synchronize()
                if i >= 2:
                    res[who].append(e0.elapsed_time(e1))
                last[who] = x.clone()
            ds4g.lib = la
            ma = sorted(res["A"])[len(res["A"]) // 2]
            mb = sorted(res["B"])[len(res["B"]) // 2]
            out[str(T)] = {"A_ms": round(ma, 4), "B_ms": round(mb, 4), "B_over_A": round(mb / ma, 4),
                           "outputs_equal": bool(torch.equal(last["A"], last["B"]))}
            progress(f"ab T={T}: {out[str(T)]}")
            del w, cw, img, cwi, ws, h, x, last
            torch.cuda.empty_cache()
    finally:
        ds4g.lib = la
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--weight-sets", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=96)
    ap.add_argument("--cpu-prefill-tokens", type=int, default=256)
    ap.add_argument("--no-graph", action="store_true", help="launch decode eagerly")
    ap.add_argument("--no-stack", action="store_true", help="skip the 43-layer workloads")
    ap.add_argument("--stack-decode-steps", type=int, default=256)
    ap.add_argument("--sections", default="decode,prefill,batch,lmhead,stack,cpu,peaks",
                    help="comma list of what to run (profiling runs pick one); the JSON line "
                         "carries only what ran")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 1 GiB on the device 5 times (calibrates the HBM byte "
                         "counters FETCH_SIZE / WRITE_SIZE against a known size) and exit")
    ap.add_argument("--probes", action="store_true",
                    help="only run the calibration probes (launch cost, read rate by access "
                         "shape, Infinity Cache reuse, the vendor GEMM) and print their JSON line")
    ap.add_argument("--ab-lib", default="",
                    help="only compare the in-tree library with this other build of it on "
                         "one-layer prefills, alternating call by call in this process, and "
                         "print their JSON line")
    ap.add_argument("--ab-reps", type=int, default=10)
    ap.add_argument("--ab-tokens", default="16994,2048,512,148")
    args = ap.parse_args()
    want = set(args.sections.split(","))
    if args.no_stack:
        want.discard("stack")
    if args.no_cpu_baseline:
        want.discard("cpu")
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        return 2

    import torch
    import synth
    import moe_dsv4_layer_amd as ds4g

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        n = 1 << 28                                    # 2^28 fp32 = 1 GiB
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n,
                          "copies": 5}))
        return 0
    if args.ab_lib:
        toks = [int(t) for t in args.ab_tokens.split(",") if t]
        print(json.dumps({"ab_prefill": ab_prefill(ds4g, synth, torch, args.ab_lib, args.ab_reps,
                                                   toks)}))
        return 0
    if args.probes:
        print(json.dumps({"probes": calibration_probes(dev),
                          "device": torch.cuda.get_device_name(dev)}))
        return 0
    wl = synth.WORKLOADS["layer_decode"]
    s = wl.layer
    cfg = ds4g.make_cfg(s)
    stream = torch.cuda.current_stream()

    # ------------------------------------------------------------ setup
    progress("setup")
    layers = []
    w_cpu = None
    for l in range(args.weight_sets):
        w = synth.layer_weights(s, wl.seed, layer=l, device=dev)
        rk = torch.zeros((s.window, s.head_dim), dtype=torch.float16, device=dev)
        rv = torch.zeros_like(rk)
        pos = torch.zeros(1, dtype=torch.int64, device=dev)
        cw = ds4g.make_weights(w)
        img = ds4g.make_f16_images(cfg, cw, dev)      # prepared once, as at weight load
        layers.append(dict(w=w, cw=cw, img=img, cwi=ds4g.make_weights(w, img), rk=rk, rv=rv,
                           pos=pos, ring=ds4g.make_ring(rk, rv, pos)))
        if l == 0:
            w_cpu = w
    T_pre = synth.WORKLOADS["layer_prefill_2048"].prompt
    ws = ds4g.alloc_workspace(ds4g.workspace_bytes(cfg, T_pre, 129280))
    h_all = synth.hidden(s.window + 64, s.hidden, wl.seed, device=dev)
    # fill each ring with 128 positions (layer-major prefill), keep the
    # decode inputs resident: one fp32 vector per layer, chained in place
    xs = []
    for L in layers:
        x = h_all[:s.window].clone()
        ds4g.layer_prefill(cfg, L["cw"], L["ring"], x, s.window, ws, stream=stream)
        xs.append(h_all[s.window].clone())
    torch.cuda.synchronize()

    def decode_step(i):
        L = layers[i % len(layers)]
        ds4g.layer_decode(cfg, L["cw"], L["ring"], xs[i % len(layers)], ws, stream=stream)

    for i in range(args.warmup):
        decode_step(i)
    torch.cuda.synchronize()

    graph = None
    if not args.no_graph:
        # one graph replays len(layers) decode steps (one per weight set);
        # positions and ring slots live on the device, so replays advance
        try:
            cs = torch.cuda.Stream()
            cs.wait_stream(stream)
            with torch.cuda.stream(cs):
                for i in range(len(layers)):
                    L = layers[i]
                    ds4g.layer_decode(cfg, L["cw"], L["ring"], xs[i], ws, stream=cs)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                for i in range(len(layers)):
                    L = layers[i]
                    ds4g.layer_decode(cfg, L["cw"], L["ring"], xs[i], ws, stream=cs)
            torch.cuda.synchronize()
            graph = g
            for _ in range(3):
                graph.replay()
            torch.cuda.synchronize()
        except Exception as e:  # capture unsupported: report eager numbers
            print(f"graph capture failed ({e}); timing eager launches", file=sys.stderr)
            graph = None

    nl = len(layers)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms_decode = steps = t_wall = dec_gbs = None
    dec_bytes = layer_decode_bytes(s)
    # ------------------------------------------------------------ decode timing
    if "decode" in want:
        progress("decode")
        nl = len(layers)
        steps = args.steps
        if graph is not None:
            steps = max(nl, (steps // nl) * nl)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        e0.record(stream)
        if graph is not None:
            for _ in range(steps // nl):
                graph.replay()
        else:
            for i in range(steps):
                decode_step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
        ms_decode = e0.elapsed_time(e1) / steps
        dec_bytes = layer_decode_bytes(s)
        dec_gbs = dec_bytes / (ms_decode * 1e-3) / 1e9

    # ------------------------------------------------------------ prefill timing
    if "prefill" in want:
        progress("prefill")
        # every call: fresh N(0, 1) rows at positions 0..2047 from an empty ring
        # (the input copy and position reset sit outside the timed events)
        hp = synth.hidden(T_pre, s.hidden, synth.WORKLOADS["layer_prefill_2048"].seed, device=dev)
        xp = torch.empty_like(hp)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.prefill_steps)]

        def prefill_call(i, evs=None, routing=None, key="cwi"):
            L = layers[i % nl]
            L["pos"].zero_()
            xp.copy_(hp)
            if evs:
                evs[0].record(stream)
            ds4g.layer_prefill(cfg, L[key], L["ring"], xp, T_pre, ws, routing, stream=stream)
            if evs:
                evs[1].record(stream)
        for i in range(2):
            prefill_call(i)
        torch.cuda.synchronize()
        for i in range(args.prefill_steps):
            prefill_call(i, ev[i])
        torch.cuda.synchronize()
        ms_prefill = sum(a.elapsed_time(b) for a, b in ev) / args.prefill_steps
        # the same calls making the fp16 images in their workspace
        for i in range(args.prefill_steps):
            prefill_call(i, ev[i], key="cw")
        torch.cuda.synchronize()
        ms_prefill_img = sum(a.elapsed_time(b) for a, b in ev) / args.prefill_steps
        cnt = torch.zeros(s.n_experts, dtype=torch.int32, device=dev)
        prefill_call(0, routing=ds4g.make_routing({"expert_count": cnt}))
        torch.cuda.synchronize()
        pre_load = (int(cnt.min().item()), int(cnt.max().item()))
        pre_tflops = layer_flops(s, T_pre) / (ms_prefill * 1e-3) / 1e12
        pre_dense_tflops = dense_gemm_flops(s, T_pre) / (ms_prefill * 1e-3) / 1e12

    # ------------------------------------------------------------ batched decode
    batch = {}
    if "batch" in want:
        progress("batched decode")
        # one token of each of B sequences per call (rings at position 128; the
        # projections, router and experts run over the B rows, weights read once)
        for B in (8, 32, 128):
            rkb = torch.zeros((B, s.window, s.head_dim), dtype=torch.float16, device=dev)
            rvb = torch.zeros_like(rkb)
            posb = torch.full((B,), s.window, dtype=torch.int64, device=dev)
            ringb = ds4g.make_ring(rkb, rvb, posb)
            xb0 = synth.hidden(B, s.hidden, 7000 + B, device=dev)
            xb = xb0.clone()
            for i in range(2):
                xb.copy_(xb0)
                ds4g.layer_decode_batch(cfg, layers[i % nl]["cwi"], ringb, xb, B, ws,
                                            stream=stream)
            torch.cuda.synchronize()
            nb_steps = 8
            e0.record(stream)
            for i in range(nb_steps):
                ds4g.layer_decode_batch(cfg, layers[i % nl]["cwi"], ringb, xb, B, ws,
                                            stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms_b = e0.elapsed_time(e1) / nb_steps
            batch[str(B)] = {"ms_per_step": round(ms_b, 4), "tok_s": round(B / (ms_b * 1e-3), 1)}
            del rkb, rvb, posb, xb, xb0

    # ------------------------------------------------------------ lm_head + sampler
    if "lmhead" in want:
        progress("lm_head + sampler")
        V = 129280
        hw = synth.head_weights(s, V, 1004, device=dev)
        logits = torch.empty(V, dtype=torch.float32, device=dev)
        tok = torch.zeros(1, dtype=torch.int32, device=dev)
        rng = torch.tensor([synth.rng_seed(1004) & 0x7FFFFFFFFFFFFFFF], dtype=torch.int64,
                           device=dev)
        xl = xs[0].clone()

        def lm_step():
            ds4g.lmhead_sample(s.hidden, V, ds4g.BF16, hw["final_norm"], s.rms_eps, hw["lm_head"],
                               xl, 0.7, 0.95, rng, logits, tok, ws, stream=stream)
        for _ in range(5):
            lm_step()
        torch.cuda.synchronize()
        n_lm = 50
        e0.record(stream)
        for _ in range(n_lm):
            lm_step()
        e1.record(stream)
        torch.cuda.synchronize()
        us_lm = e0.elapsed_time(e1) / n_lm * 1e3
        lm_bytes = 2 * V * s.hidden + 2 * s.hidden + 4 * V

    rec = {
        "metric": "decode tok/s + layer-major prefill tok/s; % HBM BW (decode), % MFMA (prefill)",
        "value": round(1e3 / ms_decode, 2) if ms_decode else None,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_decode, 5) if ms_decode else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "one full-size layer, single-token decode at position >= 128 "
                               "(hidden 4096, 64-head MQA dh 128, QKV rank 1024, window 128, "
                               "256 experts top-6 + 1 shared, SwiGLU inter 1024, bf16 weights)",
                   "weight_sets_rotated": nl, "graph": graph is not None,
                   "global_batch": 1, "seq_len": 1, "parallelism": "none",
                   "sections": sorted(want)},
    }
    if ms_decode:
        rec["roofline"] = {"bound": "hbm", "kernel": "ds4g_layer_decode (whole layer step)",
                           "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": decode_traffic(),
                           "algorithmic_bytes": dec_bytes}
        rec["wall_s_decode"] = round(t_wall, 3)
    if "prefill" in want:
        rec["prefill"] = {"workload": "same layer, layer-major prefill of 2048 fresh N(0,1) rows "
                                      "at positions 0..2047 (empty ring)",
                          "expert_load_min_max": list(pre_load),
                          "tok_s": round(T_pre / (ms_prefill * 1e-3), 1),
                          "ms": round(ms_prefill, 4),
                          "ms_images_per_call": round(ms_prefill_img, 4),
                          "tflops_all": round(pre_tflops, 1),
                          "mfma_frac_all": round(pre_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                          "weight_bytes": prefill_weight_bytes(s),
                          "hbm_frac_weights": round(prefill_weight_bytes(s) / (ms_prefill * 1e-3)
                                                    / 1e9 / HBM_PEAK_GBS, 4)}
    if "batch" in want:
        rec["decode_batch"] = {"workload": "same layer, one decode token of each of B sequences "
                                           "per call (ds4g_layer_decode_batch), weight sets "
                                           "rotated", "by_B": batch}
    if "lmhead" in want:
        rec["lmhead_sample"] = {"workload": "RMSNorm + lm_head 129280x4096 bf16 + T=0.7 top-p 0.95",
                                "us": round(us_lm, 2),
                                "hbm_frac": round(lm_bytes / (us_lm * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                                  4)}
    if "stack" in want:
        progress("43-layer stack")
        del layers, xs, ws
        torch.cuda.empty_cache()
        rec["stack43"] = bench_stack43(args.stack_decode_steps)
    if "cpu" in want:
        progress("cpu baseline")
        rec["cpu_baseline"] = cpu_baseline(s, w_cpu, h_all, args.cpu_tokens)
        rec["cpu_baseline_prefill"] = cpu_baseline_prefill(
            s, w_cpu, args.cpu_prefill_tokens, synth.WORKLOADS["layer_prefill_2048"].seed)
    if "peaks" in want:
        progress("peaks")
        rec["measured_peaks"] = measured_peaks(dev)
        if "roofline" in rec:
            rec["measured_peaks"]["roofline_frac_vs_copy"] = round(
                rec["roofline"]["achieved"] / rec["measured_peaks"]["hbm_copy_gbs"], 4)
        rec["clocks"] = gpu_clocks()
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
