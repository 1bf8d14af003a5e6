"""GPU parity of ds4g_lmhead_sample: lm_head logits against the oracle's
lm_head, and the sampled token against the oracle sampler applied to the
GPU's own logits with the same generator draw (teacher-forced)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import log, rel_l2, sampler_excused, sampler_share_tol

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import moe_dsv4_layer_amd as ds4g

LOGIT_TOL = 2e-3


def _setup(hidden, vocab, wdtype, seed):
    shape = synth.LayerShape(hidden=hidden, n_heads=1, head_dim=64, qkv_rank=64, window=1,
                             n_experts=2, top_k=1, ffn_inter=64, wdtype=wdtype)
    hw = synth.head_weights(shape, vocab, seed, device="cuda")
    ws = ds4g.alloc_workspace(ds4g.workspace_bytes(None, 0, vocab))
    return shape, hw, ws


def _run(hw, shape, vocab, x, temperature, top_p, state, ws, norm=True):
    logits = torch.empty(vocab, dtype=torch.float32, device="cuda")
    token = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rng = None
    if state is not None:   # the 64-bit generator state, stored as int64 bits
        rng = torch.tensor([np.array(state, dtype=np.uint64).view(np.int64).item()],
                           dtype=torch.int64, device="cuda")
    wd = ds4g.BF16 if shape.wdtype == synth.BF16 else ds4g.F32
    ds4g.lmhead_sample(shape.hidden, vocab, wd, hw["final_norm"] if norm else None,
                       shape.rms_eps, hw["lm_head"], x, temperature, top_p, rng, logits, token, ws)
    torch.cuda.synchronize()
    new_state = None if rng is None else int(rng.cpu().numpy().view(np.uint64)[0])
    return logits.cpu().numpy(), int(token.item()), new_state


@pytest.mark.parametrize("hidden,vocab,wdtype", [(256, 1024, synth.F32), (4096, 129280, synth.BF16),
                                                 (512, 5000, synth.BF16)])
def test_lm_head_logits_and_argmax(hidden, vocab, wdtype):
    shape, hw, ws = _setup(hidden, vocab, wdtype, 77)
    hh = {k: synth.to_host(v) for k, v in hw.items()}
    for i in range(3):
        x = synth.hidden(1, hidden, 77, stream=i, device="cuda").reshape(-1) * (1 + 3 * i)
        for norm in (True, False):
            logits, tok, _ = _run(hw, shape, vocab, x, 0.0, 0.95, None, ws, norm)
            ref = oracle.lm_head(x.cpu().numpy(), hh["final_norm"] if norm else None,
                                 hh["lm_head"], shape.rms_eps)
            e = rel_l2(logits, ref)
            log(f"lm_head V={vocab} norm={norm}: rel_l2 {e:.2e}")
            assert e < LOGIT_TOL
            assert tok == oracle.argmax(logits)          # argmax of its own logits, exactly


def _u64(s):
    return s & ((1 << 64) - 1)


@pytest.mark.parametrize("temperature,top_p", [(0.7, 0.95), (1.0, 1.0), (0.3, 0.5),
                                               (1.5, 0.99), (0.7, 1e-6), (2.0, 0.2)])
def test_sampler_teacher_forced(temperature, top_p):
    shape, hw, ws = _setup(4096, 129280, synth.BF16, 78)
    seed = synth.rng_seed(1004)
    state = seed
    agree = amb = 0
    for i in range(24):
        x = synth.hidden(1, 4096, 78, stream=i, device="cuda").reshape(-1)
        st_in = state
        logits, tok, state = _run(hw, shape, 129280, x, temperature, top_p, st_in, ws)
        g = oracle.SplitMix64(st_in)
        u = g.next_f32()
        assert _u64(state) == g.state, "generator must advance by exactly one draw"
        ref = oracle.sample(logits, temperature, top_p, u)
        if tok == ref["token"]:
            agree += 1
            continue
        # different tokens are only acceptable on a boundary of the roulette
        # or of the nucleus, closer than the GPU's fp32 weights can move it
        assert sampler_excused(ref, logits, temperature), (i, tok, ref,
                                                           sampler_share_tol(logits, temperature))
        amb += 1
    log(f"sampler T={temperature} p={top_p}: {agree} equal, {amb} on a boundary "
        f"(share tolerance {sampler_share_tol(logits, temperature):.1e})")
    assert agree >= 22


@pytest.mark.parametrize("hidden,vocab,temperature,top_p", [(1024, 262144, 0.9, 0.95),
                                                             (512, 4099, 0.7, 0.9),
                                                             (512, 4099, 1.3, 1.0)])
def test_sampler_vocab_limits_teacher_forced(hidden, vocab, temperature, top_p):
    # the largest vocabulary the call accepts (2^18: 64 weight blocks, 64
    # roulette segments) and a vocabulary that is not a multiple of the
    # 4096-entry block (a ragged last block and segment)
    shape, hw, ws = _setup(hidden, vocab, synth.BF16, 83)
    state = synth.rng_seed(1004) ^ vocab
    agree = amb = 0
    for i in range(12):
        x = synth.hidden(1, hidden, 83, stream=i, device="cuda").reshape(-1) * (1 + i % 3)
        st_in = state
        logits, tok, state = _run(hw, shape, vocab, x, temperature, top_p, st_in, ws)
        assert 0 <= tok < vocab
        g = oracle.SplitMix64(st_in)
        u = g.next_f32()
        assert _u64(state) == g.state, "generator must advance by exactly one draw"
        ref = oracle.sample(logits, temperature, top_p, u)
        if tok == ref["token"]:
            agree += 1
            continue
        assert sampler_excused(ref, logits, temperature), (i, tok, ref)
        amb += 1
    log(f"sampler V={vocab} T={temperature} p={top_p}: {agree} equal, {amb} on a boundary")
    assert agree >= 11
    # argmax at temperature 0 over the same vocabulary
    logits, tok, _ = _run(hw, shape, vocab, x, 0.0, top_p, None, ws)
    assert tok == oracle.argmax(logits)


def test_sampler_small_vocab_grid():
    # tiny vocabulary, many draws: the token histogram must follow the kept mass
    shape, hw, ws = _setup(256, 1024, synth.F32, 79)
    x = synth.hidden(1, 256, 79, device="cuda").reshape(-1) * 40.0
    logits, _, _ = _run(hw, shape, 1024, x, 0.0, 1.0, None, ws)
    state = 12345
    for i in range(200):
        st_in = state
        _, tok, state = _run(hw, shape, 1024, x, 0.8, 0.9, st_in, ws)
        u = oracle.SplitMix64(st_in).next_f32()
        ref = oracle.sample(logits, 0.8, 0.9, u)
        assert tok == ref["token"] or sampler_excused(ref, logits, 0.8), (i, tok, ref)


def _run_ex(hw, shape, vocab, x, temperature, top_p, min_p, state, ws, tdev=None):
    logits = torch.empty(vocab, dtype=torch.float32, device="cuda")
    token = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rng = torch.tensor([np.array(state, dtype=np.uint64).view(np.int64).item()],
                       dtype=torch.int64, device="cuda")
    wd = ds4g.BF16 if shape.wdtype == synth.BF16 else ds4g.F32
    ds4g.lmhead_sample_ex(shape.hidden, vocab, wd, hw["final_norm"], shape.rms_eps,
                          hw["lm_head"], x, temperature, top_p, min_p, rng, logits, token, ws,
                          temperature_dev=tdev)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), int(token.item()), int(rng.cpu().numpy().view(np.uint64)[0])


@pytest.mark.parametrize("temperature,top_p,min_p", [(0.7, 0.95, 0.05), (1.0, 1.0, 0.1),
                                                     (1.2, 0.9, 0.3), (0.7, 0.95, 0.0)])
def test_sampler_min_p_teacher_forced(temperature, top_p, min_p):
    shape, hw, ws = _setup(4096, 129280, synth.BF16, 80)
    state = synth.rng_seed(1004) ^ 0x5555
    agree = amb = 0
    for i in range(20):
        x = synth.hidden(1, 4096, 80, stream=i, device="cuda").reshape(-1) * 2.0
        st_in = state
        logits, tok, state = _run_ex(hw, shape, 129280, x, temperature, top_p, min_p, st_in, ws)
        g = oracle.SplitMix64(st_in)
        u = g.next_f32()
        assert _u64(state) == g.state, "generator must advance by exactly one draw"
        ref = oracle.sample(logits, temperature, top_p, u, min_p=min_p)
        if tok == ref["token"]:
            agree += 1
            continue
        assert sampler_excused(ref, logits, temperature), (i, tok, ref)
        amb += 1
    log(f"sampler T={temperature} p={top_p} min_p={min_p}: {agree} equal, {amb} on a boundary")
    assert agree >= 18


def test_sampler_device_temperature_override():
    # the temperature read from device memory: 0 -> argmax with the generator
    # untouched; > 0 -> the same token and draw as the host temperature
    shape, hw, ws = _setup(512, 5000, synth.BF16, 81)
    tdev = torch.zeros(1, dtype=torch.float32, device="cuda")
    for i in range(6):
        x = synth.hidden(1, 512, 81, stream=i, device="cuda").reshape(-1) * 3.0
        state = 1000 + i
        tdev.fill_(0.0)
        logits, tok, st2 = _run_ex(hw, shape, 5000, x, 0.9, 0.95, 0.0, state, ws, tdev=tdev)
        assert tok == oracle.argmax(logits) and st2 == state
        tdev.fill_(0.9)
        _, tok_d, st_d = _run_ex(hw, shape, 5000, x, 123.0, 0.95, 0.02, state, ws, tdev=tdev)
        _, tok_h, st_h = _run_ex(hw, shape, 5000, x, 0.9, 0.95, 0.02, state, ws)
        assert (tok_d, st_d) == (tok_h, st_h)
        g = oracle.SplitMix64(state)
        g.next_u64()
        assert st_d == g.state                      # exactly one draw


def test_sampler_device_temperature_in_a_graph():
    # one captured call, replayed with the device temperature switched between
    # argmax and sampling; every replay is checked against an eager call
    shape, hw, ws = _setup(512, 5000, synth.BF16, 82)
    x = synth.hidden(1, 512, 82, device="cuda").reshape(-1) * 3.0
    tdev = torch.full((1,), 0.8, dtype=torch.float32, device="cuda")
    logits = torch.empty(5000, dtype=torch.float32, device="cuda")
    token = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rng = torch.tensor([777], dtype=torch.int64, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ds4g.lmhead_sample_ex(512, 5000, ds4g.BF16, hw["final_norm"], shape.rms_eps, hw["lm_head"],
                              x, 0.0, 0.95, 0.05, rng, logits, token, ws, stream=s,
                              temperature_dev=tdev)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ds4g.lmhead_sample_ex(512, 5000, ds4g.BF16, hw["final_norm"], shape.rms_eps, hw["lm_head"],
                              x, 0.0, 0.95, 0.05, rng, logits, token, ws, stream=s,
                              temperature_dev=tdev)
    torch.cuda.synchronize()
    for i, t in enumerate([0.8, 0.0, 1.1, 0.0, 0.8]):
        tdev.fill_(t)
        state = 4242 + i
        rng.copy_(torch.tensor([state], dtype=torch.int64))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_tok, got_state = int(token.item()), int(rng.cpu().numpy().view(np.uint64)[0])
        lg, tok_e, st_e = _run_ex(hw, shape, 5000, x, t, 0.95, 0.05, state, ws)
        assert (got_tok, got_state) == (tok_e, st_e), (i, t)
        if t == 0.0:
            assert got_state == state and got_tok == oracle.argmax(lg)
