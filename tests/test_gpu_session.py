"""Prefix reuse on the GPU: a session that serves a new prompt from a ring
checkpoint plus a suffix prefill must end in exactly the state (every ring,
position, last hidden state, logits) of a session that prefills the whole
prompt at once; the checkpointed chunks and the one-shot prefill tile the
tokens differently, so this also pins that layer-major prefill does not
depend on how a prompt is split.  The resumed state is also compared with
the oracle's layer-major prefill of the new prompt (last hidden state,
rings, logits and the greedy token)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import log, rel_l2, small_shape

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from moe_dsv4_layer_amd.session import Session   # noqa: E402
from moe_dsv4_layer_amd.stack import Stack       # noqa: E402


def _stack(shape, layers, head, max_tokens):
    return Stack(shape, layers, head, max_tokens=max_tokens)


def _logits(st, h):
    st.sample(h.clone(), 0.0, 1.0)
    torch.cuda.synchronize()
    return st.logits.clone(), int(st.token.item())


def _same_state(a: Session, b: Session):
    assert a.tokens == b.tokens
    for l in range(len(a.stack.layers)):
        assert torch.equal(a.stack.pos[l], b.stack.pos[l])
        assert torch.equal(a.stack.ring_k[l], b.stack.ring_k[l]), l
        assert torch.equal(a.stack.ring_v[l], b.stack.ring_v[l]), l
    assert torch.equal(a.last_hidden, b.last_hidden)


@pytest.mark.parametrize("wdtype", [synth.BF16, synth.F32])
def test_session_reuse_is_bit_exact(wdtype):
    shape = small_shape(wdtype=wdtype)
    vocab, n_layers = 1024, 2
    layers = [synth.layer_weights(shape, 41, layer=l, device="cuda") for l in range(n_layers)]
    head = synth.head_weights(shape, vocab, 41, device="cuda")
    A = [int(t) for t in synth.token_ids(100, vocab, 41)]
    B = A[:75] + [int(t) for t in synth.token_ids(30, vocab, 42)]
    live = Session(_stack(shape, layers, head, 64), checkpoint_every=32)
    r1 = live.sync(A)
    r2 = live.sync(B)
    log(f"session {wdtype}: {r1} then {r2}")
    assert r2["via"] == "checkpoint" and r2["reused"] == 64 and r2["prefilled"] == len(B) - 64
    fresh = Session(_stack(shape, layers, head, 128))
    fresh.sync(B)
    torch.cuda.synchronize()
    _same_state(live, fresh)
    la, ta = _logits(live.stack, live.last_hidden)
    lb, tb = _logits(fresh.stack, fresh.last_hidden)
    assert torch.equal(la, lb) and ta == tb
    # the resumed session against the oracle's prefill of prompt B
    wh = [synth.weights_to_host(w) for w in layers]
    hh = {k: synth.to_host(v) for k, v in head.items()}
    rings = [oracle.Ring(shape.window, shape.head_dim) for _ in layers]
    xo, _ = oracle.stack_prefill(shape, wh, rings, oracle.embed(B, hh["embed"]))
    e_h = rel_l2(live.last_hidden.cpu().numpy(), xo[-1])
    lo = oracle.lm_head(xo[-1], hh["final_norm"], hh["lm_head"], shape.rms_eps)
    e_lg = rel_l2(la.cpu().numpy(), lo)
    lt = oracle.lm_head(live.last_hidden.cpu().numpy(), hh["final_norm"], hh["lm_head"],
                        shape.rms_eps)
    e_tf = rel_l2(la.cpu().numpy(), lt)
    e_r = max(max(rel_l2(live.stack.ring_k[l].float().cpu().numpy(), rings[l].k),
                  rel_l2(live.stack.ring_v[l].float().cpu().numpy(), rings[l].v))
              for l in range(n_layers))
    srt = np.sort(lo)
    log(f"session {wdtype} vs oracle: hidden {e_h:.2e}, logits {e_lg:.2e} (lm_head alone "
        f"{e_tf:.2e}), rings {e_r:.2e}, top-2 gap {srt[-1] - srt[-2]:.2e}")
    assert e_h < 1e-2 and e_r < 1e-2 and e_lg < 1e-2 and e_tf < 2e-3
    assert all(int(live.stack.pos[l].item()) == rings[l].pos == len(B) for l in range(n_layers))
    if srt[-1] - srt[-2] > 1e-2:
        assert ta == oracle.argmax(lo)
    # the live stream grows by decoding; a prompt that extends it is served live
    x = live.stack.embed(torch.tensor([ta], dtype=torch.int32, device="cuda"))[0]
    live.decode_token(ta, x)
    r3 = live.sync(live.tokens + [5, 6, 7])
    assert r3["via"] == "live" and r3["prefilled"] == 3
