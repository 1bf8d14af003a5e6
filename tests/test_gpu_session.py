"""Prefix reuse on the GPU: a session that serves a new prompt from a ring
checkpoint plus a suffix prefill must end in exactly the state (every ring,
position, last hidden state, logits) of a session that prefills the whole
prompt at once; the checkpointed chunks and the one-shot prefill tile the
tokens differently, so this also pins that layer-major prefill does not
depend on how a prompt is split."""
import pytest
import torch

import synth
from tests.harness import log, small_shape

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
    # the live stream grows by decoding; a prompt that extends it is served live
    x = live.stack.embed(torch.tensor([ta], dtype=torch.int32, device="cuda"))[0]
    live.decode_token(ta, x)
    r3 = live.sync(live.tokens + [5, 6, 7])
    assert r3["via"] == "live" and r3["prefilled"] == 3
