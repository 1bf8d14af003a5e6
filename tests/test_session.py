"""Prefix reuse (ds4_session_common_prefix / _sync / _rewrite_from_common)
on a stand-in stack whose state is the exact list of tokens its rings have
seen, so every route (live, checkpoint, rebuild) can be checked against a
session that prefills the whole prompt from scratch.  The GPU counterpart
(tests/test_gpu_session.py) checks bit-exactness of the real kernels."""
import torch

from moe_dsv4_layer_amd.session import Session, common_prefix


class FakeStack:
    """Rings = the token list since reset; embed/prefill/decode append."""

    def __init__(self, max_tokens=16):
        self.max_tokens, self.device = max_tokens, "cpu"
        self.seen, self.prefill_rows = [], 0

    def reset(self):
        self.seen = []

    def snapshot(self):
        return list(self.seen)

    def restore(self, snap):
        self.seen = list(snap)

    def embed(self, ids):
        return ids.to(torch.float32).reshape(-1, 1).repeat(1, 3)

    def prefill(self, x):
        self.prefill_rows += x.shape[0]
        self.seen.extend(int(v) for v in x[:, 0])
        x += len(self.seen)          # an output that depends on the whole history
        return x

    def decode(self, x):
        self.seen.append(int(x[0]))
        x += len(self.seen)
        return x


def _fresh(prompt, **kw):
    s = Session(FakeStack(), **kw)
    s.sync(prompt)
    return s


def test_common_prefix():
    assert common_prefix([1, 2, 3], [1, 2, 4]) == 2
    assert common_prefix([], [1]) == 0
    assert common_prefix([5, 6], [5, 6, 7]) == 2
    assert common_prefix([5, 6, 7], [5, 6]) == 2


def test_sync_routes():
    a = list(range(40))
    s = Session(FakeStack(), checkpoint_every=8)
    r = s.sync(a)
    assert r["via"] == "live" and r["prefilled"] == 40      # empty live stream is a prefix
    # the live stream is a prefix of the next prompt: only the suffix runs
    b = a + [100, 101, 102]
    rows = s.stack.prefill_rows
    r = s.sync(b)
    assert r == dict(via="live", common=40, reused=40, prefilled=3)
    assert s.stack.prefill_rows - rows == 3
    # divergence at 29: the checkpoint at 24 serves it
    c = a[:29] + [7, 7, 7, 7]
    r = s.sync(c)
    assert r["via"] == "checkpoint" and r["reused"] == 24 and r["prefilled"] == 9
    assert s.stack.seen == c and s.tokens == c
    assert max(p for p in s.checkpoints) == len(c)
    # every kept checkpoint is a prefix of the new stream (old-stream ones gone)
    assert all(snap == c[:p] for p, (snap, _) in s.checkpoints.items())
    # divergence before any checkpoint: rebuild
    d = [9] + a[1:5]
    r = s.sync(d)
    assert r["via"] == "rebuild" and r["prefilled"] == len(d)
    assert s.stack.seen == d


def test_resumed_state_equals_fresh_state():
    a = list(range(50))
    for cut in (0, 7, 16, 31, 49):
        b = a[:cut] + [900 + i for i in range(11)]
        s = Session(FakeStack(), checkpoint_every=16)
        s.sync(a)
        s.sync(b)
        f = _fresh(b)
        assert s.stack.seen == f.stack.seen == b
        assert torch.equal(s.last_hidden, f.last_hidden)


def test_prompt_that_is_a_prefix_of_the_live_stream():
    a = list(range(30))
    s = Session(FakeStack(), checkpoint_every=10)
    s.sync(a)
    r = s.sync(a[:20])
    assert r["via"] == "checkpoint" and r["reused"] == 20 and r["prefilled"] == 0
    assert s.stack.seen == a[:20]
    assert torch.equal(s.last_hidden, _fresh(a[:20]).last_hidden)


def test_rewrite_from_common_and_decode():
    s = Session(FakeStack(), checkpoint_every=4)
    s.sync([1, 2, 3, 4, 5, 6])
    x = torch.full((3,), 42.0)
    s.decode_token(42, x)                     # the sampled tool-call token
    assert s.tokens == [1, 2, 3, 4, 5, 6, 42]
    canonical = [1, 2, 3, 4, 5, 6, 40, 41]    # the canonical rendering differs at 6
    r = s.rewrite_from_common(canonical, common_prefix(s.tokens, canonical))
    assert r["via"] == "checkpoint" and r["reused"] == 6 and s.stack.seen == canonical
    try:
        s.rewrite_from_common([9, 9], 1)
        raise AssertionError("expected ValueError")
    except ValueError:
        pass
