"""Prefix reuse over ring checkpoints: one live token stream on a Stack.

A client sends the whole transcript every time; the server compares it with
the live session and prefills only what is new (ds4 学习笔记 第3回 "ステート
レス API と可変セッションの接続": ds4_session_common_prefix / _sync /
_rewrite_from_common, and the tool-checkpoint canonicalisation flow; 端到端
推理流程 阶段三 "KV Cache 前缀匹配"; 阶段七: rebuilding a 16846-token common
prefix costs a near-full prefill).

With a sliding-window ring the live state cannot be rewound: the slots of
positions after the common prefix have overwritten the window before it.
So the session keeps checkpoints, every layer's ring plus the position
(2 x window x head_dim fp16 per layer), at chosen positions, and a prompt
that leaves the live stream is served from the latest checkpoint at or
before the common prefix, prefilling only the rest.  Layer-major prefill
gives every token the same arithmetic whatever batch it arrives in (spans of
the attention are aligned to absolute positions, GEMM reductions do not
depend on the row tiling), so a resumed prefill reproduces the uninterrupted
one bit for bit.

The pages' third tier, a disk KV cache keyed by rendered-byte prefixes, is
out of scope here (no tokenizer, no disk); checkpoints live in device memory.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import torch

from .stack import Stack


def common_prefix(a: Sequence[int], b: Sequence[int]) -> int:
    """Length of the longest common prefix of two token streams."""
    n = min(len(a), len(b))
    i = 0
    while i < n and int(a[i]) == int(b[i]):
        i += 1
    return i


class Session:
    """The live token stream of one Stack, with ring checkpoints.

    max_checkpoints: how many checkpoints to keep (the oldest positions are
    dropped first); checkpoint_every: besides the end of every sync, take a
    checkpoint every this many prompt tokens during a prefill (0 = only at
    the end), so a later prompt that diverges inside a long prefill still
    finds one close behind the divergence.
    """

    def __init__(self, stack: Stack, max_checkpoints: int = 8, checkpoint_every: int = 0):
        self.stack = stack
        self.tokens: List[int] = []
        self.checkpoints: Dict[int, list] = {}
        self.max_checkpoints = max_checkpoints
        self.checkpoint_every = checkpoint_every
        self.last_hidden: Optional[torch.Tensor] = None   # output of the last token, all layers

    # ------------------------------------------------------------ state
    def reset(self) -> None:
        self.stack.reset()
        self.tokens = []
        self.last_hidden = None

    def checkpoint(self) -> None:
        """Snapshot every ring at the current position, with the last token's
        output (what the lm_head needs next)."""
        p = len(self.tokens)
        last = self.last_hidden.clone() if self.last_hidden is not None else None
        self.checkpoints[p] = (self.stack.snapshot(), last)
        while len(self.checkpoints) > self.max_checkpoints:
            del self.checkpoints[min(self.checkpoints)]

    def common_prefix(self, prompt: Sequence[int]) -> int:
        """ds4_session_common_prefix: tokens shared with the live stream."""
        return common_prefix(self.tokens, prompt)

    def _best_checkpoint(self, limit: int) -> Optional[int]:
        ok = [p for p in self.checkpoints if p <= limit]
        return max(ok) if ok else None

    # ------------------------------------------------------------ prefill
    def _prefill(self, ids: Sequence[int]) -> None:
        """Append ids to the live stream with layer-major prefill, in chunks
        no longer than the stack's workspace and ending at checkpoint
        boundaries."""
        st = self.stack
        i = 0
        while i < len(ids):
            n = min(len(ids) - i, st.max_tokens)
            if self.checkpoint_every > 0:
                to_next = self.checkpoint_every - len(self.tokens) % self.checkpoint_every
                n = min(n, to_next)
            chunk = list(ids[i:i + n])
            x = st.embed(torch.as_tensor(chunk, dtype=torch.int32, device=st.device))
            st.prefill(x)
            self.last_hidden = x[-1].clone()
            self.tokens.extend(int(t) for t in chunk)
            i += n
            if self.checkpoint_every > 0 and len(self.tokens) % self.checkpoint_every == 0:
                self.checkpoint()

    def _resume_from(self, prompt: Sequence[int], common: int) -> dict:
        """Bring the live stream to `prompt`, whose first `common` tokens
        equal the live stream's."""
        # checkpoints past the common prefix belong to the old stream
        for p in [p for p in self.checkpoints if p > common]:
            del self.checkpoints[p]
        if common == len(self.tokens):
            via, start = "live", common
        else:
            ck = self._best_checkpoint(common)
            if ck is None:
                self.reset()
                via, start = "rebuild", 0
            else:
                snap, last = self.checkpoints[ck]
                self.stack.restore(snap)
                self.tokens = self.tokens[:ck]
                self.last_hidden = last.clone() if last is not None else None
                via, start = "checkpoint", ck
        suffix = list(prompt[start:])
        if suffix:
            self._prefill(suffix)
        self.checkpoint()
        return dict(via=via, common=common, reused=start, prefilled=len(suffix))

    def sync(self, prompt: Sequence[int]) -> dict:
        """ds4_session_sync: make the live stream equal `prompt`, reusing the
        live state when it is a prefix of it, else the latest checkpoint at
        or before the common prefix, else rebuilding.  Returns how
        (via = live | checkpoint | rebuild) and how many tokens were reused
        and prefilled."""
        if len(prompt) == 0:
            raise ValueError("empty prompt")
        return self._resume_from(prompt, self.common_prefix(prompt))

    def rewrite_from_common(self, canonical: Sequence[int], common: int) -> dict:
        """ds4_session_rewrite_from_common: replace the live stream after
        `common` tokens by the canonical rendering (after a tool call the
        sampled tokens and the canonical transcript differ past `common`)."""
        if common < 0 or common > min(len(canonical), len(self.tokens)):
            raise ValueError("common is not a prefix of both streams")
        if list(canonical[:common]) != self.tokens[:common]:
            raise ValueError("the streams differ before common")
        return self._resume_from(canonical, common)

    # ------------------------------------------------------------ decode
    def decode_token(self, token: int, x: torch.Tensor) -> torch.Tensor:
        """Run one token (its embedding x [hidden], updated in place) through
        every layer and append it to the live stream."""
        self.stack.decode(x)
        self.tokens.append(int(token))
        self.last_hidden = x.clone()
        return x
