"""A stack of layers on one GPU, driven through the C ABI.

The driver only sequences calls: embedding (ds4g_embed), the layers in
layer-major order for a prompt (ds4g_layer_prefill, 阶段三 逐层批处理 on
ds4-learning 端到端推理流程) or one token at a time (ds4g_layer_decode,
阶段四 4.2), then the lm_head and sampler (ds4g_lmhead_sample, 阶段四 4.3).
Each layer owns a KV ring; snapshot()/restore() copy every ring and its
position, which is how a cached prefix is resumed (the rebuild-vs-reuse case
of 阶段七).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import torch

from . import (BF16, F32, alloc_workspace, embed, layer_decode, layer_prefill, lmhead_sample,
               make_cfg, make_f16_images, make_ring, make_routing, make_weights,
               workspace_bytes)


class Stack:
    def __init__(self, shape, layers: Sequence[Dict[str, torch.Tensor]],
                 head: Dict[str, torch.Tensor], max_tokens: int, device="cuda",
                 prepare_images: bool = True):
        """prepare_images (bf16 weights): make every layer's fp16
        attention-path images once (ds4g_make_f16_images), as an engine does
        when it loads weights, instead of in every prefill."""
        self.shape = shape
        self.cfg = make_cfg(shape)
        self.wdtype = BF16 if self.cfg.wdtype == BF16 else F32
        self.layers = list(layers)
        self.images = [None] * len(self.layers)
        if prepare_images and self.wdtype == BF16:
            self.images = [make_f16_images(self.cfg, make_weights(w), device)
                           for w in self.layers]
        self.cw = [make_weights(w, img) for w, img in zip(self.layers, self.images)]
        self.head = head
        self.vocab = head["lm_head"].shape[0]
        self.device = device
        dh, W = shape.head_dim, shape.window
        self.ring_k = [torch.zeros((W, dh), dtype=torch.float16, device=device) for _ in layers]
        self.ring_v = [torch.zeros((W, dh), dtype=torch.float16, device=device) for _ in layers]
        self.pos = [torch.zeros(1, dtype=torch.int64, device=device) for _ in layers]
        self.rings = [make_ring(k, v, p) for k, v, p in zip(self.ring_k, self.ring_v, self.pos)]
        self.ws = alloc_workspace(workspace_bytes(self.cfg, max_tokens, self.vocab), device)
        self.max_tokens = max_tokens
        self.logits = torch.empty(self.vocab, dtype=torch.float32, device=device)
        self.token = torch.zeros(1, dtype=torch.int32, device=device)

    # ------------------------------------------------------------ state
    def reset(self) -> None:
        for k, v, p in zip(self.ring_k, self.ring_v, self.pos):
            k.zero_()
            v.zero_()
            p.zero_()

    def snapshot(self) -> List[tuple]:
        return [(k.clone(), v.clone(), p.clone())
                for k, v, p in zip(self.ring_k, self.ring_v, self.pos)]

    def restore(self, snap) -> None:
        for (k, v, p), (sk, sv, sp) in zip(zip(self.ring_k, self.ring_v, self.pos), snap):
            k.copy_(sk)
            v.copy_(sv)
            p.copy_(sp)

    # ------------------------------------------------------------ compute
    def embed(self, ids: torch.Tensor) -> torch.Tensor:
        """ids: device int32 [T] -> fp32 [T, hidden]."""
        x = torch.empty((ids.numel(), self.shape.hidden), dtype=torch.float32, device=self.device)
        embed(self.vocab, self.shape.hidden, self.wdtype, self.head["embed"], ids, x)
        return x

    def prefill(self, x: torch.Tensor, layer_inputs: Optional[list] = None,
                routing: Optional[list] = None,
                capture: Optional[Dict[int, torch.Tensor]] = None) -> torch.Tensor:
        """Layer-major prefill of x [T, hidden] (updated in place) through
        every layer.  layer_inputs, if a list, receives a copy of each
        layer's input; capture, if a dict, a copy of the input of each layer
        named by its keys; routing, if a list of dicts, gets each layer's
        routing buffers."""
        T = x.shape[0]
        assert T <= self.max_tokens
        for l in range(len(self.layers)):
            if layer_inputs is not None:
                layer_inputs.append(x.clone())
            if capture is not None and l in capture:
                capture[l] = x.clone()
            r = make_routing(routing[l]) if routing is not None else None
            layer_prefill(self.cfg, self.cw[l], self.rings[l], x, T, self.ws, r)
        return x

    def decode(self, x: torch.Tensor, layer_inputs: Optional[list] = None) -> torch.Tensor:
        """One token x [hidden] (updated in place) through every layer."""
        for l in range(len(self.layers)):
            if layer_inputs is not None:
                layer_inputs.append(x.clone())
            layer_decode(self.cfg, self.cw[l], self.rings[l], x, self.ws)
        return x

    def sample(self, x: torch.Tensor, temperature: float, top_p: float,
               rng: Optional[torch.Tensor] = None, x_next: Optional[torch.Tensor] = None):
        """lm_head + sampler on the last hidden x [hidden]; the token stays on
        the device (self.token); x_next, if given, gets its embedding."""
        lmhead_sample(self.shape.hidden, self.vocab, self.wdtype, self.head["final_norm"],
                      self.shape.rms_eps, self.head["lm_head"], x, temperature, top_p, rng,
                      self.logits, self.token, self.ws,
                      embed_table=self.head["embed"] if x_next is not None else None,
                      x_next=x_next)
        return self.token
