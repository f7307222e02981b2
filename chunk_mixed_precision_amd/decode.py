"""Streaming decode over the mixed-precision cache.

The context grows one token per step and sequence.  Tokens of the chunk
being filled wait in an fp16 tail that attention reads directly; when the
tail holds C tokens it becomes a chunk: it is routed (one routing for every
layer: routing sharing; chunk 0 frozen to FP16 when freezing is on), each
layer's K/V chunk is quantized at the voted bitwidth and written to the
chunk's slot of its bitwidth segment (MoQAE "Overall framework" and "Key
designs"; Cocktail abstract for the segments).  When a segment outgrows its
pool, the pool is re-laid out for a larger capacity.

This module only sequences calls of the C ABI and allocates device memory
through torch; every computation runs in the library's kernels.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import torch

from . import mkv

EXPERT_BITS = (16, 4, 2)


class DecodeSession:
    """One batch of B sequences decoding in lockstep through `layers` layers.

    Router weights (w12 [2I, D] bf16, w3 [3, I] f32, b3 [3] f32) route each
    completed chunk from its tokens' hidden states.  Tables hold up to
    `max_chunks` chunks per sequence.  Pools start at `caps` slots per
    (sequence, head) and grow by `growth` (at least to what is needed) when
    a routed chunk does not fit.
    """

    def __init__(self, B: int, Hq: int, Hkv: int, d: int, C: int, layers: int, w12: torch.Tensor,
                 w3: torch.Tensor, b3: torch.Tensor, max_chunks: int, caps: Sequence[int] = (1, 1, 1),
                 growth: float = 1.5, freeze_first: bool = True, device="cuda"):
        self.B, self.Hq, self.Hkv, self.d, self.C, self.layers = B, Hq, Hkv, d, C, layers
        self.D = w12.shape[1]
        self.w12, self.w3, self.b3 = w12, w3, b3
        self.freeze_first = freeze_first
        self.growth = growth
        self.dev = device
        self.tab = mkv.RouteTables(B, max_chunks, device)
        self.n = 0              # chunks routed and quantized
        self.tail_len = 0       # tokens waiting in the tails
        self.grown = 0          # pool re-layouts so far
        self.caps = [max(1, int(c)) for c in caps]
        self.x_tail = torch.empty((B, C, self.D), dtype=torch.bfloat16, device=device)
        self.k_tail = [torch.empty((B, Hkv, C, d), dtype=torch.float16, device=device) for _ in range(layers)]
        self.v_tail = [torch.empty((B, Hkv, C, d), dtype=torch.float16, device=device) for _ in range(layers)]
        self.caches = [mkv.PackedCache(B, Hkv, d, C, self.caps, self.tab.seg_count, device) for _ in range(layers)]
        self._workspaces()
        self.ws_route = None

    # ------------------------------------------------------------ internals
    def _workspaces(self):
        self.ws_attn = [mkv.attention_workspace(self.B, self.Hq, c, self.dev) for c in self.caches]

    def _route(self, x: torch.Tensor, chunk_offset: int, logits: torch.Tensor = None):
        if logits is not None:
            mkv.route_chunks(self.tab, self.C, logits=logits, logits_in=True, freeze_first=self.freeze_first,
                             append=chunk_offset > 0, chunk_offset=chunk_offset)
            return
        B, T, D = x.shape
        need = mkv.workspace_bytes_route(B, T, D, self.w12.shape[0] // 2)
        if self.ws_route is None or self.ws_route.numel() < need:
            self.ws_route = torch.empty(need, dtype=torch.uint8, device=self.dev)
        mkv.route_chunks(self.tab, self.C, x=x, w12=self.w12, w3=self.w3, b3=self.b3,
                         freeze_first=self.freeze_first, append=chunk_offset > 0, chunk_offset=chunk_offset,
                         workspace=self.ws_route)

    def _ensure_capacity(self):
        """Grow every pool whose segment now holds more chunks than slots.
        Reads the segment counts back (one small synchronous copy per
        routed chunk batch)."""
        need = self.tab.seg_count.cpu().max(dim=0).values.tolist()
        grew = False
        for k, bits in enumerate(EXPERT_BITS):
            if need[k] <= self.caps[k]:
                continue
            new_cap = max(int(need[k]), int(math.ceil(self.caps[k] * self.growth)))
            for cache in self.caches:
                old = cache.pools[k]
                new = torch.empty(mkv.pool_bytes(bits, self.B, self.Hkv, new_cap, self.d, self.C),
                                  dtype=torch.uint8, device=self.dev)
                mkv.grow_pool(old, new, bits, self.B, self.Hkv, self.caps[k], new_cap, self.d, self.C)
                cache.pools[k] = new
                cache.caps[k] = new_cap
            self.caps[k] = new_cap
            self.grown += 1
            grew = True
        if grew:
            self._workspaces()

    def _append_chunks(self, x: torch.Tensor, kv: Sequence[Tuple[torch.Tensor, torch.Tensor]],
                       logits: torch.Tensor = None):
        T = (x if logits is None else logits).shape[1]
        self._route(x, self.n, logits)
        self._ensure_capacity()
        for cache, (k, v) in zip(self.caches, kv):
            mkv.quantize_pack_kv(k, v, self.tab, cache, chunk_offset=self.n)
        self.n += T // self.C

    # ------------------------------------------------------------ API
    def prefill(self, x: Optional[torch.Tensor], kv: Sequence[Tuple[torch.Tensor, torch.Tensor]],
                logits: torch.Tensor = None):
        """Whole chunks of context: x [B, T, D] bf16 hidden states (or, in
        their place, final per-token expert scores `logits` [B, T, 3] f32),
        kv[l] = (k, v) [B, Hkv, T, d] fp16 per layer, T a multiple of C.
        Only valid while the tail is empty."""
        if self.tail_len:
            raise ValueError("prefill needs an empty tail")
        if (x if logits is None else logits).shape[1] % self.C:
            raise ValueError("prefill takes whole chunks")
        self._append_chunks(x, kv, logits)

    def step(self, x_t: torch.Tensor, kv_t: Sequence[Tuple[torch.Tensor, torch.Tensor]],
             q_t: Sequence[torch.Tensor], out: Optional[List[torch.Tensor]] = None) -> List[torch.Tensor]:
        """One token per sequence: x_t [B, D] bf16, kv_t[l] = (k, v) [B, Hkv, d]
        fp16, q_t[l] [B, Hq, d] fp16.  Returns each layer's attention output
        [B, Hq, d] f32 over every earlier token and this one; then, if the
        chunk is complete, routes, quantizes and appends it."""
        pos = self.tail_len
        mkv.append_tail_rows(x_t, self.x_tail, pos)
        for l, (k, v) in enumerate(kv_t):
            mkv.append_tail_rows(k, self.k_tail[l], pos, v, self.v_tail[l])
        self.tail_len += 1
        outs = []
        for l in range(self.layers):
            o = None if out is None else out[l]
            outs.append(mkv.mixed_kv_decode_attention(q_t[l], self.caches[l], out=o, tail_k=self.k_tail[l],
                                                      tail_v=self.v_tail[l], tail_len=self.tail_len,
                                                      workspace=self.ws_attn[l]))
        if self.tail_len == self.C:
            self._append_chunks(self.x_tail, list(zip(self.k_tail, self.v_tail)))
            self.tail_len = 0
        return outs
