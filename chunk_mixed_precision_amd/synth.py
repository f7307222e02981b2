"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no arithmetic of the method: it only draws random tensors
with the shapes and value distributions of the workloads in ``configs``.
Every stream is a torch.Generator seeded with seed*100 + stream
(+ 10000*layer for per-layer tensors):

  1 hidden states x   2 W12   3 W3   4 K   5 V   6 q
  7 outlier key columns   8 drawn chunk mix   9 chunk means of x

The router's hidden states and weights are always drawn on the CPU, so the
same bytes exist wherever the calibration of the router bias ran; K, V and q
are drawn on the requested device.
"""
from __future__ import annotations

import math

import torch

from .configs import EXPERT_BITS, Workload


def _gen(seed: int, stream: int, layer: int = 0, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 100 + stream + 10000 * layer)
    return g


def router_inputs(w: Workload, tokens_per_seq: int = None, batch: int = None,
                  chunk_offset: int = 0, layer: int = 0):
    """x [B, T, D] bf16 (chunk-structured), W12 [2I, D] bf16, W3 [3, I] f32,
    b3 [3] f32, all on the CPU.

    x_t = (a * mu_c + z_t) / sqrt(1 + a^2) with mu_c, z_t ~ N(0, I_D), where c
    is the chunk of token t (a = w.x_chunk_share; a = 0 gives iid N(0,1)).
    ``chunk_offset`` selects which chunks' hidden states to draw (appends
    draw chunks after the prefill).  ``layer`` draws another block's hidden
    states and router (every block has its own router; layer 0 is the block
    whose routing is shared when routing sharing is on)."""
    B = w.B if batch is None else batch
    T = w.T if tokens_per_seq is None else tokens_per_seq
    D, I = w.D, w.I
    n = T // w.C
    gz = _gen(w.seed, 1 + 1000 * chunk_offset, layer)
    z = torch.randn((B, T, D), generator=gz, dtype=torch.float32)
    a = w.x_chunk_share
    if a > 0:
        gm = _gen(w.seed, 9 + 1000 * chunk_offset, layer)
        mu = torch.randn((B, n, 1, D), generator=gm, dtype=torch.float32)
        z = z.view(B, n, w.C, D)
        z.mul_(1.0 / math.sqrt(1 + a * a)).add_(mu, alpha=a / math.sqrt(1 + a * a))
        z = z.view(B, T, D)
    x = z.to(torch.bfloat16)
    del z
    w12 = (torch.randn((2 * I, D), generator=_gen(w.seed, 2, layer), dtype=torch.float32)
           * w.router_std).to(torch.bfloat16)
    w3 = torch.randn((3, I), generator=_gen(w.seed, 3, layer), dtype=torch.float32) * w.router_std
    b3 = torch.tensor(w.b3, dtype=torch.float32)
    return x, w12, w3, b3


def query_embedding(w: Workload, batch: int = None, layer: int = 0) -> torch.Tensor:
    """qe [B, D] bf16 on the CPU: a query embedding drawn near the chunk mean
    mu_c of one seeded chunk c of each sequence (the mu_c of router_inputs),
    qe = (mu_c + z) / sqrt(2), z ~ N(0, I_D); with iid hidden states
    (x_chunk_share = 0) just z."""
    B = w.B if batch is None else batch
    D, n = w.D, w.T // w.C
    z = torch.randn((B, D), generator=_gen(w.seed, 11, layer), dtype=torch.float32)
    if w.x_chunk_share > 0:
        mu = torch.randn((B, n, 1, D), generator=_gen(w.seed, 9, layer), dtype=torch.float32)
        pick = torch.randint(0, n, (B,), generator=_gen(w.seed, 10, layer))
        z = (mu[torch.arange(B), pick, 0] + z) / math.sqrt(2.0)
    return z.to(torch.bfloat16)


def decode_tokens(w: Workload, steps: int, device, layer: int = 0):
    """Per-step inputs of a streaming decode, drawn on the device: hidden
    states x [steps, B, D] bf16 (iid N(0,1)), k, v [steps, B, Hkv, d] fp16
    and q [steps, B, Hq, d] fp16 (N(0,1); outlier key columns scaled as in
    ``kv``)."""
    g = _gen(w.seed, 12, layer, device)
    x = torch.randn((steps, w.B, w.D), generator=g, device=device).to(torch.bfloat16)
    k = torch.randn((steps, w.B, w.Hkv, w.d), generator=g, device=device)
    v = torch.randn((steps, w.B, w.Hkv, w.d), generator=g, device=device)
    k.mul_(outlier_mask(w).to(device)[None, None])
    q = torch.randn((steps, w.B, w.Hq, w.d), generator=g, device=device)
    return x, k.to(torch.float16), v.to(torch.float16), q.to(torch.float16)


def outlier_mask(w: Workload) -> torch.Tensor:
    """[Hkv, d] float multiplier for the key columns (KIVI-style outlier
    channels): channels 0..k-1 of every head, or a seeded set of columns."""
    m = torch.ones((w.Hkv, w.d), dtype=torch.float32)
    if w.outlier_first_channels:
        m[:, :w.outlier_first_channels] = w.outlier_mult
    if w.outlier_cols:
        idx = torch.randperm(w.Hkv * w.d, generator=_gen(w.seed, 7))[:w.outlier_cols]
        m.view(-1)[idx] = w.outlier_mult
    return m


def kv(w: Workload, device, layer: int = 0, tokens: int = None, token_offset_stream: int = 0):
    """K, V [B, Hkv, T, d] fp16 on ``device``; K ~ N(0,1) with the outlier
    columns scaled, V ~ N(0,1)."""
    T = w.T if tokens is None else tokens
    shp = (w.B, w.Hkv, T, w.d)
    gk = _gen(w.seed, 4 + 1000 * token_offset_stream, layer, device)
    gv = _gen(w.seed, 5 + 1000 * token_offset_stream, layer, device)
    k = torch.randn(shp, generator=gk, device=device, dtype=torch.float32)
    k.mul_(outlier_mask(w).to(device)[None, :, None, :])
    k = k.to(torch.float16)
    v = torch.randn(shp, generator=gv, device=device, dtype=torch.float16)
    return k, v


def query(w: Workload, device, layer: int = 0) -> torch.Tensor:
    """q [B, Hq, d] fp16 ~ N(0, 1)."""
    g = _gen(w.seed, 6, layer, device)
    return torch.randn((w.B, w.Hq, w.d), generator=g, device=device, dtype=torch.float16)


def drawn_chunk_experts(w: Workload, n: int = None) -> torch.Tensor:
    """[B, n] expert index per chunk drawn iid from w.mix (CPU, uint8).
    This is input data (a stand-in for a trained router's decisions), not a
    vote; chunk 0 is drawn like any other chunk."""
    n = w.n if n is None else n
    u = torch.rand((w.B, n), generator=_gen(w.seed, 8), dtype=torch.float64)
    f0, f1, _ = w.mix
    e = torch.full((w.B, n), 2, dtype=torch.uint8)
    e[u < f0 + f1] = 1
    e[u < f0] = 0
    return e


def one_hot_logits(experts: torch.Tensor, C: int) -> torch.Tensor:
    """Logits [B, n*C, 3] f32 that make every token of chunk c pick
    experts[b, c] (1.0 for the chosen expert, 0.0 elsewhere)."""
    B, n = experts.shape
    z = torch.zeros((B, n, C, 3), dtype=torch.float32)
    z.scatter_(3, experts.long()[:, :, None, None].expand(B, n, C, 1), 1.0)
    return z.view(B, n * C, 3)


def bits_tensor(experts: torch.Tensor) -> torch.Tensor:
    lut = torch.tensor(EXPERT_BITS, dtype=torch.uint8)
    return lut[experts.long()]
