"""Workload shapes and byte accounting for the mixed-precision KV path.

The five workloads mirror the model families the MoQAE and XQuant pages
evaluate (LLaMA-2 7B / 13B layers, a LLaMA-3-8B-like GQA layer), each
with its sizes below; all tensors are synthetic (see ``synth``).
"""
from __future__ import annotations

import dataclasses
import json
import os
from dataclasses import dataclass, field
from typing import Optional, Tuple

EXPERT_BITS = (16, 4, 2)
GROUP = 32

_HERE = os.path.dirname(os.path.abspath(__file__))


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int                  # sequences
    Hq: int                 # query heads
    Hkv: int                # KV heads
    d: int                  # head dim
    T: int                  # cached tokens per sequence (prefill)
    C: int                  # chunk size
    D: int = 0              # router hidden size (0: router not run, mix drawn)
    I: int = 0              # router inner size
    layers: int = 1
    mix: Tuple[float, float, float] = (0.0, 1.0, 0.0)   # target chunk fractions FP16/INT4/INT2
    outlier_cols: int = 0   # number of (kv head, channel) key columns scaled up
    outlier_mult: float = 1.0
    outlier_first_channels: int = 0   # if > 0: channels 0..k-1 of every head are outliers
    x_chunk_share: float = 1.0        # a in x = (a*mu_c + z_t)/sqrt(1+a^2); 0 -> iid x
    append_chunks: int = 0            # chunks appended (routed) per step
    router_std: float = 0.02
    b3: Tuple[float, float, float] = (0.0, 0.0, 0.0)

    @property
    def n(self) -> int:
        return self.T // self.C

    @property
    def n_total(self) -> int:
        return self.n + self.append_chunks

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def routed(self) -> bool:
        return self.D > 0


def fp16_kv_bytes(layers: int, heads: int, head_dim: int, tokens: int) -> int:
    """K and V in fp16: 2 tensors x layers x heads x head_dim x 2 bytes x tokens."""
    return 2 * layers * heads * head_dim * 2 * tokens


def bytes_per_token_head(bits: int, d: int) -> int:
    """Algorithmic bytes one cached token of one KV head occupies (K and V):
    FP16: 2 x d x 2 B.  INT-b: 2 x (d*b/8 code bytes + d/32 groups x 8 B
    of float32 (scale, min))."""
    if bits == 16:
        return 4 * d
    return 2 * (d * bits // 8 + (d // GROUP) * 8)


def chunk_bytes(bits: int, d: int, C: int) -> int:
    return bytes_per_token_head(bits, d) * C


def _load_calibrated():
    p = os.path.join(_HERE, "calibrated_b3.json")
    if not os.path.exists(p):
        return {}
    with open(p) as f:
        return json.load(f)


_CAL = _load_calibrated()


def _b3(name, default=(0.0, 0.0, 0.0)):
    e = _CAL.get(name)
    return tuple(e["b3"]) if e else default


TINY = Workload(
    name="tiny-1x4x64-T1024-C128", seed=1, B=1, Hq=4, Hkv=4, d=64, T=1024, C=128,
    D=256, I=128, outlier_first_channels=4, outlier_mult=10.0, x_chunk_share=0.0,
    mix=(1 / 8, 7 / 8, 0.0))

LLAMA2_7B_32K = Workload(
    name="llama2-7b-layer-T32768-C256", seed=2, B=1, Hq=32, Hkv=32, d=128, T=32768, C=256,
    D=4096, I=1024, mix=(0.03, 0.90, 0.07), outlier_cols=82, outlier_mult=8.0,
    x_chunk_share=1.0, b3=_b3("llama2-7b-layer-T32768-C256"))

LLAMA2_13B_40L = Workload(
    name="llama2-13b-40layers-B16-T8192-C128", seed=3, B=16, Hq=40, Hkv=40, d=128, T=8192,
    C=128, layers=40, mix=(0.03, 0.79, 0.18), outlier_cols=102, outlier_mult=8.0)

LLAMA2_7B_128K = Workload(
    name="llama2-7b-layer-T131072-C128", seed=4, B=1, Hq=32, Hkv=32, d=128, T=131072, C=128,
    D=4096, I=1024, mix=(0.05, 0.35, 0.60), outlier_cols=82, outlier_mult=8.0,
    x_chunk_share=1.0, b3=_b3("llama2-7b-layer-T131072-C128"))

LLAMA3_8B_GQA = Workload(
    name="llama3-8b-gqa-B64-T8192+256-C256", seed=5, B=64, Hq=32, Hkv=8, d=128, T=8192, C=256,
    D=4096, I=1024, mix=(0.03, 0.90, 0.07), outlier_cols=20, outlier_mult=8.0,
    x_chunk_share=1.0, append_chunks=1, b3=_b3("llama3-8b-gqa-B64-T8192+256-C256"))

ALL = (TINY, LLAMA2_7B_32K, LLAMA2_13B_40L, LLAMA2_7B_128K, LLAMA3_8B_GQA)
BY_NAME = {w.name: w for w in ALL}


def scaled(w: Workload, **kw) -> Workload:
    """A copy with some fields replaced (used for reduced-size test cases)."""
    return dataclasses.replace(w, **kw)


def effective_attention_bytes(w: Workload, seg_count) -> int:
    """Algorithmic bytes one decode step reads for one layer: the packed KV of
    every (sequence, KV head) plus q (fp16) and the fp32 output.
    seg_count: iterable of per-sequence (n16, n4, n2) chunk counts."""
    total = 0
    for cnt in seg_count:
        for k, bits in enumerate(EXPERT_BITS):
            total += int(cnt[k]) * chunk_bytes(bits, w.d, w.C) * w.Hkv
    total += w.B * w.Hq * w.d * (2 + 4)
    return total
