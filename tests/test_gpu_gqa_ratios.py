"""GPU parity of decode attention at grouped-query ratios other than 1, 2
and 4 query heads per KV head: the library attends a KV head's query heads
in groups of 4, 2 and 1 (one launch pair per group), so 3 = 2 + 1, 5 = 4 +
1, 6 = 4 + 2, 8 = 4 + 4 and 16 = 4 x 4 cover every group shape and its head
offsets.  Every (sequence, query head) against the oracle, with and without
an fp16 tail, at head_dim 64 and 128; the no-allocation entry point on one
such ratio."""
import numpy as np
import pytest
import torch

from chunk_mixed_precision_amd import configs, mkv, synth
from tests import parity as P
from tests.test_gpu_parity import build_tables_from_experts, check_canary, full_check, run_quant_attn, tables_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("g,d,tail", [(3, 128, 0), (5, 64, 7), (6, 128, 29), (8, 128, 0), (8, 64, 17),
                                      (16, 128, 3)])
def test_gqa_ratio(g, d, tail):
    Hkv = 2
    w = configs.Workload(name=f"gqa-{g}to1-d{d}-t{tail}", seed=500 + 7 * g + d + tail, B=3, Hq=g * Hkv, Hkv=Hkv, d=d,
                         T=1024, C=128, mix=(0.2, 0.5, 0.3), outlier_cols=2, outlier_mult=8.0)
    note(f"{w.name}")
    experts = synth.drawn_chunk_experts(w)
    tab = build_tables_from_experts(experts, w.C, freeze=True)
    k, v = synth.kv(w, DEV)
    q = synth.query(w, DEV)
    cache, out, tk, tv = run_quant_attn(w, tab, k, v, q, w.n, tail=tail)
    bits, rank, perm, seg = tables_np(tab)
    check_canary(cache, seg)
    err = full_check(w, tab, cache, out, k, v, q, w.n, tk, tv)
    assert err <= P.ATTN_TOL


def test_gqa_ratio_no_alloc_matches_workspace_call():
    """Six query heads per KV head (groups of 4 and 2) through the
    no-allocation entry point: the same outputs as the workspace call."""
    w = configs.Workload(name="gqa-6to1-noalloc", seed=577, B=2, Hq=12, Hkv=2, d=128, T=1024, C=128,
                         mix=(0.2, 0.5, 0.3), outlier_cols=2, outlier_mult=8.0)
    note(f"{w.name}")
    experts = synth.drawn_chunk_experts(w)
    tab = build_tables_from_experts(experts, w.C, freeze=True)
    k, v = synth.kv(w, DEV)
    q = synth.query(w, DEV)
    cache, out, tk, tv = run_quant_attn(w, tab, k, v, q, w.n, tail=11)
    out2 = torch.empty_like(out)
    mkv.mixed_kv_decode_attention_noalloc(q, cache, out2, tail_k=tk, tail_v=tv)
    torch.cuda.synchronize()
    scale = out.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    rel = ((out - out2).abs() / scale).max().item()
    note(f"  no-alloc against workspace call: max rel difference {rel:.2e}")
    assert rel <= P.RUN_TO_RUN
