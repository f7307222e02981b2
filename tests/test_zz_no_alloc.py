"""The no-allocation decode attention (mkv_mixed_kv_decode_attention_noalloc,
for callers that cannot allocate device memory) against the workspace
entry point (mkv_mixed_kv_decode_attention) through the C ABI: two calls in
a row on one GPU, the second on a smaller problem, each compared with the
workspace call on the same inputs and with the oracle."""
import numpy as np
import pytest
import torch

from chunk_mixed_precision_amd import configs, mkv, synth
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"

RUN_TO_RUN = P.RUN_TO_RUN      # calls differ only in the fp32 summation order


def _problem(seed, B, Hq, Hkv, T, C, mix, tail):
    w = configs.Workload(name=f"noalloc-{seed}", seed=seed, B=B, Hq=Hq, Hkv=Hkv, d=128, T=T, C=C, mix=mix,
                         outlier_cols=3, outlier_mult=8.0)
    experts = synth.drawn_chunk_experts(w)
    tab = mkv.RouteTables(w.B, w.n, DEV)
    mkv.route_chunks(tab, w.C, logits=synth.one_hot_logits(experts, w.C).to(DEV), logits_in=True)
    torch.cuda.synchronize()
    seg = tab.seg_count.cpu().numpy()
    caps = [int(seg[:, k].max()) for k in range(3)]
    cache = mkv.PackedCache(w.B, w.Hkv, w.d, w.C, caps, tab.seg_count, DEV)
    k, v = synth.kv(w, DEV)
    mkv.quantize_pack_kv(k, v, tab, cache)
    q = synth.query(w, DEV)
    g = torch.Generator(device=DEV).manual_seed(seed)
    tk = torch.randn((B, Hkv, C, 128), generator=g, device=DEV).to(torch.float16)
    tv = torch.randn((B, Hkv, C, 128), generator=g, device=DEV).to(torch.float16)
    return w, tab, cache, q, tk, tv, tail


def _compare(w, tab, cache, q, tk, tv, tail):
    ref = mkv.mixed_kv_decode_attention(q, cache, tail_k=tk, tail_v=tv, tail_len=tail)
    out = torch.full_like(ref, float("nan"))
    mkv.mixed_kv_decode_attention_noalloc(q, cache, out, tail_k=tk, tail_v=tv, tail_len=tail)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    scale = ref.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    rel = ((out - ref).abs() / scale).max().item()
    bits, rank = P.to_np(tab.chunk_bits), P.to_np(tab.chunk_rank)
    pools = P.pools_np(cache)
    pairs = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    err = P.check_attention(cache, pools, bits, rank, w.n, P.to_np(q), P.to_np(out), pairs,
                            P.to_np(tk)[:, :, :tail], P.to_np(tv)[:, :, :tail])
    print(f"  {w.name}: no-alloc vs workspace call max rel diff {rel:.2e}; vs oracle {err:.2e}", flush=True)
    assert rel <= RUN_TO_RUN
    return out


def test_noalloc_matches_workspace_call_twice_smaller_second():
    big = _problem(301, B=3, Hq=8, Hkv=2, T=2048, C=128, mix=(0.2, 0.5, 0.3), tail=37)
    small = _problem(302, B=1, Hq=4, Hkv=4, T=512, C=128, mix=(0.3, 0.3, 0.4), tail=5)
    first = _compare(*big)
    _compare(*small)
    # the first problem again after the smaller one: nothing of the earlier
    # calls' scratch contents leaks into the result
    again = _compare(*big)
    scale = first.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    assert ((again - first).abs() / scale).max().item() <= RUN_TO_RUN
