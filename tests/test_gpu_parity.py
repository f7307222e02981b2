"""GPU parity: the HIP path (through the C ABI) against the CPU oracle,
stage by stage, on seeded synthetic inputs.  See tests/parity.py for the bars."""
import numpy as np
import pytest
import torch

from chunk_mixed_precision_amd import configs, mkv, synth
from oracle import mkv_oracle as orc
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(msg, flush=True)


def build_tables_from_experts(experts: torch.Tensor, C: int, n_max: int = None, freeze=True):
    """Drive mkv_route_chunks in logits-in mode with one-hot logits so every
    token of chunk c votes for experts[b, c]."""
    B, n = experts.shape
    tab = mkv.RouteTables(B, n_max or n, DEV)
    logits = synth.one_hot_logits(experts, C).to(DEV)
    mkv.route_chunks(tab, C, logits=logits, logits_in=True, freeze_first=freeze)
    return tab


def caps_of(tab: mkv.RouteTables, extra=0):
    seg = tab.seg_count.cpu().numpy()
    return [int(seg[:, k].max()) + extra for k in range(3)]


def tables_np(tab):
    return (P.to_np(tab.chunk_bits), P.to_np(tab.chunk_rank), P.to_np(tab.perm), P.to_np(tab.seg_count))


def run_quant_attn(w, tab, k, v, q, n_total, tail=0, canary=True, caps=None):
    caps = caps or caps_of(tab)
    cache = mkv.PackedCache(w.B, w.Hkv, w.d, w.C, caps, tab.seg_count, DEV)
    if canary:
        for p in cache.pools:
            p.fill_(0xA5)
    mkv.quantize_pack_kv(k, v, tab, cache)
    tk = tv = None
    if tail:
        g = torch.Generator(device=DEV)
        g.manual_seed(w.seed * 100 + 77)
        tk = torch.randn((w.B, w.Hkv, tail, w.d), generator=g, device=DEV).to(torch.float16)
        tv = torch.randn((w.B, w.Hkv, tail, w.d), generator=g, device=DEV).to(torch.float16)
    out = mkv.mixed_kv_decode_attention(q, cache, tail_k=tk, tail_v=tv)
    torch.cuda.synchronize()
    return cache, out, tk, tv


def check_canary(cache, seg):
    """Slots beyond each sequence's segment must still hold the fill pattern."""
    for kidx, bits in enumerate(orc.EXPERT_BITS):
        cap = cache.caps[kidx]
        if cap == 0:
            continue
        pool = P.to_np(cache.pools[kidx])
        cb = mkv.pool_bytes(bits, 1, 1, 1, cache.d, cache.C)
        body = pool[:cache.B * cache.Hkv * cap * cb].reshape(cache.B, cache.Hkv, cap, cb)
        for b in range(cache.B):
            used = int(seg[b, kidx])
            assert np.all(body[b, :, used:] == 0xA5), f"write outside segment (b={b}, bits={bits})"
        assert np.all(pool[cache.B * cache.Hkv * cap * cb:] == 0xA5)


def full_check(w, tab, cache, out, k, v, q, n_total, tk=None, tv=None, sample_chunks=None, sample_pairs=None,
               rng=None):
    bits, rank, perm, seg = tables_np(tab)
    pools = P.pools_np(cache)
    k_np, v_np, q_np = P.to_np(k), P.to_np(v), P.to_np(q)
    if sample_chunks is None:
        triples = [(b, h, c) for b in range(w.B) for h in range(w.Hkv) for c in range(n_total)]
    else:
        triples = sample_chunks
    n = P.check_quantize(cache, pools, k_np, v_np, bits, rank, triples)
    pairs = sample_pairs or [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    err = P.check_attention(cache, pools, bits, rank, n_total, q_np, P.to_np(out), pairs,
                            None if tk is None else P.to_np(tk), None if tv is None else P.to_np(tv))
    note(f"  quantize: {n} chunks exact; attention max rel err {err:.2e} over {len(pairs)} heads")
    return err


# ------------------------------------------------------------------ small, complete checks
def test_forced_pattern_d64_with_tail():
    """All three bitwidths in one sequence, every chunk and head compared,
    plus a 37-token fp16 tail (head_dim 64, chunk 128)."""
    w = configs.TINY
    note(f"forced pattern {w.name}")
    experts = orc.expert_of_bits(np.array([[16, 4, 2, 4, 2, 2, 4, 16]], np.uint8))
    tab = build_tables_from_experts(torch.from_numpy(experts), w.C)
    bits, rank, perm, seg = tables_np(tab)
    P.check_reorder_only(bits, rank, perm, seg, w.n)
    k, v = synth.kv(w, DEV)
    q = synth.query(w, DEV)
    cache, out, tk, tv = run_quant_attn(w, tab, k, v, q, w.n, tail=37)
    check_canary(cache, seg)
    full_check(w, tab, cache, out, k, v, q, w.n, tk, tv)


def test_route_tiny_router_mode():
    """Router on bf16 MFMA: logits, argmax flips only at near ties, vote,
    freezing and reorder exact."""
    w = configs.TINY
    note(f"router {w.name}")
    x, w12, w3, b3 = synth.router_inputs(w)
    tab = mkv.RouteTables(w.B, w.n, DEV)
    logits = torch.empty((w.B, w.T, 3), dtype=torch.float32, device=DEV)
    te = torch.empty((w.B, w.T), dtype=torch.uint8, device=DEV)
    mkv.route_chunks(tab, w.C, x=x.to(DEV), w12=w12.to(DEV), w3=w3.to(DEV), b3=b3.to(DEV),
                     logits=logits, token_expert=te)
    torch.cuda.synchronize()
    rep = P.check_router(x.view(-1, w.D), w12, w3, b3, w.I, P.to_np(logits).reshape(-1, 3),
                         P.to_np(te).reshape(-1))
    note(f"  router: {rep}")
    assert rep["max_abs_logit_err"] < 1e-4
    bits, rank, perm, seg = tables_np(tab)
    P.check_vote_and_reorder(P.to_np(te), w.C, bits, rank, perm, seg)
    assert bits[0, 0] == 16


@pytest.mark.parametrize("d,C,Hq,Hkv,B,T", [
    (128, 256, 4, 4, 2, 4096),    # MHA, chunk 256
    (128, 128, 8, 2, 3, 2048),    # GQA 4:1
    (128, 32, 4, 2, 2, 1024),     # GQA 2:1, one group per chunk
    (64, 64, 4, 4, 2, 1024),      # head_dim 64
    (64, 128, 8, 2, 1, 2048),     # head_dim 64, GQA 4:1
])
def test_mixed_chunks_exhaustive(d, C, Hq, Hkv, B, T):
    w = configs.Workload(name=f"mixed-d{d}-C{C}-{Hq}x{Hkv}", seed=11 + d + C, B=B, Hq=Hq, Hkv=Hkv, d=d, T=T, C=C,
                         mix=(0.2, 0.4, 0.4), outlier_cols=3, outlier_mult=8.0)
    note(f"mixed {w.name}")
    experts = synth.drawn_chunk_experts(w)
    tab = build_tables_from_experts(experts, C, freeze=True)
    k, v = synth.kv(w, DEV)
    q = synth.query(w, DEV)
    cache, out, tk, tv = run_quant_attn(w, tab, k, v, q, w.n, tail=(5 if d == 128 else 0))
    bits, rank, perm, seg = tables_np(tab)
    v_ref = orc.chunk_vote(orc.expert_of_bits(np.repeat(synth.bits_tensor(experts).numpy(), C, axis=1)), C,
                           freeze_first=True)
    assert np.array_equal(orc.expert_of_bits(bits[:, :w.n]), v_ref)
    P.check_reorder_only(bits, rank, perm, seg, w.n)
    check_canary(cache, seg)
    full_check(w, tab, cache, out, k, v, q, w.n, tk, tv)


@pytest.mark.parametrize("B,Hq,Hkv,d", [(130, 2, 2, 64), (97, 4, 2, 128), (71, 8, 2, 128)])
def test_more_than_64_sequences(B, Hq, Hkv, d):
    """Batches past one wavefront of sequences: the attention split then
    scans the sequences 64 at a time to find each range's first stream, and
    the combine finds each stream's offset the same way."""
    C, T = 128, 512
    w = configs.Workload(name=f"wide-B{B}-{Hq}x{Hkv}-d{d}", seed=5 + B, B=B, Hq=Hq, Hkv=Hkv, d=d, T=T, C=C,
                         mix=(0.3, 0.4, 0.3), outlier_cols=2, outlier_mult=8.0)
    note(f"wide batch {w.name}")
    experts = synth.drawn_chunk_experts(w)
    tab = build_tables_from_experts(experts, C, freeze=True)
    k, v = synth.kv(w, DEV)
    q = synth.query(w, DEV)
    cache, out, tk, tv = run_quant_attn(w, tab, k, v, q, w.n, tail=3)
    bits, rank, perm, seg = tables_np(tab)
    P.check_reorder_only(bits, rank, perm, seg, w.n)
    check_canary(cache, seg)
    full_check(w, tab, cache, out, k, v, q, w.n, tk, tv)


def test_without_routing_sharing_per_layer_tables():
    """The ablation without routing sharing (MoQAE, Key designs: RS off):
    every block routes its own hidden states with its own router, so every
    layer has its own tables, pools and capacities.  Each layer's route,
    vote, reorder, quantize and attention stay at parity, and the layers'
    tables differ (the ablation changes the routing)."""
    w = configs.Workload(name="wo-rs", seed=91, B=2, Hq=4, Hkv=4, d=128, T=2048, C=128, D=256, I=128,
                         layers=3, x_chunk_share=1.0, router_std=0.05, b3=(0.0, 0.02, 0.0))
    note(f"without routing sharing {w.name}")
    all_bits = []
    for layer in range(w.layers):
        x, w12, w3, b3 = synth.router_inputs(w, layer=layer)
        tab = mkv.RouteTables(w.B, w.n, DEV)
        logits = torch.empty((w.B, w.T, 3), dtype=torch.float32, device=DEV)
        te = torch.empty((w.B, w.T), dtype=torch.uint8, device=DEV)
        mkv.route_chunks(tab, w.C, x=x.to(DEV), w12=w12.to(DEV), w3=w3.to(DEV), b3=b3.to(DEV),
                         logits=logits, token_expert=te)
        torch.cuda.synchronize()
        rep = P.check_router(x.view(-1, w.D), w12, w3, b3, w.I, P.to_np(logits).reshape(-1, 3),
                             P.to_np(te).reshape(-1))
        note(f"  layer {layer} router: {rep}")
        assert rep["max_abs_logit_err"] < 1e-4
        bits, rank, perm, seg = tables_np(tab)
        P.check_vote_and_reorder(P.to_np(te), w.C, bits, rank, perm, seg)
        note(f"  layer {layer} segment counts {seg.tolist()}")
        k, v = synth.kv(w, DEV, layer=layer)
        q = synth.query(w, DEV, layer=layer)
        cache, out, _, _ = run_quant_attn(w, tab, k, v, q, w.n)
        check_canary(cache, seg)
        full_check(w, tab, cache, out, k, v, q, w.n)
        all_bits.append(bits)
    assert any(not np.array_equal(all_bits[0], b) for b in all_bits[1:])


def test_constant_groups_and_signed_zeros():
    """Groups whose values are all equal (scale 0), -0/+0 extremes, and a
    group made of two values only."""
    w = configs.Workload(name="degenerate", seed=21, B=1, Hq=2, Hkv=2, d=128, T=512, C=128)
    k = torch.zeros((1, 2, 512, 128), dtype=torch.float16)
    v = torch.zeros((1, 2, 512, 128), dtype=torch.float16)
    k[0, 0, :128] = 1.25                        # constant keys
    v[0, 0, :128] = -0.0                        # all -0 values
    k[0, 1, 128:256] = torch.where(torch.arange(128)[:, None] % 2 == 0, 3.0, -0.0).to(torch.float16)
    v[0, 1, 128:256, ::2] = 7.0
    g = torch.Generator().manual_seed(5)
    k[0, :, 256:] = torch.randn((2, 256, 128), generator=g).to(torch.float16)
    v[0, :, 256:] = torch.randn((2, 256, 128), generator=g).to(torch.float16)
    v[0, :, 300:332, 0:32] = 2.5               # constant value groups
    experts = torch.tensor([[1, 2, 1, 2]], dtype=torch.uint8)
    tab = build_tables_from_experts(experts, w.C, freeze=False)
    q = synth.query(w, DEV)
    k, v = k.to(DEV), v.to(DEV)
    cache, out, _, _ = run_quant_attn(w, tab, k, v, q, w.n)
    full_check(w, tab, cache, out, k, v, q, w.n)


def test_tail_only_and_empty_sequences():
    """A sequence with no cached chunks: attention over the tail alone, and
    zeros when there is no tail either."""
    w = configs.Workload(name="empty", seed=31, B=2, Hq=4, Hkv=2, d=128, T=256, C=128)
    tab = mkv.RouteTables(w.B, 4, DEV)          # all seg_count = 0
    cache = mkv.PackedCache(w.B, w.Hkv, w.d, w.C, [1, 1, 1], tab.seg_count, DEV)
    q = synth.query(w, DEV)
    out0 = mkv.mixed_kv_decode_attention(q, cache)
    torch.cuda.synchronize()
    assert torch.all(out0 == 0)
    g = torch.Generator(device=DEV).manual_seed(3)
    tk = torch.randn((w.B, w.Hkv, 17, w.d), generator=g, device=DEV).to(torch.float16)
    tv = torch.randn((w.B, w.Hkv, 17, w.d), generator=g, device=DEV).to(torch.float16)
    out = mkv.mixed_kv_decode_attention(q, cache, tail_k=tk, tail_v=tv)
    torch.cuda.synchronize()
    qn, kn, vn, on = P.to_np(q), P.to_np(tk), P.to_np(tv), P.to_np(out)
    for b in range(w.B):
        for hq in range(w.Hq):
            ref = orc.attention(qn[b, hq], kn[b, hq // 2].astype(np.float64), vn[b, hq // 2].astype(np.float64))
            assert np.max(np.abs(on[b, hq] - ref)) / np.max(np.abs(ref)) < P.ATTN_TOL


def test_all_fp16_equals_sdpa():
    """Every chunk FP16: the result is plain softmax attention on the fp16
    cache (torch SDPA in float64 on the CPU)."""
    w = configs.Workload(name="allfp16", seed=41, B=2, Hq=4, Hkv=4, d=128, T=1024, C=256)
    experts = torch.zeros((w.B, w.n), dtype=torch.uint8)
    tab = build_tables_from_experts(experts, w.C)
    k, v = synth.kv(w, DEV)
    q = synth.query(w, DEV)
    cache, out, _, _ = run_quant_attn(w, tab, k, v, q, w.n)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.cpu().double()[:, :, None], k.cpu().double(), v.cpu().double())[:, :, 0]
    err = ((out.cpu().double() - ref).abs().amax(-1) / ref.abs().amax(-1)).max().item()
    note(f"  all-fp16 vs SDPA rel err {err:.2e}")
    assert err < 1e-4


def test_overflow_flag_and_no_write():
    """A chunk whose rank does not fit its pool is not written; the overflow
    word is set; the chunks that fit are exact."""
    w = configs.Workload(name="overflow", seed=51, B=1, Hq=2, Hkv=2, d=128, T=512, C=128)
    experts = torch.tensor([[1, 1, 1, 2]], dtype=torch.uint8)      # three INT4 chunks, one INT2
    tab = build_tables_from_experts(experts, w.C, freeze=False)
    cache = mkv.PackedCache(w.B, w.Hkv, w.d, w.C, [0, 2, 1], tab.seg_count, DEV)
    # give the INT4 pool room for a third slot, but declare only two
    cache.pools[1] = torch.empty(mkv.pool_bytes(4, 1, 2, 3, 128, 128), dtype=torch.uint8, device=DEV)
    for p in cache.pools:
        p.fill_(0xA5)
    k, v = synth.kv(w, DEV)
    mkv.quantize_pack_kv(k, v, tab, cache)
    torch.cuda.synchronize()
    assert int(cache.overflow[0]) == 1
    used = mkv.pool_bytes(4, 1, 2, 2, 128, 128)
    assert torch.all(cache.pools[1][used:] == 0xA5)
    bits, rank, perm, seg = tables_np(tab)
    pools = P.pools_np(cache)
    n = P.check_quantize(cache, pools, P.to_np(k), P.to_np(v), bits, rank,
                         [(0, h, c) for h in range(2) for c in (0, 1, 3)])
    assert n == 6


def test_determinism():
    """Quantize/pack is bitwise deterministic.  Attention hands work units to
    wavefronts dynamically, so its fp32 summation order (and only that) can
    change between runs: outputs agree to a few fp32 rounding steps."""
    w = configs.Workload(name="determinism", seed=61, B=2, Hq=8, Hkv=2, d=128, T=2048, C=128,
                         mix=(0.1, 0.5, 0.4))
    experts = synth.drawn_chunk_experts(w)
    tab = build_tables_from_experts(experts, w.C)
    k, v = synth.kv(w, DEV)
    q = synth.query(w, DEV)
    # both caches start from the same fill, so unused slots compare equal too
    c1, o1, _, _ = run_quant_attn(w, tab, k, v, q, w.n, canary=True)
    c2, o2, _, _ = run_quant_attn(w, tab, k, v, q, w.n, canary=True)
    for a, b in zip(c1.pools, c2.pools):
        assert torch.equal(a, b)
    scale = o1.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    rel = ((o1 - o2).abs() / scale).max().item()
    note(f"attention run-to-run max rel difference {rel:.2e}")
    # two runs differ only in summation order
    assert rel <= P.RUN_TO_RUN


def test_workspace_reuse_across_calls():
    """Repeated calls on one workspace agree (to the fp32 rounding that the
    dynamic work order allows): no state leaks from one call to the next."""
    w = configs.Workload(name="reuse", seed=81, B=2, Hq=8, Hkv=4, d=128, T=2048, C=128, mix=(0.1, 0.6, 0.3))
    experts = synth.drawn_chunk_experts(w)
    tab = build_tables_from_experts(experts, w.C)
    k, v = synth.kv(w, DEV)
    q = synth.query(w, DEV)
    cache, out, _, _ = run_quant_attn(w, tab, k, v, q, w.n)
    ws = mkv.attention_workspace(w.B, w.Hq, cache, DEV)
    outs = [mkv.mixed_kv_decode_attention(q, cache, workspace=ws).clone() for _ in range(3)]
    torch.cuda.synchronize()
    scale = out.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    rels = [((o - out).abs() / scale).max().item() for o in outs]
    note(f"attention repeated-call max rel differences {[f'{r:.2e}' for r in rels]}")
    assert max(rels) <= P.RUN_TO_RUN


def test_append_mode_tables():
    """Routing a new chunk at chunk_offset keeps earlier tables, never freezes
    it, and recomputes rank/perm/seg_count over all chunks."""
    w = configs.Workload(name="append", seed=71, B=3, Hq=4, Hkv=4, d=128, T=1024, C=256, mix=(0.2, 0.5, 0.3))
    experts = synth.drawn_chunk_experts(w)                # prefill chunks 0..3
    tab = build_tables_from_experts(experts, w.C, n_max=w.n + 2)
    prior = orc.expert_of_bits(P.to_np(tab.chunk_bits)[:, :w.n])
    new = torch.tensor([[2], [0], [1]], dtype=torch.uint8)
    logits = synth.one_hot_logits(new, w.C).to(DEV)
    mkv.route_chunks(tab, w.C, logits=logits, logits_in=True, freeze_first=True, append=True, chunk_offset=w.n)
    torch.cuda.synchronize()
    bits, rank, perm, seg = tables_np(tab)
    e_new = np.repeat(new.numpy(), w.C, axis=1)
    P.check_vote_and_reorder(e_new, w.C, bits, rank, perm, seg, freeze_first=True, chunk_offset=w.n,
                             prior_experts=prior)
    # idempotent: routing the same chunk again gives the same tables
    mkv.route_chunks(tab, w.C, logits=logits, logits_in=True, freeze_first=True, append=True, chunk_offset=w.n)
    torch.cuda.synchronize()
    b2, r2, p2, s2 = tables_np(tab)
    assert np.array_equal(b2, bits) and np.array_equal(r2, rank) and np.array_equal(s2, seg)


def test_routing_freezing_off():
    w = configs.TINY
    experts = torch.full((1, w.n), 2, dtype=torch.uint8)
    tab = build_tables_from_experts(experts, w.C, freeze=False)
    assert P.to_np(tab.chunk_bits)[0, 0] == 2
    tab = build_tables_from_experts(experts, w.C, freeze=True)
    assert P.to_np(tab.chunk_bits)[0, 0] == 16
