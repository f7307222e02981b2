"""GPU parity at the workloads' full sizes, in the launch configuration the
bench uses.  Everything the oracle can afford is compared in full (votes,
reorder tables); the rest on seeded samples (router rows, packed chunks,
attention heads)."""
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


def tables_np(tab):
    return (P.to_np(tab.chunk_bits), P.to_np(tab.chunk_rank), P.to_np(tab.perm), P.to_np(tab.seg_count))


def sample_chunks(rng, bits, B, Hkv, n, per_bits=6, chunk_offset=0):
    """A few chunks of every bitwidth present, on random sequences and heads."""
    out = []
    for want in (16, 4, 2):
        idx = np.argwhere(bits[:, chunk_offset:chunk_offset + n] == want)
        if len(idx) == 0:
            continue
        pick = idx[rng.choice(len(idx), size=min(per_bits, len(idx)), replace=False)]
        for b, c in pick:
            out.append((int(b), int(rng.integers(Hkv)), int(c)))
    return out


def routed_single_layer(w, n_rows=2048, n_heads=3):
    rng = np.random.default_rng(w.seed)
    note(f"{w.name}: route {w.B}x{w.T} tokens, D={w.D}, I={w.I}")
    x, w12, w3, b3 = synth.router_inputs(w)
    tab = mkv.RouteTables(w.B, w.n, DEV)
    logits = torch.empty((w.B, w.T, 3), dtype=torch.float32, device=DEV)
    te = torch.empty((w.B, w.T), dtype=torch.uint8, device=DEV)
    mkv.route_chunks(tab, w.C, x=x.to(DEV), w12=w12.to(DEV), w3=w3.to(DEV), b3=b3.to(DEV), logits=logits,
                     token_expert=te)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(w.B * w.T, size=n_rows, replace=False))
    rep = P.check_router(x.view(-1, w.D), w12, w3, b3, w.I, P.to_np(logits).reshape(-1, 3),
                         P.to_np(te).reshape(-1), rows=rows)
    note(f"  router on {n_rows} sampled tokens: {rep}")
    bits, rank, perm, seg = tables_np(tab)
    P.check_vote_and_reorder(P.to_np(te), w.C, bits, rank, perm, seg)
    frac = seg.sum(0) / seg.sum()
    note(f"  chunk mix {seg.sum(0).tolist()} -> {np.round(frac, 4).tolist()} (target {list(w.mix)})")
    assert np.max(np.abs(frac - np.asarray(w.mix))) <= 0.03
    del x
    k, v = synth.kv(w, DEV)
    q = synth.query(w, DEV)
    caps = [int(seg[:, kk].max()) for kk in range(3)]
    cache = mkv.PackedCache(w.B, w.Hkv, w.d, w.C, caps, tab.seg_count, DEV)
    mkv.quantize_pack_kv(k, v, tab, cache)
    out = mkv.mixed_kv_decode_attention(q, cache)
    torch.cuda.synchronize()
    pools = P.pools_np(cache)
    triples = sample_chunks(rng, bits, w.B, w.Hkv, w.n)
    n = P.check_quantize(cache, pools, P.to_np(k), P.to_np(v), bits, rank, triples)
    pairs = [(0, int(h)) for h in rng.choice(w.Hq, size=n_heads, replace=False)]
    err = P.check_attention(cache, pools, bits, rank, w.n, P.to_np(q), P.to_np(out), pairs)
    note(f"  quantize: {n} sampled chunks exact; attention rel err {err:.2e} on heads {pairs}")


def test_llama2_7b_32k_layer():
    routed_single_layer(configs.LLAMA2_7B_32K)


def test_llama2_7b_128k_layer():
    routed_single_layer(configs.LLAMA2_7B_128K, n_heads=2)


class _SequenceView:
    """One sequence of a packed cache, addressed as a cache of B = 1: the
    pools are laid out [B][Hkv][cap][...], so sequence b's part of each pool
    is one contiguous run of bytes."""

    def __init__(self, cache, b):
        self.B, self.Hkv, self.d, self.C, self.caps = 1, cache.Hkv, cache.d, cache.C, cache.caps
        self.pools_np = []
        for k, bits in enumerate(orc.EXPERT_BITS):
            per = mkv.pool_bytes(bits, 1, cache.Hkv, cache.caps[k], cache.d, cache.C)
            self.pools_np.append(P.to_np(cache.pools[k][b * per:(b + 1) * per]))


@pytest.mark.timeout(900)
def test_llama2_13b_40_layers_sampled():
    """One routing table (drawn mix, routing sharing) for 40 layers.  Every
    query head of sequences 0, 7 and 15 in layers 0, 19 and 39, plus every
    head of 5 seeded random (layer, sequence) pairs, is compared with the
    oracle over all 8192 cached tokens; sampled chunks of every bitwidth are
    compared bit for bit in each layer built."""
    w = configs.LLAMA2_13B_40L
    rng = np.random.default_rng(w.seed)
    experts = synth.drawn_chunk_experts(w)
    tab = mkv.RouteTables(w.B, w.n, DEV)
    mkv.route_chunks(tab, w.C, logits=synth.one_hot_logits(experts, w.C).to(DEV), logits_in=True)
    torch.cuda.synchronize()
    bits, rank, perm, seg = tables_np(tab)
    P.check_reorder_only(bits, rank, perm, seg, w.n)
    avg = float((seg * np.array([16, 4, 2])).sum() / seg.sum())
    note(f"{w.name}: mix {seg.sum(0).tolist()}, {avg:.3f} bits per value")
    caps = [int(seg[:, kk].max()) for kk in range(3)]
    pairs = {layer: [0, 7, 15] for layer in (0, 19, 39)}
    for _ in range(5):
        layer, b = int(rng.integers(w.layers)), int(rng.integers(w.B))
        pairs.setdefault(layer, [])
        if b not in pairs[layer]:
            pairs[layer].append(b)
    note(f"  (layer, sequences) checked: {sorted(pairs.items())}")
    for layer in sorted(pairs):
        k, v = synth.kv(w, DEV, layer=layer)
        q = synth.query(w, DEV, layer=layer)
        cache = mkv.PackedCache(w.B, w.Hkv, w.d, w.C, caps, tab.seg_count, DEV)
        mkv.quantize_pack_kv(k, v, tab, cache)
        out = mkv.mixed_kv_decode_attention(q, cache)
        torch.cuda.synchronize()
        q_np, out_np = P.to_np(q), P.to_np(out)
        n = 0
        worst = 0.0
        for b in pairs[layer]:
            view = _SequenceView(cache, b)
            triples = sample_chunks(rng, bits[b:b + 1], 1, w.Hkv, w.n, per_bits=2)
            n += P.check_quantize(view, view.pools_np, P.to_np(k[b:b + 1]), P.to_np(v[b:b + 1]),
                                  bits[b:b + 1], rank[b:b + 1], triples)
            err = P.check_attention(view, view.pools_np, bits[b:b + 1], rank[b:b + 1], w.n, q_np[b:b + 1],
                                    out_np[b:b + 1], [(0, hq) for hq in range(w.Hq)])
            worst = max(worst, err)
        note(f"  layer {layer}: sequences {pairs[layer]}, all {w.Hq} heads each: attention rel err {worst:.2e}; "
             f"{n} chunks exact")
        del k, v, cache, out


def test_llama3_8b_gqa_append_step():
    """Prefill tables (drawn mix) for 32 chunks per sequence, then one decode
    step: route the 64 appended 256-token chunks (router mode, append),
    quantize them into their segments, attend over 8448 tokens (GQA 4:1)."""
    w = configs.LLAMA3_8B_GQA
    rng = np.random.default_rng(w.seed)
    experts = synth.drawn_chunk_experts(w)
    experts[:, 0] = 0
    tab = mkv.RouteTables(w.B, w.n_total, DEV)
    mkv.route_chunks(tab, w.C, logits=synth.one_hot_logits(experts, w.C).to(DEV), logits_in=True)
    torch.cuda.synchronize()
    prior = orc.expert_of_bits(P.to_np(tab.chunk_bits)[:, :w.n])
    x, w12, w3, b3 = synth.router_inputs(w, tokens_per_seq=w.C, chunk_offset=w.n)
    logits = torch.empty((w.B, w.C, 3), dtype=torch.float32, device=DEV)
    te = torch.empty((w.B, w.C), dtype=torch.uint8, device=DEV)
    mkv.route_chunks(tab, w.C, x=x.to(DEV), w12=w12.to(DEV), w3=w3.to(DEV), b3=b3.to(DEV), logits=logits,
                     token_expert=te, append=True, chunk_offset=w.n)
    torch.cuda.synchronize()
    rep = P.check_router(x.view(-1, w.D), w12, w3, b3, w.I, P.to_np(logits).reshape(-1, 3),
                         P.to_np(te).reshape(-1))
    note(f"{w.name}: router on all {w.B * w.C} appended tokens: {rep}")
    bits, rank, perm, seg = tables_np(tab)
    P.check_vote_and_reorder(P.to_np(te), w.C, bits, rank, perm, seg, chunk_offset=w.n, prior_experts=prior)
    caps = [int(seg[:, kk].max()) for kk in range(3)]
    cache = mkv.PackedCache(w.B, w.Hkv, w.d, w.C, caps, tab.seg_count, DEV)
    k, v = synth.kv(w, DEV)
    mkv.quantize_pack_kv(k, v, tab, cache)
    ka, va = synth.kv(w, DEV, tokens=w.C, token_offset_stream=1)
    mkv.quantize_pack_kv(ka, va, tab, cache, chunk_offset=w.n)
    q = synth.query(w, DEV)
    out = mkv.mixed_kv_decode_attention(q, cache)
    torch.cuda.synchronize()
    pools = P.pools_np(cache)
    n = P.check_quantize(cache, pools, P.to_np(k), P.to_np(v), bits, rank,
                         sample_chunks(rng, bits, w.B, w.Hkv, w.n, per_bits=4))
    app = [(int(b), int(rng.integers(w.Hkv)), 0) for b in rng.choice(w.B, size=8, replace=False)]
    n += P.check_quantize(cache, pools, P.to_np(ka), P.to_np(va), bits, rank, app, chunk_offset=w.n)
    pairs = [(int(b), int(hq)) for b in rng.choice(w.B, size=3, replace=False)
             for hq in rng.choice(w.Hq, size=4, replace=False)]
    err = P.check_attention(cache, pools, bits, rank, w.n_total, P.to_np(q), P.to_np(out), pairs)
    note(f"  quantize: {n} chunks exact (incl. appended); attention rel err {err:.2e} on {len(pairs)} heads")
