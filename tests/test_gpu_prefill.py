"""GPU parity of chunked-prefill attention over the mixed cache: every
compared query row against the oracle's causal attention over the GPU's own
packed chunks (dequantized) and the chunk's exact fp16 keys and values."""
import numpy as np
import pytest
import torch

from chunk_mixed_precision_amd import configs, mkv, synth
from oracle import mkv_oracle as orc
from tests import parity as P
from tests.test_gpu_parity import build_tables_from_experts, caps_of

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(msg, flush=True)


def run_prefill(w, experts, Pn, seed_q=0):
    tab = build_tables_from_experts(experts, w.C, freeze=True)
    k, v = synth.kv(w, DEV)
    cache = mkv.PackedCache(w.B, w.Hkv, w.d, w.C, caps_of(tab), tab.seg_count, DEV)
    mkv.quantize_pack_kv(k, v, tab, cache)
    g = torch.Generator(device=DEV)
    g.manual_seed(w.seed * 100 + 55 + seed_q)
    q = torch.randn((w.B, w.Hq, Pn, w.d), generator=g, device=DEV).to(torch.float16)
    kn = torch.randn((w.B, w.Hkv, Pn, w.d), generator=g, device=DEV).to(torch.float16)
    vn = torch.randn((w.B, w.Hkv, Pn, w.d), generator=g, device=DEV).to(torch.float16)
    out = mkv.mixed_kv_prefill_attention(q, cache, kn, vn)
    torch.cuda.synchronize()
    return tab, cache, q, kn, vn, out


def check_prefill(w, tab, cache, q, kn, vn, out, heads, rows):
    """Max over the listed (b, hq) and query rows of |o - ref|_inf / |ref|_inf."""
    bits, rank = P.to_np(tab.chunk_bits), P.to_np(tab.chunk_rank)
    pools = P.pools_np(cache)
    q_np, kn_np, vn_np, o_np = P.to_np(q), P.to_np(kn), P.to_np(vn), P.to_np(out)
    g = w.Hq // w.Hkv
    worst = 0.0
    memo = {}
    for (b, hq) in heads:
        h = hq // g
        if (b, h) not in memo:
            memo[(b, h)] = P.dequant_sequence_head(cache, pools, bits[b], rank[b], w.n, b, h)
        kh, vh = memo[(b, h)]
        for i in rows:
            k_all = np.concatenate([kh, kn_np[b, h, :i + 1].astype(np.float64)])
            v_all = np.concatenate([vh, vn_np[b, h, :i + 1].astype(np.float64)])
            ref = orc.attention(q_np[b, hq, i].astype(np.float64), k_all, v_all)
            err = np.max(np.abs(o_np[b, hq, i] - ref)) / max(np.max(np.abs(ref)), 1e-30)
            worst = max(worst, err)
            assert err <= P.ATTN_TOL, f"prefill rel err {err:.3e} at (b={b}, hq={hq}, i={i})"
    return worst


@pytest.mark.parametrize("d,C,Hq,Hkv,B,T,Pn", [
    (128, 128, 4, 4, 2, 1024, 128),    # MHA, one query tile
    (128, 256, 8, 2, 1, 2048, 300),    # GQA 4:1, three query tiles, ragged
    (64, 64, 4, 2, 2, 512, 100),       # head_dim 64, GQA 2:1, ragged
])
def test_prefill_attention_mixed_cache(d, C, Hq, Hkv, B, T, Pn):
    w = configs.Workload(name=f"prefill-d{d}-C{C}-{Hq}x{Hkv}", seed=71 + d + C, B=B, Hq=Hq, Hkv=Hkv, d=d, T=T, C=C,
                         mix=(0.2, 0.4, 0.4), outlier_cols=3, outlier_mult=8.0)
    note(f"prefill {w.name}, P={Pn}")
    experts = synth.drawn_chunk_experts(w)
    tab, cache, q, kn, vn, out = run_prefill(w, experts, Pn)
    heads = [(b, hq) for b in range(B) for hq in range(Hq)]
    err = check_prefill(w, tab, cache, q, kn, vn, out, heads, range(Pn))
    note(f"  max rel err {err:.2e} over {len(heads) * Pn} query rows")


def test_prefill_attention_without_cache():
    """A sequence with no cached chunks: causal attention over the chunk alone
    (query 0 returns its own value)."""
    w = configs.Workload(name="prefill-empty", seed=77, B=2, Hq=2, Hkv=2, d=128, T=256, C=128)
    experts = torch.tensor([[1, 2], [0, 1]], dtype=torch.uint8)
    tab = build_tables_from_experts(experts, w.C, freeze=False)
    seg0 = tab.seg_count.clone()
    tab.seg_count[0].zero_()                      # sequence 0: empty cache
    k, v = synth.kv(w, DEV)
    cache = mkv.PackedCache(w.B, w.Hkv, w.d, w.C, [int(x) for x in seg0.max(0).values.tolist()], tab.seg_count, DEV)
    mkv.quantize_pack_kv(k, v, tab, cache)
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    Pn = 37
    q = torch.randn((w.B, w.Hq, Pn, w.d), generator=g, device=DEV).to(torch.float16)
    kn = torch.randn((w.B, w.Hkv, Pn, w.d), generator=g, device=DEV).to(torch.float16)
    vn = torch.randn((w.B, w.Hkv, Pn, w.d), generator=g, device=DEV).to(torch.float16)
    out = mkv.mixed_kv_prefill_attention(q, cache, kn, vn)
    torch.cuda.synchronize()
    o = P.to_np(out)
    assert np.allclose(o[0, :, 0], P.to_np(vn)[0, :, 0].astype(np.float32), rtol=0, atol=1e-6)
    q_np, kn_np, vn_np = P.to_np(q), P.to_np(kn), P.to_np(vn)
    for hq in range(w.Hq):
        ref = orc.prefill_attention(q_np[0, hq].astype(np.float64), np.zeros((0, w.d)), np.zeros((0, w.d)),
                                    kn_np[0, hq].astype(np.float64), vn_np[0, hq].astype(np.float64))
        err = np.max(np.abs(o[0, hq] - ref), axis=1) / np.max(np.abs(ref), axis=1)
        assert err.max() <= P.ATTN_TOL


def test_prefill_attention_full_size_llama2_7b_32k_sampled():
    """The llama2-7b 32k layer (32 heads, 32768 cached tokens at the 3/90/7
    mix) with a 256-token chunk; sampled heads and query rows."""
    w = configs.Workload(name="prefill-7b-32k", seed=79, B=1, Hq=32, Hkv=32, d=128, T=32768, C=256,
                         mix=(0.03, 0.90, 0.07), outlier_cols=82, outlier_mult=8.0)
    note(f"prefill {w.name}, P=256")
    experts = synth.drawn_chunk_experts(w)
    tab, cache, q, kn, vn, out = run_prefill(w, experts, 256)
    rng = np.random.default_rng(3)
    heads = [(0, int(hq)) for hq in rng.choice(32, 4, replace=False)]
    rows = [0, 1, 31, 32, 127, 128, 200, 255]
    err = check_prefill(w, tab, cache, q, kn, vn, out, heads, rows)
    note(f"  max rel err {err:.2e} over {len(heads) * len(rows)} sampled query rows")


def test_prefill_attention_full_size_llama2_13b_sampled():
    """The llama2-13b shape (16 sequences, 40 heads, 8192 cached tokens at
    chunk 128) with a 128-token chunk: the 128-query workgroups whose two
    halves take alternate group blocks; sampled sequences, heads and rows."""
    w = configs.Workload(name="prefill-13b-8k", seed=83, B=16, Hq=40, Hkv=40, d=128, T=8192, C=128,
                         mix=(0.05, 0.75, 0.20), outlier_cols=100, outlier_mult=8.0)
    note(f"prefill {w.name}, P=128")
    experts = synth.drawn_chunk_experts(w)
    tab, cache, q, kn, vn, out = run_prefill(w, experts, 128)
    rng = np.random.default_rng(4)
    heads = [(int(b), int(hq)) for b, hq in zip(rng.choice(16, 6), rng.choice(40, 6))] + [(15, 39)]
    rows = [0, 1, 31, 32, 63, 64, 100, 127]
    err = check_prefill(w, tab, cache, q, kn, vn, out, heads, rows)
    note(f"  max rel err {err:.2e} over {len(heads) * len(rows)} sampled query rows")


def test_prefill_attention_is_deterministic():
    """The prefill's splits and block order are fixed by the shapes (no work
    tickets), so two calls on the same inputs agree bit for bit, in both
    workgroup modes (P <= 128 and P > 128)."""
    w = configs.Workload(name="prefill-repeat", seed=91, B=2, Hq=8, Hkv=2, d=128, T=2048, C=128,
                         mix=(0.2, 0.4, 0.4), outlier_cols=3, outlier_mult=8.0)
    experts = synth.drawn_chunk_experts(w)
    for Pn in (100, 200):
        tab, cache, q, kn, vn, out = run_prefill(w, experts, Pn)
        again = mkv.mixed_kv_prefill_attention(q, cache, kn, vn)
        torch.cuda.synchronize()
        assert torch.equal(out, again), f"prefill differs between calls at P={Pn}"
        note(f"  P={Pn}: bit-identical over {out.numel()} outputs")
