"""GPU parity at the limits the C ABI states, each against the oracle:

  - the router on token counts that are not a multiple of its 256-token tile,
    at the smallest hidden and inner sizes it takes (D = 64, I = 128) and with
    an odd number of K steps and two inner tiles;
  - the largest chunk (C = 1024): quantization bit-exact, decode attention
    with the largest fp16 tail (4095 tokens) in a row longer than the tail,
    and chunked prefill over it;
  - the smallest chunk (C = 32, one group per chunk) under chunked prefill
    with segments of odd length, one query and a ragged query count.
"""
import numpy as np
import pytest
import torch

from chunk_mixed_precision_amd import configs, mkv, synth
from oracle import mkv_oracle as orc
from tests import parity as P
from tests.test_gpu_parity import build_tables_from_experts, caps_of, check_canary, tables_np
from tests.test_gpu_prefill import check_prefill, run_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("B,T,C,D,I", [
    (3, 160, 32, 64, 128),      # 480 tokens: one full token tile and a ragged one
    (2, 1056, 96, 192, 256),    # 2112 tokens, three K steps, two inner tiles
])
def test_router_ragged_token_tiles(B, T, C, D, I):
    w = configs.Workload(name=f"router-B{B}-T{T}-C{C}-D{D}-I{I}", seed=5 + D + I, B=B, Hq=1, Hkv=1, d=64,
                         T=T, C=C, D=D, I=I, x_chunk_share=0.5)
    note(f"router {w.name}")
    x, w12, w3, b3 = synth.router_inputs(w)
    tab = mkv.RouteTables(B, T // C, DEV)
    logits = torch.empty((B, T, 3), dtype=torch.float32, device=DEV)
    te = torch.empty((B, T), dtype=torch.uint8, device=DEV)
    mkv.route_chunks(tab, C, x=x.to(DEV), w12=w12.to(DEV), w3=w3.to(DEV), b3=b3.to(DEV),
                     logits=logits, token_expert=te)
    torch.cuda.synchronize()
    rep = P.check_router(x.view(-1, D), w12, w3, b3, I, P.to_np(logits).reshape(-1, 3), P.to_np(te).reshape(-1))
    note(f"  router: {rep}")
    assert rep["max_abs_logit_err"] <= 1e-5 * max(1.0, rep["max_abs_logit"]) + 1e-6
    bits, rank, perm, seg = tables_np(tab)
    P.check_vote_and_reorder(P.to_np(te), C, bits, rank, perm, seg)


@pytest.mark.parametrize("d,Hq,Hkv", [(128, 4, 2), (64, 2, 2)])
def test_largest_chunk_and_tail(d, Hq, Hkv):
    """C = 1024, chunks FP16 (frozen), INT2, INT4, INT2; a tail of 4095
    tokens in rows of 4100."""
    w = configs.Workload(name=f"chunk1024-d{d}-{Hq}x{Hkv}", seed=131 + d, B=1, Hq=Hq, Hkv=Hkv, d=d, T=4096, C=1024,
                         outlier_cols=2, outlier_mult=8.0)
    note(f"largest chunk {w.name}")
    experts = torch.from_numpy(orc.expert_of_bits(np.array([[16, 2, 4, 2]], np.uint8)))
    tab = build_tables_from_experts(experts, w.C)
    k, v = synth.kv(w, DEV)
    q = synth.query(w, DEV)
    cache = mkv.PackedCache(w.B, w.Hkv, w.d, w.C, caps_of(tab), tab.seg_count, DEV)
    for p in cache.pools:
        p.fill_(0xA5)
    mkv.quantize_pack_kv(k, v, tab, cache)
    g = torch.Generator(device=DEV)
    g.manual_seed(w.seed * 100 + 9)
    tk = torch.randn((w.B, w.Hkv, 4100, d), generator=g, device=DEV).to(torch.float16)
    tv = torch.randn((w.B, w.Hkv, 4100, d), generator=g, device=DEV).to(torch.float16)
    out = mkv.mixed_kv_decode_attention(q, cache, tail_k=tk, tail_v=tv, tail_len=4095)
    torch.cuda.synchronize()
    bits, rank, perm, seg = tables_np(tab)
    check_canary(cache, seg)
    pools = P.pools_np(cache)
    n = P.check_quantize(cache, pools, P.to_np(k), P.to_np(v), bits, rank,
                         [(0, h, c) for h in range(w.Hkv) for c in range(w.n)])
    err = P.check_attention(cache, pools, bits, rank, w.n, P.to_np(q), P.to_np(out),
                            [(0, hq) for hq in range(Hq)], P.to_np(tk[:, :, :4095]), P.to_np(tv[:, :, :4095]))
    note(f"  quantize: {n} chunks exact; attention with 4095-token tail: max rel err {err:.2e}")

    Pn = 1024
    tab2, cache2, q2, kn, vn, out2 = run_prefill(w, experts, Pn)
    rows = sorted(set(range(0, Pn, 61)) | {1, 31, 32, 33, 255, 256, Pn - 2, Pn - 1})
    err = check_prefill(w, tab2, cache2, q2, kn, vn, out2, [(0, hq) for hq in range(Hq)], rows)
    note(f"  prefill P={Pn} over the 1024-token chunks: max rel err {err:.2e} over {len(rows) * Hq} rows")


@pytest.mark.parametrize("d,Pn", [(64, 1), (64, 33), (128, 1), (128, 97)])
def test_prefill_one_group_chunks_odd_segments(d, Pn):
    """C = 32: FP16, INT4 and INT2 segments of 1, 3 and 7 chunks (2, 5 and 4
    in the second sequence), so the cache is walked in pairs of blocks with an
    odd block left over; one query, or a query count that leaves a ragged
    tile."""
    w = configs.Workload(name=f"prefill-C32-d{d}", seed=211 + d + Pn, B=2, Hq=4, Hkv=2, d=d, T=11 * 32, C=32,
                         outlier_cols=2, outlier_mult=8.0)
    note(f"prefill {w.name}, P={Pn}")
    experts = torch.from_numpy(orc.expert_of_bits(np.array(
        [[16, 4, 2, 4, 2, 4, 2, 2, 2, 2, 2],
         [16, 2, 4, 4, 2, 16, 4, 4, 2, 4, 2]], np.uint8)))
    tab, cache, q, kn, vn, out = run_prefill(w, experts, Pn)
    seg = P.to_np(tab.seg_count)
    assert seg.tolist() == [[1, 3, 7], [2, 5, 4]]
    heads = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
    err = check_prefill(w, tab, cache, q, kn, vn, out, heads, range(Pn))
    note(f"  max rel err {err:.2e} over {len(heads) * Pn} query rows")
