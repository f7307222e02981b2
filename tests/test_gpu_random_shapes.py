"""GPU parity on seeded random shapes inside the C ABI's limits: head_dim,
chunk size (any multiple of 32 up to 512), query heads per KV head,
sequences, chunks per sequence, fp16 tail length, chunk mix and prefill
chunk length are drawn once from a fixed seed.  Every shape goes through
quantize + pack (every chunk compared bit for bit), decode attention over
the packed chunks and the tail (every head), and chunked prefill (sampled
heads and query rows), each against the oracle."""
import numpy as np
import pytest
import torch

from chunk_mixed_precision_amd import configs, mkv, synth
from oracle import mkv_oracle as orc
from tests import parity as P
from tests.test_gpu_parity import build_tables_from_experts, check_canary, full_check, run_quant_attn, tables_np
from tests.test_gpu_prefill import check_prefill, run_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(msg, flush=True)


def _shapes(count=10, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        d = int(rng.choice([64, 128]))
        C = 32 * int(rng.integers(1, 17))                  # 32 .. 512
        g = int(rng.choice([1, 2, 4]))
        Hkv = int(rng.integers(1, 6))
        B = int(rng.integers(1, 8))
        n = int(rng.integers(1, 10))
        tail = int(rng.choice([0, 1, 17, C - 1]))
        f = rng.dirichlet([1.0, 1.0, 1.0])
        Pn = int(rng.integers(1, 301))
        out.append((i, d, C, g, Hkv, B, n, tail, (float(f[0]), float(f[1]), float(f[2])), Pn))
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("i,d,C,g,Hkv,B,n,tail,mix,Pn", SHAPES, ids=[
    f"s{s[0]}-d{s[1]}-C{s[2]}-g{s[3]}-Hkv{s[4]}-B{s[5]}-n{s[6]}-tail{s[7]}-P{s[9]}" for s in SHAPES])
def test_random_shape(i, d, C, g, Hkv, B, n, tail, mix, Pn):
    w = configs.Workload(name=f"random-{i}", seed=300 + i, B=B, Hq=g * Hkv, Hkv=Hkv, d=d, T=n * C, C=C,
                         mix=mix, outlier_cols=2, outlier_mult=8.0)
    note(f"shape {i}: d={d} C={C} Hq={w.Hq} Hkv={Hkv} B={B} chunks={n} tail={tail} mix={np.round(mix, 2)} P={Pn}")
    experts = synth.drawn_chunk_experts(w)
    freeze = bool(i % 2 == 0)
    tab = build_tables_from_experts(experts, C, freeze=freeze)
    bits, rank, perm, seg = tables_np(tab)
    v_ref = orc.chunk_vote(orc.expert_of_bits(np.repeat(synth.bits_tensor(experts).numpy(), C, axis=1)), C,
                           freeze_first=freeze)
    assert np.array_equal(orc.expert_of_bits(bits[:, :n]), v_ref)
    P.check_reorder_only(bits, rank, perm, seg, n)
    k, v = synth.kv(w, DEV)
    q = synth.query(w, DEV)
    cache, out, tk, tv = run_quant_attn(w, tab, k, v, q, n, tail=tail)
    check_canary(cache, seg)
    full_check(w, tab, cache, out, k, v, q, n, tk, tv)

    tab2, cache2, q2, kn, vn, out2 = run_prefill(w, experts, Pn)
    rng = np.random.default_rng(i)
    heads = sorted({(int(b), int(hq)) for b, hq in zip(rng.integers(0, B, 4), rng.integers(0, w.Hq, 4))})
    rows = sorted({0, Pn - 1} | {int(r) for r in rng.integers(0, Pn, 4)})
    err = check_prefill(w, tab2, cache2, q2, kn, vn, out2, heads, rows)
    note(f"  prefill: max rel err {err:.2e} over {len(heads) * len(rows)} rows")
