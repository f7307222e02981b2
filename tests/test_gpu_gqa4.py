"""GPU parity of decode attention with four query heads per KV head, whose
row pairs split each group block by data and load only the rows they use:
every (sequence, query head) against the oracle on caches of one bitwidth
alone, on segments of odd group-block counts (the last unit of a segment
then has a row pair past its end), on segments that change bitwidth inside
a wavefront's run of units, with and without an fp16 tail, at head_dim 64
and 128."""
import numpy as np
import pytest
import torch

from chunk_mixed_precision_amd import configs, synth
from oracle import mkv_oracle as orc
from tests import parity as P
from tests.test_gpu_parity import build_tables_from_experts, check_canary, full_check, run_quant_attn, tables_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [16, 4, 2])
def test_gqa4_one_bitwidth(d, bits):
    """Every chunk of one bitwidth (no freezing), 7 one-group chunks per
    stream: 7 group blocks, so the last unit has dead row pairs."""
    n, C = 7, 32
    w = configs.Workload(name=f"gqa4-only{bits}-d{d}", seed=401 + d + bits, B=3, Hq=8, Hkv=2, d=d, T=n * C, C=C,
                         outlier_cols=2, outlier_mult=8.0)
    note(f"{w.name}")
    experts = torch.from_numpy(orc.expert_of_bits(np.full((w.B, n), bits, np.uint8)))
    tab = build_tables_from_experts(experts, C, freeze=False)
    bits_t, rank, perm, seg = tables_np(tab)
    assert seg[:, orc.EXPERT_BITS.index(bits)].tolist() == [n] * w.B
    k, v = synth.kv(w, DEV)
    q = synth.query(w, DEV)
    cache, out, tk, tv = run_quant_attn(w, tab, k, v, q, n, tail=0)
    check_canary(cache, seg)
    err = full_check(w, tab, cache, out, k, v, q, n, tk, tv)
    assert err <= P.ATTN_TOL


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tail", [0, 29])
def test_gqa4_ragged_segments(d, tail):
    """Three sequences with segments of 1-6 one-group chunks each (odd and
    even block counts, an empty INT2 segment in one sequence), so units of
    every bitwidth end with a live or a dead row pair and a wavefront's
    prefetch crosses from one segment to the next."""
    C = 32
    pattern = np.array([[16, 4, 2, 4, 2, 4, 2, 2, 4, 16, 4],
                        [16, 16, 16, 4, 4, 4, 4, 4, 16, 16, 4],
                        [2, 4, 2, 2, 16, 2, 4, 2, 2, 2, 16]], np.uint8)
    n = pattern.shape[1]
    w = configs.Workload(name=f"gqa4-ragged-d{d}-t{tail}", seed=433 + d + tail, B=3, Hq=8, Hkv=2, d=d, T=n * C, C=C,
                         outlier_cols=2, outlier_mult=8.0)
    note(f"{w.name}")
    experts = torch.from_numpy(orc.expert_of_bits(pattern))
    tab = build_tables_from_experts(experts, C, freeze=False)
    bits_t, rank, perm, seg = tables_np(tab)
    assert seg.tolist() == [[2, 5, 4], [5, 6, 0], [2, 2, 7]]
    k, v = synth.kv(w, DEV)
    q = synth.query(w, DEV)
    cache, out, tk, tv = run_quant_attn(w, tab, k, v, q, n, tail=tail)
    check_canary(cache, seg)
    err = full_check(w, tab, cache, out, k, v, q, n, tk, tv)
    assert err <= P.ATTN_TOL
