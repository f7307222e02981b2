"""GPU parity of the similarity-based chunk selection (Cocktail abstract:
chunk-level quantization search) against the CPU oracle: similarities, the
bitwidths they give, and the reorder tables built on the GPU's own bits."""
import numpy as np
import pytest
import torch

from chunk_mixed_precision_amd import configs, mkv, synth
from oracle import mkv_oracle as orc
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"
SIM_TOL = 1e-5   # |sim_gpu - sim_oracle|: fp32 sums of bf16 products against fp64
SIM_EPS = 1e-4   # a bitwidth may differ from the oracle's only this close to a threshold


def note(msg):
    print(msg, flush=True)


def oracle_sim(x, qe, C):
    B, T, D = x.shape
    xf = orc.bf16_bits_to_f64(P.bf16_bits(x).reshape(-1, D)).reshape(B, T, D)
    return orc.chunk_similarity(xf, orc.bf16_bits_to_f64(P.bf16_bits(qe)), C)


def check_selection(sim_ref, sim_gpu, bits_gpu, tau_hi, tau_lo, freeze, chunk_offset=0):
    """Similarities within SIM_TOL; bitwidths equal to the oracle's except
    where the oracle's similarity is within SIM_EPS of a threshold (counted)."""
    n = sim_ref.shape[1]
    err = float(np.abs(sim_gpu - sim_ref).max())
    assert err <= SIM_TOL, err
    e_ref = orc.similarity_experts(sim_ref, tau_hi, tau_lo, freeze, chunk_offset)
    e_gpu = orc.expert_of_bits(bits_gpu[:, chunk_offset:chunk_offset + n])
    near = np.minimum(np.abs(sim_ref - tau_hi), np.abs(sim_ref - tau_lo)) <= SIM_EPS
    diff = e_ref != e_gpu
    assert not np.any(diff & ~near), np.argwhere(diff & ~near)[:5]
    return {"chunks": int(sim_ref.size), "max_abs_sim_err": err, "near_threshold": int(near.sum()),
            "flips": int(diff.sum()), "mix": np.bincount(e_gpu.ravel(), minlength=3).tolist()}


def tables_np(tab):
    return (P.to_np(tab.chunk_bits), P.to_np(tab.chunk_rank), P.to_np(tab.perm), P.to_np(tab.seg_count))


def run_select(tab, C, x, qe, tau_hi, tau_lo, freeze=True, append=False, chunk_offset=0):
    n_new = x.shape[1] // C
    sim = torch.empty((x.shape[0], n_new), dtype=torch.float32, device=DEV)
    mkv.select_chunks_by_similarity(tab, C, x.to(DEV), qe.to(DEV), tau_hi, tau_lo, sim=sim, freeze_first=freeze,
                                    append=append, chunk_offset=chunk_offset)
    torch.cuda.synchronize()
    return P.to_np(sim).astype(np.float64)


@pytest.mark.parametrize("D,C,freeze", [(256, 128, True), (320, 32, False), (1024, 256, True)])
def test_similarity_selection_small(D, C, freeze):
    w = configs.Workload(name=f"sim-D{D}-C{C}", seed=31 + D + C, B=3, Hq=4, Hkv=4, d=128, T=8 * C * 2, C=C,
                         D=D, I=128, x_chunk_share=1.0)
    note(f"similarity {w.name}")
    x, *_ = synth.router_inputs(w)
    qe = synth.query_embedding(w)
    tau_hi, tau_lo = 0.3, -0.02
    tab = mkv.RouteTables(w.B, w.n, DEV)
    sim_gpu = run_select(tab, w.C, x, qe, tau_hi, tau_lo, freeze=freeze)
    sim_ref = oracle_sim(x, qe, w.C)
    bits, rank, perm, seg = tables_np(tab)
    rep = check_selection(sim_ref, sim_gpu, bits, tau_hi, tau_lo, freeze)
    note(f"  {rep}")
    assert all(m > 0 for m in rep["mix"])          # every bitwidth occurs
    P.check_reorder_only(bits, rank, perm, seg, w.n)


def test_similarity_selection_append_and_zero_vectors():
    """Appended chunks keep the earlier tables and are never frozen; a zero
    query embedding and an all-zero chunk have similarity 0."""
    w = configs.Workload(name="sim-append", seed=47, B=3, Hq=4, Hkv=4, d=128, T=1024, C=128, D=512, I=128,
                         x_chunk_share=1.0)
    note(f"similarity {w.name}")
    prior = torch.tensor([[1, 2, 0, 1, 1, 2, 2, 1], [2, 2, 2, 2, 1, 1, 1, 1], [0, 1, 2, 0, 1, 2, 0, 1]],
                         dtype=torch.uint8)
    tab = mkv.RouteTables(w.B, w.n + 4, DEV)
    mkv.route_chunks(tab, w.C, logits=synth.one_hot_logits(prior, w.C).to(DEV), logits_in=True, freeze_first=True)
    x, *_ = synth.router_inputs(w, tokens_per_seq=4 * w.C, chunk_offset=w.n)
    x[1, w.C:2 * w.C] = 0                          # an all-zero chunk
    qe = synth.query_embedding(w)
    qe[2] = 0                                      # a zero query
    tau_hi, tau_lo = 0.05, 0.0
    sim_gpu = run_select(tab, w.C, x, qe, tau_hi, tau_lo, freeze=True, append=True, chunk_offset=w.n)
    sim_ref = oracle_sim(x, qe, w.C)
    assert sim_gpu[1, 1] == 0.0 and np.all(sim_gpu[2] == 0.0)
    bits, rank, perm, seg = tables_np(tab)
    rep = check_selection(sim_ref, sim_gpu, bits, tau_hi, tau_lo, True, chunk_offset=w.n)
    note(f"  {rep}")
    prior_bits = orc.bits_of(orc.chunk_vote(np.repeat(prior.numpy(), w.C, axis=1), w.C, freeze_first=True))
    assert np.array_equal(bits[:, :w.n], prior_bits)
    P.check_reorder_only(bits, rank, perm, seg, w.n + 4)


def test_similarity_selection_full_size_llama2_7b_32k():
    """The llama2-7b 32k shape: 32768 tokens x 4096 dims of embeddings, 128
    chunks of 256, every chunk checked."""
    w = configs.LLAMA2_7B_32K
    note(f"similarity {w.name}")
    x, *_ = synth.router_inputs(w)
    qe = synth.query_embedding(w)
    tau_hi, tau_lo = 0.3, 0.0
    tab = mkv.RouteTables(w.B, w.n, DEV)
    sim_gpu = run_select(tab, w.C, x, qe, tau_hi, tau_lo)
    sim_ref = oracle_sim(x, qe, w.C)
    bits, rank, perm, seg = tables_np(tab)
    rep = check_selection(sim_ref, sim_gpu, bits, tau_hi, tau_lo, True)
    note(f"  {rep}")
    P.check_reorder_only(bits, rank, perm, seg, w.n)
