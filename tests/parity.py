"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare every stage with the oracle on the same input bytes.

Stage rules (the build's parity bar):
  router    logits within the fp32-accumulation error of the oracle's fp64
            logits; an expert may differ only where the oracle's top-2 gap is
            <= 1e-4 (counted).
  vote      the oracle's vote rerun on the GPU's token experts equals the GPU's
            chunk bitwidths exactly (freezing included).
  reorder   the oracle's stable partition of the GPU's chunk bitwidths equals
            rank, perm and seg_count exactly.
  quantize  every compared chunk: codes equal, scale and min bit-equal, FP16
            bytes equal.
  attention max over (b, hq) of |o_gpu - o_ref|_inf / |o_ref|_inf <= 2e-3,
            o_ref = fp64 attention on the GPU's own packed cache.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import mkv_oracle as orc
from tests import layout_ref

ATTN_TOL = 2e-3
NEAR_TIE = 1e-4
# Two attention calls on the same inputs differ only in the fp32 summation
# order (work units are handed to wavefronts dynamically).  The measured
# spread stays below about 1.1e-5 of max|o| per (sequence, head); this bound
# leaves a few times that.
RUN_TO_RUN = 5e-5


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def check_router(x, w12, w3, b3, inner, logits_gpu, experts_gpu, rows=None):
    """x [N, D] bf16 (CPU or GPU), logits_gpu [N, 3], experts_gpu [N].
    rows: optional sample of token rows.  Returns a report dict; raises on a
    flip outside the near-tie band."""
    xb = bf16_bits(x)
    if rows is not None:
        xb = xb[rows]
        logits_gpu = logits_gpu[rows]
        experts_gpu = experts_gpu[rows]
    z = orc.router_logits(orc.bf16_bits_to_f64(xb), orc.bf16_bits_to_f64(bf16_bits(w12)),
                          to_np(w3).astype(np.float64), to_np(b3).astype(np.float64), inner)
    e_ref = orc.token_experts(z)
    zs = np.sort(z, axis=1)
    gap = zs[:, 2] - zs[:, 1]
    flips = e_ref != experts_gpu
    bad = flips & (gap > NEAR_TIE)
    rep = {"tokens": int(len(z)), "flips": int(flips.sum()), "near_tie": int((gap <= NEAR_TIE).sum()),
           "max_abs_logit_err": float(np.max(np.abs(logits_gpu.astype(np.float64) - z))),
           "max_abs_logit": float(np.max(np.abs(z)))}
    assert not bad.any(), f"router flips outside the near-tie band: {rep}"
    return rep


def check_vote_and_reorder(experts_gpu_bt, C, chunk_bits_gpu, rank_gpu, perm_gpu, seg_gpu,
                           freeze_first=True, chunk_offset=0, prior_experts=None):
    """experts_gpu_bt [B, Tnew]; tables [B, n_max] (only the first n_total
    columns are meaningful).  prior_experts: [B, chunk_offset] chunk experts
    kept from earlier calls (append mode)."""
    v_new = orc.chunk_vote(experts_gpu_bt, C, freeze_first=freeze_first, chunk_offset=chunk_offset)
    n_new = v_new.shape[1]
    n_total = chunk_offset + n_new
    got = orc.expert_of_bits(chunk_bits_gpu[:, chunk_offset:n_total])
    assert np.array_equal(got, v_new), "vote mismatch"
    v_all = v_new if prior_experts is None else np.concatenate([prior_experts, v_new], axis=1)
    perm, rank, seg = orc.reorder(v_all)
    assert np.array_equal(rank_gpu[:, :n_total], rank), "chunk_rank mismatch"
    assert np.array_equal(perm_gpu[:, :n_total], perm), "perm mismatch"
    assert np.array_equal(seg_gpu, seg), "seg_count mismatch"
    return v_all


def check_reorder_only(chunk_bits_gpu, rank_gpu, perm_gpu, seg_gpu, n_total):
    v = orc.expert_of_bits(chunk_bits_gpu[:, :n_total])
    perm, rank, seg = orc.reorder(v)
    assert np.array_equal(rank_gpu[:, :n_total], rank)
    assert np.array_equal(perm_gpu[:, :n_total], perm)
    assert np.array_equal(seg_gpu, seg)
    return v


def pools_np(cache):
    return [to_np(p) for p in cache.pools]


def check_quantize(cache, pools, k_np, v_np, chunk_bits, chunk_rank, triples, chunk_offset=0):
    """triples: (b, h, c) with c the chunk index *within k_np/v_np* (the
    chunk's table index is chunk_offset + c).  Compares every listed chunk
    exactly with the oracle.  Returns the number of chunks compared."""
    d, C, Hkv = cache.d, cache.C, cache.Hkv
    by_bits = {}
    for (b, h, c) in triples:
        bits = int(chunk_bits[b, chunk_offset + c])
        slot = int(chunk_rank[b, chunk_offset + c])
        by_bits.setdefault(bits, []).append((b, h, c, slot))
    n = 0
    for bits, items in by_bits.items():
        kidx = orc.EXPERT_BITS.index(bits)
        dec = layout_ref.decode_chunks(pools[kidx], bits, Hkv, cache.caps[kidx], d, C,
                                       [(b, h, slot) for (b, h, c, slot) in items])
        for (b, h, c, slot), got in zip(items, dec):
            kk = k_np[b, h, c * C:(c + 1) * C]
            vv = v_np[b, h, c * C:(c + 1) * C]
            ref = orc.quantize_chunk(kk, vv, bits)
            where = f"(b={b}, h={h}, chunk={chunk_offset + c}, bits={bits}, slot={slot})"
            if bits == 16:
                assert np.array_equal(got["k"].view(np.uint16), ref["k"].view(np.uint16)), "fp16 K " + where
                assert np.array_equal(got["v"].view(np.uint16), ref["v"].view(np.uint16)), "fp16 V " + where
            else:
                for key in ("kq", "vq"):
                    if not np.array_equal(got[key], ref[key]):
                        bad = np.argwhere(got[key] != ref[key])[:5]
                        raise AssertionError(f"{key} codes differ at {bad.tolist()} {where}")
                for key in ("ks", "km", "vs", "vm"):
                    gb = np.ascontiguousarray(got[key]).view(np.uint32)
                    rb = np.ascontiguousarray(ref[key].astype(np.float32)).view(np.uint32)
                    if not np.array_equal(gb, rb):
                        bad = np.argwhere(gb != rb)[:5]
                        raise AssertionError(f"{key} bits differ at {bad.tolist()} {where}")
            n += 1
    return n


def dequant_sequence_head(cache, pools, chunk_bits_row, chunk_rank_row, n_total, b, h):
    """The GPU's packed chunks of (b, h) decoded and dequantized (fp64),
    concatenated in chunk order: (k_hat [T, d], v_hat [T, d])."""
    d, C, Hkv = cache.d, cache.C, cache.Hkv
    ks, vs = [], []
    slots = {}
    for c in range(n_total):
        bits = int(chunk_bits_row[c])
        slots.setdefault(bits, []).append((c, int(chunk_rank_row[c])))
    parts = {}
    for bits, items in slots.items():
        kidx = orc.EXPERT_BITS.index(bits)
        dec = layout_ref.decode_chunks(pools[kidx], bits, Hkv, cache.caps[kidx], d, C,
                                       [(b, h, s) for (c, s) in items])
        for (c, s), ch in zip(items, dec):
            parts[c] = orc.dequant_chunk(ch)
    for c in range(n_total):
        ks.append(parts[c][0])
        vs.append(parts[c][1])
    if not ks:
        return np.zeros((0, d)), np.zeros((0, d))
    return np.concatenate(ks), np.concatenate(vs)


def check_attention(cache, pools, chunk_bits, chunk_rank, n_total, q_np, out_np, pairs,
                    tail_k=None, tail_v=None, tol=ATTN_TOL):
    """pairs: (b, hq).  Returns the max relative error."""
    Hq = q_np.shape[1]
    g = Hq // cache.Hkv
    worst = 0.0
    memo = {}
    for (b, hq) in pairs:
        h = hq // g
        if (b, h) not in memo:
            kh, vh = dequant_sequence_head(cache, pools, chunk_bits[b], chunk_rank[b], n_total, b, h)
            if tail_k is not None and tail_k.shape[2] > 0:
                kh = np.concatenate([kh, tail_k[b, h].astype(np.float64)])
                vh = np.concatenate([vh, tail_v[b, h].astype(np.float64)])
            memo[(b, h)] = (kh, vh)
        kh, vh = memo[(b, h)]
        if len(kh) == 0:
            ref = np.zeros(cache.d)
            assert np.all(out_np[b, hq] == 0), "empty (b, h) must give zeros"
            continue
        ref = orc.attention(q_np[b, hq].astype(np.float64), kh, vh)
        err = np.max(np.abs(out_np[b, hq].astype(np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30)
        worst = max(worst, err)
        assert err <= tol, f"attention rel err {err:.3e} > {tol} at (b={b}, hq={hq})"
    return worst
