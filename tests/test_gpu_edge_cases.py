"""GPU parity on the method's edge cases, compared both with the oracle and
with values fixed by hand:

  - the chunk vote on crafted per-token scores (MoQAE notes, "Key designs",
    quantization-aware experts: every token takes its highest-scoring expert
    and the chunk takes the most frequent one; count ties and exact score
    ties go to the higher-precision expert), with routing freezing on and off;
  - the hand-worked quantization groups of tests/golden/quant_hand_cases.json
    (round-half-even ties, the reciprocal-versus-divide case, a scale that is
    not representable, constant groups and signed-zero minima) pushed through
    mkv_quantize_pack_kv as key groups (32 tokens of one channel) and value
    groups (32 channels of one token), compared bit for bit with the golden
    codes, scales and minima.
"""
import json
import os
import struct

import numpy as np
import pytest
import torch

from chunk_mixed_precision_amd import mkv
from oracle import mkv_oracle as orc
from tests import layout_ref
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def note(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ crafted votes
C32 = 32
ONE_ABOVE_1 = float(np.nextafter(np.float32(1.0), np.float32(2.0)))


def _count_chunk(rng, c0, c1, c2):
    """Scores for 32 tokens whose winners occur c0, c1, c2 times, in a random
    token order: the winner scores 2 + u, the others u' < 1."""
    winners = np.array([0] * c0 + [1] * c1 + [2] * c2)
    rng.shuffle(winners)
    z = rng.random((32, 3)).astype(np.float32)
    z[np.arange(32), winners] = 2.0 + z[np.arange(32), winners]
    return z, winners


def _crafted_chunks(rng):
    """(scores [32, 3], token experts [32], expected chunk bits) per chunk."""
    out = []
    for counts, bits in (((11, 11, 10), 16), ((10, 11, 11), 4), ((10, 10, 12), 2),
                         ((16, 0, 16), 16), ((0, 16, 16), 4), ((5, 5, 22), 2)):
        z, e = _count_chunk(rng, *counts)
        out.append((z, e, bits))
    # exact score ties on every token
    out.append((np.tile(np.float32([0.25, 0.25, 0.25]), (32, 1)), np.zeros(32, int), 16))
    out.append((np.tile(np.float32([0.0, 0.5, 0.5]), (32, 1)), np.ones(32, int), 4))
    out.append((np.tile(np.float32([-1.0, -3.0, -1.0]), (32, 1)), np.zeros(32, int), 16))
    # a one-ulp lead decides the token
    out.append((np.tile(np.float32([0.0, 1.0, ONE_ABOVE_1]), (32, 1)), np.full(32, 2), 2))
    return out


@pytest.mark.parametrize("freeze", [True, False])
def test_vote_on_crafted_scores_c32(freeze):
    rng = np.random.default_rng(2024)
    chunks = _crafted_chunks(rng)
    n = len(chunks)
    orders = [list(range(n)), list(rng.permutation(n))]          # two sequences, different chunk 0
    B = len(orders)
    z = np.zeros((B, n * C32, 3), np.float32)
    e_want = np.zeros((B, n * C32), np.uint8)
    bits_want = np.zeros((B, n), np.uint8)
    for b, order in enumerate(orders):
        for c, idx in enumerate(order):
            zz, ee, bb = chunks[idx]
            z[b, c * C32:(c + 1) * C32] = zz
            e_want[b, c * C32:(c + 1) * C32] = ee
            bits_want[b, c] = bb
        if freeze:
            bits_want[b, 0] = 16
    note(f"crafted votes, freeze={freeze}: expected bits {bits_want.tolist()}")
    tab = mkv.RouteTables(B, n, DEV)
    te = torch.empty((B, n * C32), dtype=torch.uint8, device=DEV)
    mkv.route_chunks(tab, C32, logits=torch.from_numpy(z).to(DEV), logits_in=True, freeze_first=freeze,
                     token_expert=te)
    torch.cuda.synchronize()
    te_np = P.to_np(te)
    bits, rank, perm, seg = (P.to_np(t) for t in (tab.chunk_bits, tab.chunk_rank, tab.perm, tab.seg_count))
    assert np.array_equal(te_np, e_want), "token experts differ from the hand-fixed winners"
    assert np.array_equal(te_np, orc.token_experts(z.astype(np.float64)))
    assert np.array_equal(bits, bits_want), f"chunk bits {bits.tolist()}"
    P.check_vote_and_reorder(te_np, C32, bits, rank, perm, seg, freeze_first=freeze)


# ------------------------------------------------------------------ golden quantizer groups
def _golden():
    with open(os.path.join(GOLD, "quant_hand_cases.json")) as f:
        cases = json.load(f)["cases"]
    out = []
    for c in cases:
        n = len(c["head"])
        vals = np.array(list(c["head"]) + [c["fill"]] * (32 - n), np.float16)
        codes = np.array(list(c["codes_head"]) + [c["codes_fill"]] * (32 - n), np.uint8)
        s_bits = int(c["s_hex"], 16) if "s_hex" in c else struct.unpack("<I", struct.pack("<f", c["s"]))[0]
        mn_bits = int(c["mn_hex"], 16) if "mn_hex" in c else struct.unpack("<I", struct.pack("<f", c["mn"]))[0]
        out.append(dict(name=c["name"], bits=c["bits"], vals=vals, codes=codes, s=s_bits, mn=mn_bits))
    return out


@pytest.mark.parametrize("d", [64, 128])
def test_quantize_golden_groups_bit_exact(d):
    """Chunk 0 is INT4 and chunk 1 INT2 (freezing off, C = 32).  Key channel
    j of a chunk holds golden group (j mod #groups) along its 32 tokens;
    value group g of token t holds golden group ((NG*t + g) mod #groups)
    along its 32 channels."""
    cases = _golden()
    by_bits = {4: [c for c in cases if c["bits"] == 4], 2: [c for c in cases if c["bits"] == 2]}
    NG = d // 32
    k = np.zeros((1, 1, 64, d), np.float16)
    v = np.zeros((1, 1, 64, d), np.float16)
    want = {}
    for ci, bits in enumerate((4, 2)):
        gs = by_bits[bits]
        for j in range(d):
            k[0, 0, 32 * ci:32 * ci + 32, j] = gs[j % len(gs)]["vals"]
        for t in range(32):
            for g in range(NG):
                v[0, 0, 32 * ci + t, 32 * g:32 * g + 32] = gs[(NG * t + g) % len(gs)]["vals"]
        want[bits] = gs
    tab = mkv.RouteTables(1, 2, DEV)
    z = torch.zeros((1, 64, 3), dtype=torch.float32)
    z[0, :32, 1] = 1.0
    z[0, 32:, 2] = 1.0
    mkv.route_chunks(tab, 32, logits=z.to(DEV), logits_in=True, freeze_first=False)
    cache = mkv.PackedCache(1, 1, d, 32, [0, 1, 1], tab.seg_count, DEV)
    kt, vt = torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV)
    mkv.quantize_pack_kv(kt, vt, tab, cache)
    torch.cuda.synchronize()
    pools = P.pools_np(cache)
    for ci, bits in enumerate((4, 2)):
        gs = want[bits]
        kidx = orc.EXPERT_BITS.index(bits)
        got = layout_ref.decode_chunks(pools[kidx], bits, 1, 1, d, 32, [(0, 0, 0)])[0]
        for j in range(d):
            gc = gs[j % len(gs)]
            where = f"key channel {j}, INT{bits} group {gc['name']}"
            assert np.array_equal(got["kq"][:, j], gc["codes"]), where
            assert int(np.float32(got["ks"][0, j]).view(np.uint32)) == gc["s"], where
            assert int(np.float32(got["km"][0, j]).view(np.uint32)) == gc["mn"], where
        for t in range(32):
            for g in range(NG):
                gc = gs[(NG * t + g) % len(gs)]
                where = f"value token {t} group {g}, INT{bits} group {gc['name']}"
                assert np.array_equal(got["vq"][t, 32 * g:32 * g + 32], gc["codes"]), where
                assert int(np.float32(got["vs"][t, g]).view(np.uint32)) == gc["s"], where
                assert int(np.float32(got["vm"][t, g]).view(np.uint32)) == gc["mn"], where
    # the same chunks against the oracle, and attention over them
    bits_np, rank_np = P.to_np(tab.chunk_bits), P.to_np(tab.chunk_rank)
    P.check_quantize(cache, pools, k, v, bits_np, rank_np, [(0, 0, 0), (0, 0, 1)])
    q = torch.randn((1, 1, d), generator=torch.Generator().manual_seed(9)).to(torch.float16)
    out = mkv.mixed_kv_decode_attention(q.to(DEV), cache)
    torch.cuda.synchronize()
    err = P.check_attention(cache, pools, bits_np, rank_np, 2, q.numpy(), P.to_np(out), [(0, 0)])
    note(f"golden groups d={d}: {len(cases)} groups bit-exact as keys and values; attention rel err {err:.2e}")
