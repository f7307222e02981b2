"""GPU parity of streaming decode: tokens appended one at a time into the
fp16 tail, each full chunk routed, quantized and appended, pools grown as
segments fill.  Every checked step's attention is compared with the oracle
over the GPU's own packed chunks plus the exact fp16 tokens of the tail;
routed chunks and their codes are compared with the oracle as in the
one-shot path."""
import numpy as np
import pytest
import torch

from chunk_mixed_precision_amd import configs, decode, mkv, synth
from oracle import mkv_oracle as orc
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("d,C,Hq,Hkv,layers", [(128, 32, 4, 2, 2), (64, 64, 2, 2, 1)])
def test_streaming_decode_matches_oracle(d, C, Hq, Hkv, layers):
    B, prefill_chunks, steps = 2, 2, 3 * C + 5
    T0 = prefill_chunks * C
    T = T0 + ((steps + C - 1) // C) * C
    w = configs.Workload(name=f"decode-d{d}-C{C}", seed=61 + d + C, B=B, Hq=Hq, Hkv=Hkv, d=d, T=T, C=C, D=256,
                         I=128, x_chunk_share=1.0, router_std=0.05, b3=(0.0, 0.02, 0.0))
    note(f"streaming decode {w.name}, {steps} steps after {T0} prefill tokens, {layers} layer(s)")
    x, w12, w3, b3 = synth.router_inputs(w)
    kv = [synth.kv(w, DEV, layer=l) for l in range(layers)]
    qg = torch.Generator(device=DEV)
    qg.manual_seed(w.seed * 100 + 88)
    qs = torch.randn((steps, layers, B, Hq, d), generator=qg, device=DEV).to(torch.float16)
    xd = x.to(DEV)
    sess = decode.DecodeSession(B, Hq, Hkv, d, C, layers, w12.to(DEV), w3.to(DEV), b3.to(DEV),
                                max_chunks=T // C, caps=(1, 1, 1))
    sess.prefill(xd[:, :T0].contiguous(), [(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous()) for k, v in kv])

    # oracle routing of every chunk of the whole context (near ties may flip)
    z, e_tok, v_ref, _, _, _ = orc.route(P.bf16_bits(x), P.bf16_bits(w12), w3.numpy().astype(np.float64),
                                         b3.numpy().astype(np.float64), w.I, C)
    zs = np.sort(z, axis=-1)
    tie_chunk = ((zs[..., 2] - zs[..., 1]) <= 1e-4).reshape(B, T // C, C).any(axis=2)

    k_np = [P.to_np(k) for k, _ in kv]
    v_np = [P.to_np(v) for _, v in kv]
    check_at = {0, C - 2, C - 1, C, 2 * C - 1, 2 * C + 3, steps - 1}
    worst = 0.0
    for s in range(steps):
        t = T0 + s
        outs = sess.step(xd[:, t].contiguous(), [(k[:, :, t].contiguous(), v[:, :, t].contiguous()) for k, v in kv],
                         [qs[s, l] for l in range(layers)])
        if s not in check_at:
            continue
        torch.cuda.synchronize()
        n_cached = T0 // C + (s + 1) // C        # chunks in the cache after this step's flush
        tail_start = n_cached * C
        tail_len = t + 1 - tail_start
        bits, rank, perm, seg = (P.to_np(sess.tab.chunk_bits), P.to_np(sess.tab.chunk_rank),
                                 P.to_np(sess.tab.perm), P.to_np(sess.tab.seg_count))
        assert sess.n == n_cached and sess.tail_len == tail_len
        # the attention of this step saw the chunks cached before it and the
        # tail as it stood (the flush, if any, came after)
        n_seen = T0 // C + s // C
        seen_tail = t + 1 - n_seen * C
        for l in range(layers):
            pools = P.pools_np(sess.caches[l])
            tk = k_np[l][:, :, n_seen * C:t + 1]
            tv = v_np[l][:, :, n_seen * C:t + 1]
            assert tk.shape[2] == seen_tail
            err = P.check_attention(sess.caches[l], pools, bits, rank, n_seen, P.to_np(qs[s, l]),
                                    P.to_np(outs[l]), [(b, hq) for b in range(B) for hq in range(Hq)], tk, tv)
            worst = max(worst, err)
        # routing, reorder and codes of everything cached so far
        P.check_reorder_only(bits, rank, perm, seg, n_cached)
        got = orc.expert_of_bits(bits[:, :n_cached])
        mism = (got != v_ref[:, :n_cached]) & ~tie_chunk[:, :n_cached]
        assert not mism.any(), np.argwhere(mism)
        for l in range(layers):
            pools = P.pools_np(sess.caches[l])
            P.check_quantize(sess.caches[l], pools, k_np[l], v_np[l], bits, rank,
                             [(b, h, c) for b in range(B) for h in range(Hkv) for c in range(n_cached)])
        note(f"  step {s}: {n_cached} chunks cached, tail {tail_len}, caps {sess.caps}, "
             f"pool re-layouts {sess.grown}, attention max rel err so far {worst:.2e}")
    assert sess.grown > 0                     # the pools did grow from one slot
    for c in sess.caches:
        assert int(c.overflow.cpu()[0]) == 0
