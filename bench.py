#!/usr/bin/env python3
"""Throughput of the chunk-adaptive mixed-precision KV path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
of the named workload, one call of each:
  pack    mkv_quantize_pack_kv   K/V of every chunk -> packed FP16/INT4/INT2 segments
  route   mkv_route_chunks       router GEMM (bf16 MFMA) -> vote -> freezing -> reorder
  attend  mkv_mixed_kv_decode_attention   one decode query per (sequence, head)

Inputs are resident in HBM before timing starts.  The routing of the
synthetic hidden states is the same in every step, so no call depends on
another call of the same step.  The packed cache is kept in R copies
(R >= 4, >= 1 GiB in total): step i packs into copy i % R and attends over
copy (i + 1) % R, whose bytes are identical (same inputs, same deterministic
kernels) and were written R - 1 steps earlier, so the 256 MB last-level
cache cannot serve the attention read.  The router runs between the two so
that the 207 MB just written by the pack (a prefill-time write that a decode
step does not make) leaves the last-level cache while the router computes,
not while attention reads.

Prints one JSON line.  value = decode-attention effective GB/s (packed KV
bytes + q + out per launch / attention time); the quantize rate, router rate
and per-kernel times are reported beside it, and so is the time of the
alternative selector (mkv_select_chunks_by_similarity: chunk bitwidths from
the similarity to a query embedding) over the same hidden states, timed on
its own after the steps.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FP16_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 MFMA, published


def parse():
    from chunk_mixed_precision_amd import configs
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=configs.LLAMA2_7B_32K.name, choices=[w.name for w in configs.ALL])
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the oracle timing on the host (0 disables it)")
    ap.add_argument("--routing-ablation", type=int, default=0, metavar="L",
                    help="also time L-layer steps with routing sharing (one route, L x quantize + attend) "
                         "and without it (every layer routes its own hidden states)")
    ap.add_argument("--prefill-chunk", type=int, default=256, metavar="P",
                    help="also time chunked-prefill attention of P new tokens per sequence over the same "
                         "cache (0 disables)")
    ap.add_argument("--decode-steps", type=int, default=0, metavar="N",
                    help="also time N streaming-decode steps (one token per sequence, full chunks routed, "
                         "quantized and appended) on the grouped-query workload")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before timing, run one device-to-device copy of this many MiB (a known-size "
                         "kernel that calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
ATTN_SOURCES = ("chunk_mixed_precision_amd/csrc/attn.hip", "chunk_mixed_precision_amd/csrc/mkv_kernels.h",
                "chunk_mixed_precision_amd/csrc/mkv_internal.h")


def attention_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per attention call from committed rocprofv3 FETCH_SIZE and
    WRITE_SIZE counts (scaled by the counts of a known-size copy), or None if
    none were taken for this workload or the attention sources changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("attention_source_sha256") != attention_source_hash():
        return None
    return rec


def cpu_baseline(w, k, v, q, tab_bits, budget_s):
    """The CPU oracle (as it stands) on a bounded sample of the same workload:
    whole (sequence 0, KV head h) slices, quantized then attended, one thread,
    head after head (starting over at head 0) until the time budget is spent."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from chunk_mixed_precision_amd import configs
    from oracle import mkv_oracle as orc

    bits_row = tab_bits[0]
    g = w.Hq // w.Hkv
    t_quant = t_attn = 0.0
    nbytes = 0
    heads = 0
    tokens = 0
    passes = 0
    with threadpool_limits(limits=1):
        for i in range(1 << 30):
            h = i % w.Hkv
            passes += h == 0
            kk = k[0, h].cpu().numpy()
            vv = v[0, h].cpu().numpy()
            qq = q[0, h * g:(h + 1) * g].cpu().numpy()
            t0 = time.perf_counter()
            chunks = [orc.quantize_chunk(kk[c * w.C:(c + 1) * w.C], vv[c * w.C:(c + 1) * w.C], int(bits_row[c]))
                      for c in range(w.n)]
            t1 = time.perf_counter()
            deq = [orc.dequant_chunk(ch) for ch in chunks]
            kh = np.concatenate([d[0] for d in deq])
            vh = np.concatenate([d[1] for d in deq])
            for j in range(g):
                orc.attention(qq[j].astype(np.float64), kh, vh)
            t2 = time.perf_counter()
            t_quant += t1 - t0
            t_attn += t2 - t1
            nbytes += sum(configs.chunk_bytes(int(b), w.d, w.C) for b in bits_row[:w.n]) + g * w.d * 6
            tokens += w.T
            heads += 1
            if t_quant + t_attn >= budget_s:
                break
    return {
        "value": round(nbytes / t_attn / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": (f"sequence 0 of {w.name}, {heads} (sequence, KV head) slices in {passes} pass(es) over its "
                   f"{w.Hkv} KV heads: oracle dequant + fp64 attention over {w.T} tokens per head "
                   f"({t_attn:.1f} s); oracle quantize of the same slices {tokens / t_quant:.0f} tokens/s per "
                   f"head-slice ({t_quant:.1f} s); numpy, 1 thread"),
    }


def routing_ablation(w, L, steps, warmup):
    """Whole L-layer steps with and without routing sharing (MoQAE, Key
    designs).  Every layer has its own K/V, query, hidden states and router;
    with sharing, layer 0's tables serve every layer, without it each layer
    routes its own chunks and gets its own tables and pool capacities."""
    import numpy as np
    import torch
    from chunk_mixed_precision_amd import mkv, synth
    dev = "cuda"
    layers = []
    for l in range(L):
        x, w12, w3, b3 = synth.router_inputs(w, layer=l)
        k, v = synth.kv(w, dev, layer=l)
        layers.append({"x": x.to(dev), "w12": w12.to(dev), "w3": w3.to(dev), "b3": b3.to(dev),
                       "k": k, "v": v, "q": synth.query(w, dev, layer=l),
                       "tab": mkv.RouteTables(w.B, w.n, dev)})
        del x
    ws_route = torch.empty(mkv.workspace_bytes_route(w.B, w.T, w.D, w.I), dtype=torch.uint8, device=dev)
    for ly in layers:
        mkv.route_chunks(ly["tab"], w.C, x=ly["x"], w12=ly["w12"], w3=ly["w3"], b3=ly["b3"], workspace=ws_route)
    torch.cuda.synchronize()

    def caches_for(tabs):
        out = []
        for tab in tabs:
            seg = tab.seg_count.cpu().numpy()
            caps = [int(seg[:, kk].max()) for kk in range(3)]
            c = mkv.PackedCache(w.B, w.Hkv, w.d, w.C, caps, tab.seg_count, dev)
            out.append((c, mkv.attention_workspace(w.B, w.Hq, c, dev)))
        return out

    res = {"layers": L}
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    for mode in ("shared", "per_layer"):
        tabs = [layers[0]["tab"]] * L if mode == "shared" else [ly["tab"] for ly in layers]
        cw = caches_for(tabs)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]

        def step(i, rec):
            if rec:
                ev[i][0].record()
            for l, ly in enumerate(layers):
                if mode == "per_layer" or l == 0:
                    mkv.route_chunks(tabs[l], w.C, x=ly["x"], w12=ly["w12"], w3=ly["w3"], b3=ly["b3"],
                                     workspace=ws_route)
                mkv.quantize_pack_kv(ly["k"], ly["v"], tabs[l], cw[l][0])
                mkv.mixed_kv_decode_attention(ly["q"], cw[l][0], out=out, workspace=cw[l][1])
            if rec:
                ev[i][1].record()

        for i in range(warmup):
            step(i, False)
        torch.cuda.synchronize()
        for i in range(steps):
            step(i, True)
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in ev])
        res[mode] = {"ms_per_step": round(float(t.mean()), 4),
                     "chunk_mix_per_layer": [[int(s) for s in tb.seg_count.cpu().numpy().sum(0)] for tb in tabs]}
        del cw
    res["per_layer_over_shared"] = round(res["per_layer"]["ms_per_step"] / res["shared"]["ms_per_step"], 4)
    return res


def streaming_decode(steps: int):
    """Streaming decode on the llama3-8b GQA shape: the 8192-token prefill
    (drawn chunk mix) in the packed cache, then `steps` steps of one token
    per sequence into the fp16 tail; every C-th step routes, quantizes and
    appends the completed chunk (the router on the chunk's hidden states)."""
    import numpy as np
    import torch
    from chunk_mixed_precision_amd import configs, decode, synth
    dev = "cuda"
    w = configs.BY_NAME["llama3-8b-gqa-B64-T8192+256-C256"]
    _, w12, w3, b3 = synth.router_inputs(w, tokens_per_seq=w.C, batch=1)
    k, v = synth.kv(w, dev)
    logits = synth.one_hot_logits(synth.drawn_chunk_experts(w), w.C).to(dev)
    n_max = w.n + (steps + w.C - 1) // w.C + 1
    sess = decode.DecodeSession(w.B, w.Hq, w.Hkv, w.d, w.C, 1, w12.to(dev), w3.to(dev), b3.to(dev),
                                max_chunks=n_max)
    sess.prefill(None, [(k, v)], logits=logits)
    del k, v, logits
    xs, ks, vs, qs = synth.decode_tokens(w, steps, dev)
    out = [torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)]
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    flush = []
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record()
        sess.step(xs[s], [(ks[s], vs[s])], [qs[s]], out=out)
        ev[s][1].record()
        flush.append(sess.tail_len == 0)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
    fl = np.array(flush)
    return {"workload": w.name, "layers": 1, "steps": steps, "prefill_tokens": w.T,
            "context_tokens_at_end": w.T + steps,
            "step_us": round(float(t[~fl].mean()), 2), "step_us_p90": round(float(np.percentile(t[~fl], 90)), 2),
            "flush_step_us": None if not fl.any() else round(float(t[fl].mean()), 2),
            "flushes": int(fl.sum()), "pool_relayouts": sess.grown,
            "decode_tokens_per_s": round(w.B * steps / wall, 1)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(pass --gpus 1; sharding is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from chunk_mixed_precision_amd import configs, mkv, synth

    w = configs.BY_NAME[args.workload]
    if not w.routed or w.append_chunks or w.layers != 1:
        print(f"bench.py times the single-layer routed workloads; {w.name} is a parity-test case",
              file=sys.stderr)
        sys.exit(2)
    dev = "cuda"
    torch.cuda.set_device(0)
    mkv.lib()

    # ---------------- inputs, resident in HBM
    x, w12, w3, b3 = synth.router_inputs(w)
    x, w12, w3, b3 = x.to(dev), w12.to(dev), w3.to(dev), b3.to(dev)
    k, v = synth.kv(w, dev)
    q = synth.query(w, dev)
    tab = mkv.RouteTables(w.B, w.n, dev)
    ws_route = torch.empty(mkv.workspace_bytes_route(w.B, w.T, w.D, w.I), dtype=torch.uint8, device=dev)
    mkv.route_chunks(tab, w.C, x=x, w12=w12, w3=w3, b3=b3, workspace=ws_route)
    torch.cuda.synchronize()
    seg = tab.seg_count.cpu().numpy()
    caps = [int(seg[:, kk].max()) for kk in range(3)]
    one = mkv.PackedCache(w.B, w.Hkv, w.d, w.C, caps, tab.seg_count, dev)
    cache_bytes = one.nbytes()
    R = max(4, math.ceil((1 << 30) / cache_bytes))
    caches = [one] + [mkv.PackedCache(w.B, w.Hkv, w.d, w.C, caps, tab.seg_count, dev) for _ in range(R - 1)]
    for c in caches:
        mkv.quantize_pack_kv(k, v, tab, c)
    ws_attn = mkv.attention_workspace(w.B, w.Hq, one, dev)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()

    nev = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nev)]

    # one step in the order of the data flow: route and vote, quantize/pack with that routing,
    # then decode attention.  Attention reads the cache copy written R - 1 steps earlier, so the
    # bytes quantize has just written cannot serve it from the last-level cache.
    def step(i, rec):
        e = ev[i] if rec else None
        if e:
            e[0].record()
        mkv.route_chunks(tab, w.C, x=x, w12=w12, w3=w3, b3=b3, workspace=ws_route)
        if e:
            e[1].record()
        mkv.quantize_pack_kv(k, v, tab, caches[i % R])
        if e:
            e[2].record()
        mkv.mixed_kv_decode_attention(q, caches[(i + 1) % R], out=out, workspace=ws_attn)
        if e:
            e[3].record()

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the alternative selector (similarity to a query embedding) on the same hidden states
    qe = synth.query_embedding(w).to(dev)
    tab_sim = mkv.RouteTables(w.B, w.n, dev)
    ws_sim = torch.empty(mkv.workspace_bytes_similarity(w.B, w.T, w.D, w.C), dtype=torch.uint8, device=dev)
    for _ in range(3):
        mkv.select_chunks_by_similarity(tab_sim, w.C, x, qe, 0.3, 0.0, workspace=ws_sim)
    ev_sim = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nev)]
    for i in range(nev):
        ev_sim[i][0].record()
        mkv.select_chunks_by_similarity(tab_sim, w.C, x, qe, 0.3, 0.0, workspace=ws_sim)
        ev_sim[i][1].record()
    torch.cuda.synchronize()
    t_sim = np.array([a.elapsed_time(b) for a, b in ev_sim]) * 1e-3
    sim_bytes = w.B * w.T * w.D * 2 + w.B * w.D * 2 + w.B * w.n * (1 + 4 + 4)

    # chunked prefill: P new tokens per sequence attend over the same caches (rotated) and causally
    # over themselves, on the matrix cores
    pre = None
    if args.prefill_chunk > 0:
        Pn = args.prefill_chunk
        gq = torch.Generator(device=dev)
        gq.manual_seed(w.seed * 100 + 55)
        pq = torch.randn((w.B, w.Hq, Pn, w.d), generator=gq, device=dev).to(torch.float16)
        pkn = torch.randn((w.B, w.Hkv, Pn, w.d), generator=gq, device=dev).to(torch.float16)
        pvn = torch.randn((w.B, w.Hkv, Pn, w.d), generator=gq, device=dev).to(torch.float16)
        pout = torch.empty((w.B, w.Hq, Pn, w.d), dtype=torch.float32, device=dev)
        pws = torch.empty(mkv.workspace_bytes_prefill(w.B, w.Hq, Pn, w.d, w.C, caps), dtype=torch.uint8, device=dev)
        for i in range(3):
            mkv.mixed_kv_prefill_attention(pq, caches[i % R], pkn, pvn, out=pout, workspace=pws)
        ev_pre = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nev)]
        for i in range(nev):
            ev_pre[i][0].record()
            mkv.mixed_kv_prefill_attention(pq, caches[i % R], pkn, pvn, out=pout, workspace=pws)
            ev_pre[i][1].record()
        torch.cuda.synchronize()
        t_pre = float(np.mean([a.elapsed_time(b) for a, b in ev_pre])) * 1e-3
        ctx = w.T
        pre_flop = 4.0 * w.B * w.Hq * Pn * w.d * (ctx + (Pn + 1) / 2.0)
        pre_bytes = (configs.effective_attention_bytes(w, seg) - w.B * w.Hq * w.d * 6
                     + w.B * w.Hq * Pn * w.d * (2 + 4) + 2 * w.B * w.Hkv * Pn * w.d * 2)
        pre = {"P": Pn, "us": round(t_pre * 1e6, 2),
               "roofline": {"bound": "mfma", "achieved": round(pre_flop / t_pre / 1e12, 2),
                            "peak": FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(pre_flop / t_pre / 1e12 / FP16_PEAK_TFLOPS, 4),
                            "flop_per_launch": pre_flop},
               "effective_gbs": round(pre_bytes / t_pre / 1e9, 1), "bytes_per_launch": pre_bytes}
        del pq, pkn, pvn, pout, pws

    # a plain device-to-device copy on the same box, for scale: bytes read + written per second
    cp_bytes = 512 << 20
    csrc = torch.ones(cp_bytes, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    for _ in range(3):
        cdst.copy_(csrc)
    ev_cp = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for a, b in ev_cp:
        a.record()
        cdst.copy_(csrc)
        b.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * cp_bytes / (float(np.median([a.elapsed_time(b) for a, b in ev_cp])) * 1e-3) / 1e9
    del csrc, cdst

    t_route = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(nev)]) * 1e-3
    t_pack = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(nev)]) * 1e-3
    t_attn = np.array([ev[i][2].elapsed_time(ev[i][3]) for i in range(nev)]) * 1e-3

    attn_bytes = configs.effective_attention_bytes(w, seg)
    traffic = measured_traffic(w.name)
    pack_read = w.B * w.Hkv * w.T * w.d * 2 * 2
    pack_write = sum(int(seg[b, kk]) * configs.chunk_bytes(bits, w.d, w.C) * w.Hkv
                     for b in range(w.B) for kk, bits in enumerate(configs.EXPERT_BITS))
    router_flop = 2.0 * w.B * w.T * w.D * 2 * w.I + 2.0 * w.B * w.T * w.I * 3
    a_mean = float(t_attn.mean())
    attn_gbs = attn_bytes / a_mean / 1e9
    avg_bits = float(sum(seg[:, kk].sum() * bits for kk, bits in enumerate(configs.EXPERT_BITS)) / seg.sum())

    res = {
        "metric": "mixed-KV decode attention effective HBM GB/s (% of peak) + quantize tokens/s",
        "value": round(attn_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic (seeded), random-init router",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
                   "context": w.T, "chunk": w.C, "router_hidden": w.D, "router_inner": w.I,
                   "chunk_mix": [int(s) for s in seg.sum(0)], "avg_bits": round(avg_bits, 3),
                   "cache_copies": R},
        "roofline": {"bound": "hbm", "achieved": round(attn_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_call"],
                     "kernel": "mkv_mixed_kv_decode_attention call (attn_tile_kernel + attn_combine_kernel)",
                     "bytes_per_launch": attn_bytes, "avg_launch_us": round(a_mean * 1e6, 3)},
        "quantize_tokens_per_s": round(w.B * w.T / float(t_pack.mean()), 1),
        "device_copy": {"gbs": round(copy_gbs, 1), "bytes_moved": 2 * cp_bytes,
                        "attention_frac_of_copy": round(attn_gbs / copy_gbs, 4)},
        "kernels": {
            "route": {"us": round(float(t_route.mean()) * 1e6, 2),
                      "roofline": {"bound": "mfma", "achieved": round(router_flop / float(t_route.mean()) / 1e12, 2),
                                   "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                   "frac": round(router_flop / float(t_route.mean()) / 1e12 / BF16_PEAK_TFLOPS, 4),
                                   "flop_per_launch": router_flop}},
            "pack": {"us": round(float(t_pack.mean()) * 1e6, 2),
                     "roofline": {"bound": "hbm", "achieved": round((pack_read + pack_write) / float(t_pack.mean()) / 1e9, 2),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round((pack_read + pack_write) / float(t_pack.mean()) / 1e9 / HBM_PEAK_GBS, 4),
                                  "bytes_per_launch": pack_read + pack_write}},
            "select_similarity": {
                "us": round(float(t_sim.mean()) * 1e6, 2),
                "roofline": {"bound": "hbm", "achieved": round(sim_bytes / float(t_sim.mean()) / 1e9, 2),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(sim_bytes / float(t_sim.mean()) / 1e9 / HBM_PEAK_GBS, 4),
                             "bytes_per_launch": sim_bytes}},
            "prefill_attend": pre,
            "attend": {"us": round(a_mean * 1e6, 2), "us_p10": round(float(np.percentile(t_attn, 10)) * 1e6, 2),
                       "us_p90": round(float(np.percentile(t_attn, 90)) * 1e6, 2), "bytes": attn_bytes,
                       "traffic": None if traffic is None else {
                           "bytes_per_call": traffic["bytes_per_call"],
                           "ratio_to_algorithmic": traffic["ratio_to_algorithmic"],
                           "fetch_factor": traffic["calibration"]["fetch_factor"],
                           "write_factor": traffic["calibration"]["write_factor"],
                           "source": "profiles/pmc_traffic.json"}},
        },
    }
    if args.routing_ablation > 0:
        del caches, x
        torch.cuda.empty_cache()
        res["routing_ablation"] = routing_ablation(w, args.routing_ablation, max(3, args.steps // 4), 2)
    if args.decode_steps > 0:
        res["streaming_decode"] = streaming_decode(args.decode_steps)
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(w, k, v, q, tab.chunk_bits.cpu().numpy(), args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
