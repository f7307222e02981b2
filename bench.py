#!/usr/bin/env python3
"""Throughput of the chunk-adaptive mixed-precision KV path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
of the named workload:
  route   mkv_route_chunks       router GEMM (bf16 MFMA) -> vote -> freezing -> reorder
                                 (for the drawn-mix 40-layer shape: vote and reorder of
                                 per-token scores, no router GEMM)
  pack    mkv_quantize_pack_kv   K/V of the routed chunks -> packed FP16/INT4/INT2
                                 segments, once per layer
  attend  mkv_mixed_kv_decode_attention   one decode query per (sequence, query
                                 head), once per layer

The default workload is the largest one that fits one GPU: the llama2-13b
shape, 40 layers under one shared routing (16 sequences x 8192 tokens, 40
heads, chunk 128), one decode token per sequence through all 40 layers.
The llama2-7b layers at 32k and 128k tokens and the llama3-8b GQA append
step can be named with --workload.

Inputs are resident in HBM before timing starts, and no attention read can
be served by the 256 MB last-level cache (see each workload class).

Prints one JSON line.  value = decode-attention effective GB/s: the packed
KV + q + out bytes of one layer's attention call divided by that call's
average time (HIP events around the step's attention calls, launch gaps
included).  The quantize rate, the router rate and the chunked-prefill and
similarity-selection times are reported beside it, and so is the oracle on
the host's cores (cpu_baseline).
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
    ap.add_argument("--workload", default=configs.LLAMA2_13B_40L.name,
                    choices=[w.name for w in configs.ALL if w is not configs.TINY])
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the oracle timing on the host (0 disables it)")
    ap.add_argument("--routing-ablation", type=int, default=0, metavar="L",
                    help="also time L-layer steps with routing sharing (one route, L x quantize + attend) "
                         "and without it (every layer routes its own hidden states)")
    ap.add_argument("--prefill-chunk", type=int, default=-1, metavar="P",
                    help="also time chunked-prefill attention of P new tokens per sequence over the (first "
                         "layer's) cache (default: one chunk; 0 disables)")
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


# ---------------------------------------------------------------- CPU baseline (the oracle)
def _cpu_threads() -> int:
    """Host cores this process may use: its CPU affinity, bounded by the
    cgroup CPU quota where one is set, and capped at 16 (one GPU's share of
    a shared box)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    for path in ("/sys/fs/cgroup/cpu.max", "/sys/fs/cgroup/cpu/cpu.cfs_quota_us"):
        try:
            with open(path) as f:
                parts = f.read().split()
            if path.endswith("cpu.max"):
                if parts[0] != "max":
                    n = min(n, max(1, int(int(parts[0]) / int(parts[1]))))
            else:
                quota = int(parts[0])
                if quota > 0:
                    with open("/sys/fs/cgroup/cpu/cpu.cfs_period_us") as f:
                        n = min(n, max(1, quota // int(f.read().split()[0])))
            break
        except (OSError, ValueError, IndexError):
            continue
    return max(1, min(16, n))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _pool_init():
    """Runs once in each worker at start: loads numpy and the oracle and
    takes one tiny chunk through them, so that no timed task pays a
    worker's first-call costs."""
    import numpy as np
    from multiprocessing import resource_tracker
    from threadpoolctl import threadpool_limits
    from oracle import mkv_oracle as orc
    globals()["_TPL"] = threadpool_limits(limits=1)     # one BLAS thread per worker process
    # Workers only attach the bench process's shared-memory blocks, which
    # that process creates and unlinks.  Attaching would register a block
    # with the resource tracker the workers share with it as if the worker
    # owned it, so shared-memory entries stay out of the tracker here.
    reg, unreg = resource_tracker.register, resource_tracker.unregister
    resource_tracker.register = lambda name, rtype: None if rtype == "shared_memory" else reg(name, rtype)
    resource_tracker.unregister = lambda name, rtype: None if rtype == "shared_memory" else unreg(name, rtype)
    rng = np.random.default_rng(0)
    k = rng.standard_normal((32, 64)).astype(np.float16)
    v = rng.standard_normal((32, 64)).astype(np.float16)
    kh, vh = orc.dequant_chunk(orc.quantize_chunk(k, v, 4))
    orc.attention(rng.standard_normal(64), kh, vh)


def _oracle_slice(args):
    """One (sequence, layer, KV head) slice through the oracle: quantize and
    pack every chunk at its bitwidth, dequantize, and attend with each query
    head of the GQA group.  The slice's arrays are read from a shared-memory
    block (name, then (offset, shape, dtype) of k, v, q and the chunk
    bitwidths).  Returns (quantize s, attention s, algorithmic attention
    bytes, tokens)."""
    import numpy as np
    from multiprocessing import shared_memory
    from chunk_mixed_precision_amd import configs
    from oracle import mkv_oracle as orc
    name, parts, C, d = args
    shm = shared_memory.SharedMemory(name=name)    # attached only: the bench process unlinks it
    try:
        kk, vv, qq, bits_row = (np.ndarray(shape, dtype=np.dtype(dt), buffer=shm.buf, offset=off)
                                for off, shape, dt in parts)
        n = len(bits_row)
        t0 = time.perf_counter()
        chunks = [orc.quantize_chunk(kk[c * C:(c + 1) * C], vv[c * C:(c + 1) * C], int(bits_row[c]))
                  for c in range(n)]
        t1 = time.perf_counter()
        deq = [orc.dequant_chunk(ch) for ch in chunks]
        kh = np.concatenate([x[0] for x in deq])
        vh = np.concatenate([x[1] for x in deq])
        for j in range(qq.shape[0]):
            orc.attention(qq[j].astype(np.float64), kh, vh)
        t2 = time.perf_counter()
        nbytes = sum(configs.chunk_bytes(int(b), d, C) for b in bits_row) + qq.shape[0] * d * 6
        del kk, vv, qq, bits_row, chunks, deq, kh, vh
    finally:
        shm.close()
    return t1 - t0, t2 - t1, nbytes, n * C


def _share_slices(slices):
    """Copy (k, v, q, bits, C, d) slices into one shared-memory block; returns
    the block and one task argument per slice."""
    shm, parts = _share_arrays([sl[:4] for sl in slices])
    return shm, [(shm.name, p, sl[4], sl[5]) for p, sl in zip(parts, slices)]


def _oracle_router(args):
    """Oracle router logits (float64) for a block of tokens; returns seconds.
    The block's bf16 hidden states, W12, W3 and b3 are read from a
    shared-memory block (name, then their (offset, shape, dtype))."""
    import numpy as np
    from multiprocessing import shared_memory
    from oracle import mkv_oracle as orc
    name, parts, inner = args
    shm = shared_memory.SharedMemory(name=name)    # attached only: the bench process unlinks it
    try:
        xb, w12b, w3, b3 = (np.ndarray(shape, dtype=np.dtype(dt), buffer=shm.buf, offset=off)
                            for off, shape, dt in parts)
        t0 = time.perf_counter()
        orc.router_logits(orc.bf16_bits_to_f64(xb), orc.bf16_bits_to_f64(w12b), w3, b3, inner)
        dt = time.perf_counter() - t0
        del xb, w12b, w3, b3
    finally:
        shm.close()
    return dt


def _share_arrays(groups):
    """Copy groups of arrays into one shared-memory block; returns the block
    and, per group, the (offset, shape, dtype) of its arrays."""
    import numpy as np
    from multiprocessing import shared_memory
    total = sum(a.nbytes + 64 for g in groups for a in g)
    shm = shared_memory.SharedMemory(create=True, size=max(total, 1))
    out = []
    off = 0
    for g in groups:
        parts = []
        for a in g:
            a = np.ascontiguousarray(a)
            np.ndarray(a.shape, dtype=a.dtype, buffer=shm.buf, offset=off)[...] = a
            parts.append((off, a.shape, a.dtype.str))
            off += (a.nbytes + 63) // 64 * 64
        out.append(tuple(parts))
    return shm, out


def make_cpu_pool():
    """Worker processes for the oracle timing, started before this process
    touches the GPU.  They are spawned (a fresh interpreter each) with every
    BLAS/OpenMP thread count set to 1 in their environment, so that each
    worker computes on one thread from its first numpy call, whatever
    threading the host's numpy would otherwise set up."""
    import multiprocessing as mp
    n = _cpu_threads()
    keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS",
            "NUMEXPR_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in keys}
    os.environ.update({k: "1" for k in keys})
    try:
        pool = mp.get_context("spawn").Pool(n, initializer=_pool_init)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return pool, n


def cpu_baseline(pool, ncores, wl, budget_s):
    """The CPU oracle (as it stands) on a bounded sample of the same
    workload: whole (sequence, layer, KV head) slices of the bench's own
    inputs, quantized then attended, each in one worker process with one
    numpy thread.  Every worker first takes one slice untimed; one slice
    then runs alone three times (the fastest gives the one-thread figures).
    Waves of 2, 4, ... slices then run side by side to find how many
    workers the host actually gives this process (the CPU share of a shared
    box need not show in its affinity mask), and the rest of the budget of
    about `budget_s` seconds of task time runs at the fastest width.  The
    slices are copied to a shared-memory block before any timing (a task
    passes only its offsets); every width is timed by the wall clock around
    its wave.  For routed workloads the oracle router also runs on blocks of
    256 tokens."""
    gen = wl.cpu_slices()
    shm, distinct = _share_slices([next(gen) for _ in range(min(wl.w.Hkv, 8))])   # on the host before any timing
    try:
        return _cpu_baseline_runs(pool, ncores, wl, budget_s, distinct)
    finally:
        shm.close()
        shm.unlink()


def _cpu_baseline_runs(pool, ncores, wl, budget_s, distinct):
    count = [0]

    def take(k):
        out = [distinct[(count[0] + j) % len(distinct)] for j in range(k)]
        count[0] += k
        return out

    def wave(k):
        t0 = time.perf_counter()
        res = pool.map(_oracle_slice, take(k), chunksize=1)
        return time.perf_counter() - t0, res

    wave(ncores)                                     # every worker runs one slice untimed
    solos = [wave(1) for _ in range(3)]              # one slice alone, the fastest of three
    w1, res1 = min(solos, key=lambda x: x[0])
    solo = res1[0]
    spent = sum(r[1][0][0] + r[1][0][1] for r in solos)
    scan = {1: round(1.0 / w1, 3)}
    best_k, best_rate = 1, 1.0 / w1
    k = 2
    while k <= ncores and spent < budget_s / 2:
        wall, res = wave(k)
        spent += sum(r[0] + r[1] for r in res)
        scan[k] = round(k / wall, 3)
        if k / wall > best_rate * 1.1:
            best_k, best_rate = k, k / wall
        k *= 2
    tq = ta = 0.0
    nbytes = tokens = 0
    wall = 0.0
    n = 0
    while n == 0 or (spent < budget_s and wall < budget_s):
        dt, res = wave(best_k)
        wall += dt
        tq += sum(r[0] for r in res)
        ta += sum(r[1] for r in res)
        spent += sum(r[0] + r[1] for r in res)
        nbytes += sum(r[2] for r in res)
        tokens += sum(r[3] for r in res)
        n += len(res)
    out = {
        "value": round(nbytes / (wall * ta / (tq + ta)) / 1e9, 4), "unit": "GB/s", "cores": best_k, "kind": "oracle",
        "one_thread_value": round(solo[2] / solo[1] / 1e9, 4),
        "cpu_model": _cpu_model(),
        "quantize_tokens_per_s": round(tokens / (wall * tq / (tq + ta)), 1),
        "quantize_tokens_per_s_one_thread": round(solo[3] / solo[0], 1),
        "slices_per_s_by_workers": scan,
    }
    sample = (f"{n} (sequence, layer, KV head) slices of {wl.w.name} ({wl.slice_desc}), each quantized "
              f"and packed by the oracle (numpy float32), dequantized and attended in float64 with its "
              f"{wl.w.group} query head(s); {best_k} worker process(es) side by side (the fastest of "
              f"1..{ncores} tried), one numpy thread each, {wall:.1f} s wall; value = attention bytes / the "
              f"attention share of the wall time; one-thread figures from the fastest of three runs of one "
              f"slice alone")
    rt = wl.cpu_router_blocks()
    if rt is not None:
        blocks, flop_per_block = rt
        blocks = blocks[:best_k]
        shm, parts = _share_arrays([b[:4] for b in blocks])
        try:
            tasks = [(shm.name, p, b[4]) for p, b in zip(parts, blocks)]
            solo_r = pool.apply(_oracle_router, (tasks[0],))
            t0 = time.perf_counter()
            pool.map(_oracle_router, tasks, chunksize=1)
            rwall = time.perf_counter() - t0
        finally:
            shm.close()
            shm.unlink()
        out["router_tflops"] = round(len(blocks) * flop_per_block / rwall / 1e12, 5)
        out["router_tflops_one_thread"] = round(flop_per_block / solo_r / 1e12, 5)
        sample += f"; router: {len(blocks)} blocks of 256 tokens in float64 side by side ({rwall:.1f} s wall)"
    out["sample"] = sample
    return out


# ---------------------------------------------------------------- workloads
class SingleLayerRouted:
    """One layer of a routed workload (llama2-7b at 32k or 128k tokens).  A
    step: route every token (router GEMM, vote, freezing, reorder), quantize
    and pack the whole prefill with that routing, then one decode attention
    call.  The packed cache is kept in R copies (R >= 4, >= 1 GiB): step i
    packs copy i % R and attends over copy (i + 1) % R, whose bytes are
    identical and were written R - 1 steps earlier, so the 256 MB last-level
    cache cannot serve the attention read."""

    layers = 1

    def __init__(self, w, dev):
        import torch
        from chunk_mixed_precision_amd import mkv, synth
        self.w = w
        x, w12, w3, b3 = synth.router_inputs(w)
        self.x_cpu_bits, self.w12_cpu_bits = x, w12
        self.x, self.w12, self.w3, self.b3 = x.to(dev), w12.to(dev), w3.to(dev), b3.to(dev)
        self.k, self.v = synth.kv(w, dev)
        self.q = synth.query(w, dev)
        self.tab = mkv.RouteTables(w.B, w.n, dev)
        self.ws_route = torch.empty(mkv.workspace_bytes_route(w.B, w.T, w.D, w.I), dtype=torch.uint8, device=dev)
        mkv.route_chunks(self.tab, w.C, x=self.x, w12=self.w12, w3=self.w3, b3=self.b3, workspace=self.ws_route)
        torch.cuda.synchronize()
        self.seg = self.tab.seg_count.cpu().numpy()
        self.caps = [int(self.seg[:, kk].max()) for kk in range(3)]
        one = mkv.PackedCache(w.B, w.Hkv, w.d, w.C, self.caps, self.tab.seg_count, dev)
        self.R = max(4, math.ceil((1 << 30) / one.nbytes()))
        self.caches = [one] + [mkv.PackedCache(w.B, w.Hkv, w.d, w.C, self.caps, self.tab.seg_count, dev)
                               for _ in range(self.R - 1)]
        for c in self.caches:
            mkv.quantize_pack_kv(self.k, self.v, self.tab, c)
        self.ws_attn = mkv.attention_workspace(w.B, w.Hq, one, dev)
        self.out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
        self.route_tokens = w.B * w.T
        self.pack_tokens = w.B * w.T
        self.slice_desc = f"sequence 0, {w.T} tokens per head"

    def step(self, i, e):
        from chunk_mixed_precision_amd import mkv
        w = self.w
        e and e[0].record()
        mkv.route_chunks(self.tab, w.C, x=self.x, w12=self.w12, w3=self.w3, b3=self.b3, workspace=self.ws_route)
        e and e[1].record()
        mkv.quantize_pack_kv(self.k, self.v, self.tab, self.caches[i % self.R])
        e and e[2].record()
        mkv.mixed_kv_decode_attention(self.q, self.caches[(i + 1) % self.R], out=self.out, workspace=self.ws_attn)
        e and e[3].record()

    def attention_cache(self):
        return self.caches[0]

    def cpu_slices(self):
        w = self.w
        bits = self.tab.chunk_bits.cpu().numpy()[0, :w.n]
        g = w.group
        for i in range(1 << 30):
            h = i % w.Hkv
            yield (self.k[0, h].cpu().numpy(), self.v[0, h].cpu().numpy(),
                   self.q[0, h * g:(h + 1) * g].cpu().numpy(), bits, w.C, w.d)

    def cpu_router_blocks(self):
        import numpy as np
        import torch
        w = self.w
        xb = self.x_cpu_bits.reshape(-1, w.D).view(torch.int16).numpy().view(np.uint16)
        wb = self.w12_cpu_bits.view(torch.int16).numpy().view(np.uint16)
        w3 = self.w3.cpu().numpy().astype(np.float64)
        b3 = self.b3.cpu().numpy().astype(np.float64)
        blocks = [(xb[j * 256:(j + 1) * 256], wb, w3, b3, w.I) for j in range(_cpu_threads())]
        return blocks, 256 * (2.0 * w.D * 2 * w.I + 2.0 * w.I * 3)


class MultiLayerShared:
    """The llama2-13b shape: 40 layers under one routing (routing sharing),
    each with its own K, V and query.  The chunk bitwidths are drawn per
    sequence (no router is run for this shape); a step votes and reorders
    them (logits-in route: each token's scores pick its chunk's drawn
    expert, then the chunk vote, freezing and the stable reorder), quantizes
    and packs every layer's prefill into that layer's cache, then runs one
    decode attention call per layer.  Attention of layer l reads the cache
    written 40 quantize calls and l attention calls earlier (40 GB of other
    traffic), which the 256 MB last-level cache cannot serve."""

    def __init__(self, w, dev):
        import torch
        from chunk_mixed_precision_amd import mkv, synth
        self.w = w
        self.layers = w.layers
        experts = synth.drawn_chunk_experts(w)
        self.logits = synth.one_hot_logits(experts, w.C).to(dev)
        self.tab = mkv.RouteTables(w.B, w.n, dev)
        mkv.route_chunks(self.tab, w.C, logits=self.logits, logits_in=True)
        torch.cuda.synchronize()
        self.seg = self.tab.seg_count.cpu().numpy()
        self.caps = [int(self.seg[:, kk].max()) for kk in range(3)]
        self.kv = []
        self.q = []
        self.caches = []
        for l in range(w.layers):
            self.kv.append(synth.kv(w, dev, layer=l))
            self.q.append(synth.query(w, dev, layer=l))
            self.caches.append(mkv.PackedCache(w.B, w.Hkv, w.d, w.C, self.caps, self.tab.seg_count, dev))
            mkv.quantize_pack_kv(self.kv[l][0], self.kv[l][1], self.tab, self.caches[l])
        self.R = 1
        self.ws_attn = mkv.attention_workspace(w.B, w.Hq, self.caches[0], dev)
        self.out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
        self.route_tokens = w.B * w.T
        self.pack_tokens = w.B * w.T
        self.slice_desc = f"sequence 0 of layer 0, {w.T} tokens per head"

    def step(self, i, e):
        from chunk_mixed_precision_amd import mkv
        w = self.w
        e and e[0].record()
        mkv.route_chunks(self.tab, w.C, logits=self.logits, logits_in=True)
        e and e[1].record()
        for l in range(self.layers):
            mkv.quantize_pack_kv(self.kv[l][0], self.kv[l][1], self.tab, self.caches[l])
        e and e[2].record()
        for l in range(self.layers):
            mkv.mixed_kv_decode_attention(self.q[l], self.caches[l], out=self.out, workspace=self.ws_attn)
        e and e[3].record()

    def attention_cache(self):
        return self.caches[0]

    def cpu_slices(self):
        w = self.w
        bits = self.tab.chunk_bits.cpu().numpy()[0, :w.n]
        k, v = self.kv[0]
        for i in range(1 << 30):
            h = i % w.Hkv
            yield (k[0, h].cpu().numpy(), v[0, h].cpu().numpy(), self.q[0][0, h:h + 1].cpu().numpy(), bits,
                   w.C, w.d)

    def cpu_router_blocks(self):
        return None


class AppendStep:
    """The llama3-8b GQA shape: 64 sequences with 8192 tokens prefilled
    (drawn chunk mix, chunk 0 FP16), and per step one new 256-token chunk
    per sequence: route its 16384 tokens (router GEMM, vote and reorder of
    all 33 chunks, append mode), quantize and pack it into its segment
    (slot of chunk 32, rewritten every step, so the state stays the same),
    then decode attention over 8448 tokens (32 query heads over 8 KV heads).
    The cache is kept in R copies (>= 1 GiB), rotated as for one layer."""

    layers = 1

    def __init__(self, w, dev):
        import torch
        from chunk_mixed_precision_amd import mkv, synth
        self.w = w
        experts = synth.drawn_chunk_experts(w)
        experts[:, 0] = 0
        self.tab = mkv.RouteTables(w.B, w.n_total, dev)
        mkv.route_chunks(self.tab, w.C, logits=synth.one_hot_logits(experts, w.C).to(dev), logits_in=True)
        x, w12, w3, b3 = synth.router_inputs(w, tokens_per_seq=w.C, chunk_offset=w.n)
        self.x_cpu_bits, self.w12_cpu_bits = x, w12
        self.x, self.w12, self.w3, self.b3 = x.to(dev), w12.to(dev), w3.to(dev), b3.to(dev)
        self.ws_route = torch.empty(mkv.workspace_bytes_route(w.B, w.C, w.D, w.I), dtype=torch.uint8, device=dev)
        mkv.route_chunks(self.tab, w.C, x=self.x, w12=self.w12, w3=self.w3, b3=self.b3, workspace=self.ws_route,
                         append=True, chunk_offset=w.n)
        torch.cuda.synchronize()
        self.seg = self.tab.seg_count.cpu().numpy()
        self.caps = [int(self.seg[:, kk].max()) for kk in range(3)]
        k, v = synth.kv(w, dev)
        self.ka, self.va = synth.kv(w, dev, tokens=w.C, token_offset_stream=1)
        self.q = synth.query(w, dev)
        one = mkv.PackedCache(w.B, w.Hkv, w.d, w.C, self.caps, self.tab.seg_count, dev)
        self.R = max(4, math.ceil((1 << 30) / one.nbytes()))
        self.caches = [one] + [mkv.PackedCache(w.B, w.Hkv, w.d, w.C, self.caps, self.tab.seg_count, dev)
                               for _ in range(self.R - 1)]
        for c in self.caches:
            mkv.quantize_pack_kv(k, v, self.tab, c)
            mkv.quantize_pack_kv(self.ka, self.va, self.tab, c, chunk_offset=w.n)
        self.k_cpu_src = (k, v)
        self.ws_attn = mkv.attention_workspace(w.B, w.Hq, one, dev)
        self.out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
        self.route_tokens = w.B * w.C
        self.pack_tokens = w.B * w.C
        self.slice_desc = f"sequence 0, {w.T} prefilled tokens per KV head"

    def step(self, i, e):
        from chunk_mixed_precision_amd import mkv
        w = self.w
        e and e[0].record()
        mkv.route_chunks(self.tab, w.C, x=self.x, w12=self.w12, w3=self.w3, b3=self.b3, workspace=self.ws_route,
                         append=True, chunk_offset=w.n)
        e and e[1].record()
        mkv.quantize_pack_kv(self.ka, self.va, self.tab, self.caches[i % self.R], chunk_offset=w.n)
        e and e[2].record()
        mkv.mixed_kv_decode_attention(self.q, self.caches[(i + 1) % self.R], out=self.out, workspace=self.ws_attn)
        e and e[3].record()

    def attention_cache(self):
        return self.caches[0]

    def cpu_slices(self):
        w = self.w
        bits = self.tab.chunk_bits.cpu().numpy()[0, :w.n]
        k, v = self.k_cpu_src
        g = w.group
        for i in range(1 << 30):
            h = i % w.Hkv
            yield (k[0, h].cpu().numpy(), v[0, h].cpu().numpy(), self.q[0, h * g:(h + 1) * g].cpu().numpy(), bits,
                   w.C, w.d)

    def cpu_router_blocks(self):
        import numpy as np
        import torch
        w = self.w
        xb = self.x_cpu_bits.reshape(-1, w.D).view(torch.int16).numpy().view(np.uint16)
        wb = self.w12_cpu_bits.view(torch.int16).numpy().view(np.uint16)
        w3 = self.w3.cpu().numpy().astype(np.float64)
        b3 = self.b3.cpu().numpy().astype(np.float64)
        blocks = [(xb[j * 256:(j + 1) * 256], wb, w3, b3, w.I) for j in range(_cpu_threads())]
        return blocks, 256 * (2.0 * w.D * 2 * w.I + 2.0 * w.I * 3)


def make_workload(w, dev):
    if w.layers > 1:
        return MultiLayerShared(w, dev)
    if w.append_chunks:
        return AppendStep(w, dev)
    if w.routed:
        return SingleLayerRouted(w, dev)
    raise SystemExit(f"bench.py does not time {w.name}: it fits the last-level cache (a parity-test case)")


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
        print("bench.py measures one GPU: the library has no multi-GPU path; run it with --gpus 1 "
              "(each GPU would hold whole (sequence, KV head) streams of its own)", file=sys.stderr)
        sys.exit(2)

    # the oracle's worker processes start before anything touches the GPU
    pool, ncores = make_cpu_pool() if args.cpu_seconds > 0 else (None, 0)

    import numpy as np
    import torch

    from chunk_mixed_precision_amd import configs, mkv, synth

    w = configs.BY_NAME[args.workload]
    dev = "cuda"
    torch.cuda.set_device(0)
    mkv.lib()

    # ---------------- inputs, resident in HBM; tables and caches built once
    wl = make_workload(w, dev)
    seg, caps = wl.seg, wl.caps
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()

    nev = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nev)]
    for i in range(args.warmup):
        wl.step(i, None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        wl.step(i, ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    t_route = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(nev)]) * 1e-3
    t_pack = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(nev)]) * 1e-3
    t_attn = np.array([ev[i][2].elapsed_time(ev[i][3]) for i in range(nev)]) * 1e-3

    # the alternative selector (similarity to a query embedding) on the same hidden states
    sim = None
    if isinstance(wl, SingleLayerRouted):
        qe = synth.query_embedding(w).to(dev)
        tab_sim = mkv.RouteTables(w.B, w.n, dev)
        ws_sim = torch.empty(mkv.workspace_bytes_similarity(w.B, w.T, w.D, w.C), dtype=torch.uint8, device=dev)
        for _ in range(3):
            mkv.select_chunks_by_similarity(tab_sim, w.C, wl.x, qe, 0.3, 0.0, workspace=ws_sim)
        ev_sim = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nev)]
        for i in range(nev):
            ev_sim[i][0].record()
            mkv.select_chunks_by_similarity(tab_sim, w.C, wl.x, qe, 0.3, 0.0, workspace=ws_sim)
            ev_sim[i][1].record()
        torch.cuda.synchronize()
        t_sim = float(np.mean([a.elapsed_time(b) for a, b in ev_sim])) * 1e-3
        sim_bytes = w.B * w.T * w.D * 2 + w.B * w.D * 2 + w.B * w.n * (1 + 4 + 4)
        sim = {"us": round(t_sim * 1e6, 2),
               "roofline": {"bound": "hbm", "achieved": round(sim_bytes / t_sim / 1e9, 2), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(sim_bytes / t_sim / 1e9 / HBM_PEAK_GBS, 4),
                            "bytes_per_launch": sim_bytes}}
        del tab_sim, ws_sim

    # chunked prefill: P new tokens per sequence attend over the (first layer's) cache and causally over
    # themselves, on the matrix cores
    pre = None
    Pn = w.C if args.prefill_chunk < 0 else args.prefill_chunk
    if Pn > 0:
        cache0 = wl.attention_cache()
        gq = torch.Generator(device=dev)
        gq.manual_seed(w.seed * 100 + 55)
        pq = torch.randn((w.B, w.Hq, Pn, w.d), generator=gq, device=dev).to(torch.float16)
        pkn = torch.randn((w.B, w.Hkv, Pn, w.d), generator=gq, device=dev).to(torch.float16)
        pvn = torch.randn((w.B, w.Hkv, Pn, w.d), generator=gq, device=dev).to(torch.float16)
        pout = torch.empty((w.B, w.Hq, Pn, w.d), dtype=torch.float32, device=dev)
        pws = torch.empty(mkv.workspace_bytes_prefill(w.B, w.Hq, Pn, w.d, w.C, caps), dtype=torch.uint8, device=dev)
        for i in range(3):
            mkv.mixed_kv_prefill_attention(pq, cache0, pkn, pvn, out=pout, workspace=pws)
        npre = max(3, min(nev, 10))
        ev_pre = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(npre)]
        for i in range(npre):
            ev_pre[i][0].record()
            mkv.mixed_kv_prefill_attention(pq, cache0, pkn, pvn, out=pout, workspace=pws)
            ev_pre[i][1].record()
        torch.cuda.synchronize()
        t_pre = float(np.mean([a.elapsed_time(b) for a, b in ev_pre])) * 1e-3
        ctx = int(seg.sum(1).max()) * w.C
        pre_flop = 4.0 * w.Hq * Pn * w.d * (float(seg.sum(1).sum()) * w.C + w.B * (Pn + 1) / 2.0)
        pre_bytes = (configs.effective_attention_bytes(w, seg) - w.B * w.Hq * w.d * 6
                     + w.B * w.Hq * Pn * w.d * (2 + 4) + 2 * w.B * w.Hkv * Pn * w.d * 2)
        pre = {"P": Pn, "context": ctx, "us": round(t_pre * 1e6, 2),
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

    L = wl.layers
    attn_bytes = configs.effective_attention_bytes(w, seg)          # one layer's call
    traffic = measured_traffic(w.name)
    pack_tokens = wl.pack_tokens                                    # per layer and step
    pack_read = pack_tokens * w.Hkv * w.d * 2 * 2
    if isinstance(wl, AppendStep):
        new = wl.tab.chunk_bits.cpu().numpy()[:, w.n]
        pack_write = sum(configs.chunk_bytes(int(b), w.d, w.C) * w.Hkv for b in new)
    else:
        pack_write = sum(int(seg[b, kk]) * configs.chunk_bytes(bits, w.d, w.C) * w.Hkv
                         for b in range(w.B) for kk, bits in enumerate(configs.EXPERT_BITS))
    a_call = float(t_attn.mean()) / L                               # average duration of one layer's call
    attn_gbs = attn_bytes / a_call / 1e9
    p_call = float(t_pack.mean()) / L
    avg_bits = float(sum(seg[:, kk].sum() * bits for kk, bits in enumerate(configs.EXPERT_BITS)) / seg.sum())
    route = {"us": round(float(t_route.mean()) * 1e6, 2), "tokens": wl.route_tokens}
    if w.routed:
        router_flop = 2.0 * wl.route_tokens * w.D * 2 * w.I + 2.0 * wl.route_tokens * w.I * 3
        route["roofline"] = {"bound": "mfma", "achieved": round(router_flop / float(t_route.mean()) / 1e12, 2),
                             "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(router_flop / float(t_route.mean()) / 1e12 / BF16_PEAK_TFLOPS, 4),
                             "flop_per_launch": router_flop}
    else:
        route["note"] = ("drawn chunk mix: the route call votes and reorders per-token scores (logits-in), "
                         "no router GEMM")

    cfg = {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
           "context": int(seg.sum(1).max()) * w.C, "chunk": w.C, "layers": L,
           "chunk_mix": [int(x) for x in seg.sum(0)], "avg_bits": round(avg_bits, 3)}
    if w.routed:
        cfg.update(router_hidden=w.D, router_inner=w.I)
    if w.append_chunks:
        cfg["appended_chunks_per_step"] = w.append_chunks
    if wl.R > 1:
        cfg["cache_copies"] = wl.R

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
        "config": cfg,
        "roofline": {"bound": "hbm", "achieved": round(attn_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_call"],
                     "kernel": "mkv_mixed_kv_decode_attention call (attn_tile_kernel + attn_combine_kernel)",
                     "bytes_per_launch": attn_bytes, "launches_per_step": L,
                     "avg_launch_us": round(a_call * 1e6, 3)},
        "quantize_tokens_per_s": round(pack_tokens / p_call, 1),
        "device_copy": {"gbs": round(copy_gbs, 1), "bytes_moved": 2 * cp_bytes,
                        "attention_frac_of_copy": round(attn_gbs / copy_gbs, 4)},
        "kernels": {
            "route": route,
            "pack": {"us_per_layer": round(p_call * 1e6, 2), "layers": L,
                     "roofline": {"bound": "hbm", "achieved": round((pack_read + pack_write) / p_call / 1e9, 2),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round((pack_read + pack_write) / p_call / 1e9 / HBM_PEAK_GBS, 4),
                                  "bytes_per_launch": pack_read + pack_write}},
            "select_similarity": sim,
            "prefill_attend": pre,
            "attend": {"us_per_layer": round(a_call * 1e6, 2),
                       "us_per_step": round(float(t_attn.mean()) * 1e6, 2),
                       "us_per_step_p10": round(float(np.percentile(t_attn, 10)) * 1e6, 2),
                       "us_per_step_p90": round(float(np.percentile(t_attn, 90)) * 1e6, 2),
                       "bytes_per_layer": attn_bytes, "bytes_per_step": attn_bytes * L,
                       "traffic": None if traffic is None else {
                           "bytes_per_call": traffic["bytes_per_call"],
                           "ratio_to_algorithmic": traffic["ratio_to_algorithmic"],
                           "fetch_factor": traffic["calibration"]["fetch_factor"],
                           "write_factor": traffic["calibration"]["write_factor"],
                           "source": "profiles/pmc_traffic.json"}},
        },
    }
    if args.routing_ablation > 0:
        del wl
        torch.cuda.empty_cache()
        wa = w if (w.routed and w.layers == 1 and not w.append_chunks) else configs.LLAMA2_7B_32K
        res["routing_ablation"] = routing_ablation(wa, args.routing_ablation, max(3, args.steps // 4), 2)
        wl = None
    if args.decode_steps > 0:
        res["streaming_decode"] = streaming_decode(args.decode_steps)
    if pool is not None:
        if wl is None:
            wl = make_workload(w, dev)
        res["cpu_baseline"] = cpu_baseline(pool, ncores, wl, args.cpu_seconds)
        pool.close()
        pool.join()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
