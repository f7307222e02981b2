"""CPU checks of bench.py's host-side logic: the oracle timing harness
(worker pool, shared-memory slices, the worker-count scan) runs on a small
stand-in workload, reports its fields, and leaves no shared-memory block
behind.  No GPU is touched."""
import os

import numpy as np
import pytest

import bench
from chunk_mixed_precision_amd import configs


class _SmallWorkload:
    """Slices shaped like the 13B workload's, at 1024 tokens per head."""

    def __init__(self):
        self.w = configs.scaled(configs.LLAMA2_13B_40L, T=1024)
        self.slice_desc = "stand-in slices of 1024 tokens"

    def cpu_slices(self):
        rng = np.random.default_rng(0)
        w = self.w
        bits = np.array([16, 4, 4, 2, 4, 4, 2, 4], np.uint8)
        while True:
            k = rng.standard_normal((w.T, w.d)).astype(np.float16)
            v = rng.standard_normal((w.T, w.d)).astype(np.float16)
            q = rng.standard_normal((1, w.d)).astype(np.float16)
            yield k, v, q, bits, w.C, w.d

    def cpu_router_blocks(self):
        rng = np.random.default_rng(1)
        D, I = 128, 128
        xb = (rng.standard_normal((256, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        wb = (rng.standard_normal((2 * I, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        w3 = rng.standard_normal((3, I))
        b3 = np.zeros(3)
        return [(xb, wb, w3, b3, I)] * 2, 256 * (2.0 * D * 2 * I + 2.0 * I * 3)


def _shm_names():
    """Shared-memory blocks (Python names them psm_*); the pool's own named
    semaphores are left out."""
    if not os.path.isdir("/dev/shm"):
        return set()
    return {n for n in os.listdir("/dev/shm") if n.startswith("psm_")}


def test_cpu_baseline_harness_runs_and_cleans_up():
    before = _shm_names()
    pool, ncores = bench.make_cpu_pool()
    try:
        res = bench.cpu_baseline(pool, ncores, _SmallWorkload(), 1.0)
    finally:
        pool.close()
        pool.join()
    assert res["kind"] == "oracle" and res["unit"] == "GB/s"
    assert 1 <= res["cores"] <= min(16, os.cpu_count() or 1)
    assert res["value"] > 0 and res["one_thread_value"] > 0
    assert res["quantize_tokens_per_s"] > 0 and res["router_tflops"] > 0
    assert res["cpu_model"]
    assert set(res["slices_per_s_by_workers"]) >= {1}
    assert "slices" in res["sample"]
    assert _shm_names() <= before, "shared-memory blocks left behind"


def test_cpu_threads_is_bounded():
    assert 1 <= bench._cpu_threads() <= 16
