"""CPU checks of the Python binding's argument checks: a tensor of the wrong
dtype, shape or device is refused before the library is asked to launch
anything.  The library's compute entry points are replaced by a stand-in
that fails the test if it is ever reached."""
import os

import pytest
import torch

from chunk_mixed_precision_amd import mkv

pytestmark = pytest.mark.skipif(not os.path.exists(mkv.LIB_PATH), reason="libmkv.so not built")

COMPUTE = ("mkv_route_chunks", "mkv_select_chunks_by_similarity", "mkv_quantize_pack_kv",
           "mkv_mixed_kv_decode_attention", "mkv_mixed_kv_prefill_attention", "mkv_append_tail_rows",
           "mkv_grow_pool")


class _NoLaunch:
    """The real library for sizing helpers; a failure for every call that
    would enqueue GPU work."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in COMPUTE:
            def reached(*a, **k):
                raise AssertionError(f"{name} was reached: the binding should have refused its arguments")
            return reached
        return getattr(self._real, name)


@pytest.fixture(autouse=True)
def no_launch(monkeypatch):
    real = mkv.lib()
    monkeypatch.setattr(mkv, "_lib", _NoLaunch(real))
    yield


B, Hq, Hkv, d, C, T = 2, 4, 2, 128, 128, 256


def tables(b=B, n=4):
    return mkv.RouteTables(b, n, "cpu")


def cache(b=B):
    t = tables(b)
    return mkv.PackedCache(b, Hkv, d, C, [1, 2, 1], t.seg_count, "cpu")


def f16(*shape):
    return torch.zeros(shape, dtype=torch.float16)


def test_attention_q_batch_must_match_cache():
    with pytest.raises(ValueError, match="q has shape"):
        mkv.mixed_kv_decode_attention(f16(B - 1, Hq, d), cache())


def test_attention_q_dtype_and_head_dim():
    with pytest.raises(TypeError, match="q must be torch.float16"):
        mkv.mixed_kv_decode_attention(torch.zeros((B, Hq, d)), cache())
    with pytest.raises(ValueError, match="q has shape"):
        mkv.mixed_kv_decode_attention(f16(B, Hq, 64), cache())


def test_attention_host_tensor_is_refused():
    with pytest.raises(ValueError, match="must be on the GPU"):
        mkv.mixed_kv_decode_attention(f16(B, Hq, d), cache())


def test_attention_out_and_tail_shapes():
    q = f16(B, Hq, d)
    with pytest.raises(ValueError, match="out has shape"):
        mkv.mixed_kv_decode_attention(q, cache(), out=torch.zeros((B, Hq + 1, d)))
    with pytest.raises(TypeError, match="out must be torch.float32"):
        mkv.mixed_kv_decode_attention(q, cache(), out=f16(B, Hq, d))
    with pytest.raises(ValueError, match="go together"):
        mkv.mixed_kv_decode_attention(q, cache(), tail_k=f16(B, Hkv, 8, d))
    with pytest.raises(ValueError, match="tail_v has shape"):
        mkv.mixed_kv_decode_attention(q, cache(), tail_k=f16(B, Hkv, 8, d), tail_v=f16(B, Hkv, 7, d))
    with pytest.raises(ValueError, match="tail_len"):
        mkv.mixed_kv_decode_attention(q, cache(), tail_k=f16(B, Hkv, 8, d), tail_v=f16(B, Hkv, 8, d),
                                      tail_len=9)


def test_attention_pool_smaller_than_its_capacity():
    c = cache()
    c.pools[1] = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match=r"cache.pools\[1\] holds"):
        mkv.mixed_kv_decode_attention(f16(B, Hq, d), c)


def test_attention_seg_count_shape():
    c = cache()
    c.seg_count = torch.zeros((B + 1, 3), dtype=torch.int32)
    with pytest.raises(ValueError, match="cache.seg_count has shape"):
        mkv.mixed_kv_decode_attention(f16(B, Hq, d), c)


def test_quantize_checks():
    k = f16(B, Hkv, T, d)
    with pytest.raises(TypeError, match="k must be torch.float16"):
        mkv.quantize_pack_kv(k.to(torch.bfloat16), k, tables(), cache())
    with pytest.raises(ValueError, match="k has shape"):
        mkv.quantize_pack_kv(f16(B, Hkv + 1, T, d), k, tables(), cache())
    with pytest.raises(ValueError, match="v has shape"):
        mkv.quantize_pack_kv(k, f16(B, Hkv, T - C, d), tables(), cache())
    with pytest.raises(ValueError, match="routing tables are for 1 sequences"):
        mkv.quantize_pack_kv(k, k, tables(1), cache())
    with pytest.raises(ValueError, match="must be on the GPU"):
        mkv.quantize_pack_kv(k, k, tables(), cache())


def test_route_checks():
    D, I = 256, 128
    x = torch.zeros((B, T, D), dtype=torch.bfloat16)
    w12 = torch.zeros((2 * I, D), dtype=torch.bfloat16)
    w3, b3 = torch.zeros((3, I)), torch.zeros(3)
    ws = torch.zeros(mkv.workspace_bytes_route(B, T, D, I), dtype=torch.uint8)
    with pytest.raises(ValueError, match="x has shape"):          # tables hold fewer rows than x
        mkv.route_chunks(tables(1), C, x=x, w12=w12, w3=w3, b3=b3, workspace=ws)
    with pytest.raises(TypeError, match="x must be torch.bfloat16"):
        mkv.route_chunks(tables(), C, x=x.float(), w12=w12, w3=w3, b3=b3, workspace=ws)
    with pytest.raises(ValueError, match="w12 has shape"):
        mkv.route_chunks(tables(), C, x=x, w12=w12[:, :128], w3=w3, b3=b3, workspace=ws)
    with pytest.raises(ValueError, match="w3 has shape"):
        mkv.route_chunks(tables(), C, x=x, w12=w12, w3=torch.zeros((3, 2 * I)), b3=b3, workspace=ws)
    with pytest.raises(ValueError, match="logits has shape"):
        mkv.route_chunks(tables(), C, x=x, w12=w12, w3=w3, b3=b3, workspace=ws, logits=torch.zeros((B, T, 2)))
    with pytest.raises(ValueError, match="token_expert has shape"):
        mkv.route_chunks(tables(), C, x=x, w12=w12, w3=w3, b3=b3, workspace=ws,
                         token_expert=torch.zeros((B, T + 1), dtype=torch.uint8))
    with pytest.raises(ValueError, match="logits has shape"):
        mkv.route_chunks(tables(), C, logits=torch.zeros((B + 1, T, 3)), logits_in=True)
    with pytest.raises(ValueError, match="must be on the GPU"):
        mkv.route_chunks(tables(), C, logits=torch.zeros((B, T, 3)), logits_in=True)


def test_similarity_checks():
    D = 256
    x = torch.zeros((B, T, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="qe has shape"):
        mkv.select_chunks_by_similarity(tables(), C, x, torch.zeros((B, D + 64), dtype=torch.bfloat16), 0.5, 0.0)
    with pytest.raises(ValueError, match="sim has shape"):
        mkv.select_chunks_by_similarity(tables(), C, x, torch.zeros((B, D), dtype=torch.bfloat16), 0.5, 0.0,
                                        sim=torch.zeros((B, 3)))


def test_prefill_checks():
    P = 64
    q = f16(B, Hq, P, d)
    with pytest.raises(ValueError, match="k_new has shape"):
        mkv.mixed_kv_prefill_attention(q, cache(), f16(B, Hkv, P - 1, d), f16(B, Hkv, P, d))
    with pytest.raises(ValueError, match="q has shape"):
        mkv.mixed_kv_prefill_attention(f16(B + 1, Hq, P, d), cache(), f16(B, Hkv, P, d), f16(B, Hkv, P, d))
    with pytest.raises(ValueError, match="must be on the GPU"):
        mkv.mixed_kv_prefill_attention(q, cache(), f16(B, Hkv, P, d), f16(B, Hkv, P, d))


def test_stream_helper_checks():
    with pytest.raises(ValueError, match="a_tail has shape"):
        mkv.append_tail_rows(f16(B, Hkv, d), f16(B, Hkv + 1, 8, d), 0)
    with pytest.raises(TypeError, match="share one 2-byte dtype"):
        mkv.append_tail_rows(torch.zeros((B, Hkv, d)), torch.zeros((B, Hkv, 8, d)), 0)
    with pytest.raises(ValueError, match="pos 8 outside"):
        mkv.append_tail_rows(f16(B, Hkv, d), f16(B, Hkv, 8, d), 8)
    small = torch.zeros(16, dtype=torch.uint8)
    big = torch.zeros(mkv.pool_bytes(4, B, Hkv, 3, d, C), dtype=torch.uint8)
    with pytest.raises(ValueError, match="src holds"):
        mkv.grow_pool(small, big, 4, B, Hkv, 2, 3, d, C)
    with pytest.raises(ValueError, match="dst holds"):
        mkv.grow_pool(big, small, 4, B, Hkv, 2, 3, d, C)
