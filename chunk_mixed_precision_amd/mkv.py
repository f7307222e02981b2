"""ctypes binding over libmkv.so (C ABI in include/mkv.h).

Argument marshalling only: every step of the path runs in the HIP library.
Tensors are torch tensors on the GPU; their data pointers and the current
torch stream are handed to the library as plain pointers.  If the library
is not built, the first call raises (there is no CPU fallback).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

from .configs import EXPERT_BITS, GROUP

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmkv.so")

MKV_OK = 0
MKV_ERR_ARG = -1
MKV_ERR_UNSUPPORTED = -2
MKV_ERR_WORKSPACE = -3
MKV_ERR_HIP = -4
MKV_ERR_SCRATCH = -5

MKV_FREEZE_FIRST = 0x1
MKV_LOGITS_IN = 0x2
MKV_APPEND = 0x4

MKV_OP_ROUTE = 1
MKV_OP_ATTENTION = 2
MKV_OP_SIMILARITY = 3
MKV_OP_PREFILL = 4

EXPORTED = (
    "mkv_route_chunks", "mkv_select_chunks_by_similarity", "mkv_quantize_pack_kv",
    "mkv_mixed_kv_decode_attention", "mkv_mixed_kv_decode_attention_noalloc", "mkv_mixed_kv_prefill_attention", "mkv_append_tail_rows", "mkv_grow_pool",
    "mkv_workspace_bytes", "mkv_group_bytes", "mkv_pool_bytes",
    "mkv_status_string", "mkv_last_hip_error", "mkv_version",
)


class MkvTables(ctypes.Structure):
    _fields_ = [("chunk_bits", ctypes.c_void_p), ("chunk_rank", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("seg_count", ctypes.c_void_p),
                ("n_max", ctypes.c_int)]


class MkvCache(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("Hkv", ctypes.c_int), ("d", ctypes.c_int), ("C", ctypes.c_int),
                ("cap", ctypes.c_int * 3), ("pool", ctypes.c_void_p * 3),
                ("seg_count", ctypes.c_void_p), ("overflow", ctypes.c_void_p)]


class MkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Open libmkv.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m chunk_mixed_precision_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, u, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
        L.mkv_route_chunks.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, u, vp,
                                       ctypes.POINTER(MkvTables), i, vp, sz, vp]
        L.mkv_route_chunks.restype = i
        L.mkv_select_chunks_by_similarity.argtypes = [vp, vp, i, i, i, i, ctypes.c_float, ctypes.c_float, u,
                                                      vp, ctypes.POINTER(MkvTables), i, vp, sz, vp]
        L.mkv_select_chunks_by_similarity.restype = i
        L.mkv_quantize_pack_kv.argtypes = [vp, vp, i, i, ctypes.POINTER(MkvTables),
                                           ctypes.POINTER(MkvCache), vp]
        L.mkv_quantize_pack_kv.restype = i
        L.mkv_mixed_kv_decode_attention.argtypes = [vp, i, ctypes.POINTER(MkvCache), vp, vp, i, i,
                                                    vp, vp, sz, vp]
        L.mkv_mixed_kv_decode_attention_noalloc.argtypes = [vp, i, ctypes.POINTER(MkvCache), vp, vp, i, i, vp, vp]
        L.mkv_mixed_kv_decode_attention_noalloc.restype = i
        L.mkv_mixed_kv_prefill_attention.argtypes = [vp, i, i, ctypes.POINTER(MkvCache), vp, vp, vp, vp, sz, vp]
        L.mkv_mixed_kv_prefill_attention.restype = i
        L.mkv_append_tail_rows.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
        L.mkv_append_tail_rows.restype = i
        L.mkv_grow_pool.argtypes = [vp, vp, i, i, i, i, i, i, i, vp]
        L.mkv_grow_pool.restype = i
        L.mkv_mixed_kv_decode_attention.restype = i
        L.mkv_workspace_bytes.argtypes = [i, i, i, i, i, i, ctypes.POINTER(ctypes.c_int)]
        L.mkv_workspace_bytes.restype = sz
        L.mkv_group_bytes.argtypes = [i, i]
        L.mkv_group_bytes.restype = sz
        L.mkv_pool_bytes.argtypes = [i, i, i, i, i, i]
        L.mkv_pool_bytes.restype = sz
        L.mkv_status_string.argtypes = [i]
        L.mkv_status_string.restype = ctypes.c_char_p
        L.mkv_last_hip_error.argtypes = []
        L.mkv_last_hip_error.restype = i
        L.mkv_version.argtypes = []
        L.mkv_version.restype = i
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != MKV_OK:
        msg = lib().mkv_status_string(status).decode()
        if status == MKV_ERR_HIP:
            msg += f"; hip error {lib().mkv_last_hip_error()}"
        raise MkvError(status, f"{what}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    """Device address of a tensor's data.  The C ABI takes dense row-major
    arrays, so a strided view is refused rather than read as if dense."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("the C ABI needs contiguous tensors (call .contiguous() on views)")
    return ctypes.c_void_p(t.data_ptr())


class _Args:
    """Checks of the tensor arguments of one call, made before anything is
    launched: dtype, shape (None entries are free) and density first, for
    every argument, then that each one lives on a GPU.  The C ABI sees only
    addresses and the sizes passed beside them, so a tensor of the wrong
    type or size, or a host tensor, would otherwise be read or written as
    whatever the kernel expects."""

    def __init__(self):
        self.seen = []

    def need(self, t, name: str, dtype: torch.dtype, shape: Sequence = None, optional: bool = False):
        if t is None:
            if optional:
                return
            raise ValueError(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if shape is not None:
            ok = t.dim() == len(shape) and all(w is None or int(w) == int(g) for w, g in zip(shape, t.shape))
            if not ok:
                want = "[" + ", ".join("*" if w is None else str(int(w)) for w in shape) + "]"
                raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: the C ABI needs contiguous tensors (call .contiguous() on views)")
        self.seen.append((name, t))

    def need_bytes(self, t, name: str, nbytes: int):
        """A byte buffer (uint8) of at least nbytes bytes."""
        self.need(t, name, torch.uint8)
        if t.numel() < nbytes:
            raise ValueError(f"{name} holds {t.numel()} bytes, needs {nbytes}")

    def tables(self, tables: "RouteTables", B: int):
        if tables.B != B:
            raise ValueError(f"routing tables are for {tables.B} sequences, the call has {B}")
        n = tables.n_max
        self.need(tables.chunk_bits, "tables.chunk_bits", torch.uint8, (B, n))
        self.need(tables.chunk_rank, "tables.chunk_rank", torch.int32, (B, n))
        self.need(tables.perm, "tables.perm", torch.int32, (B, n))
        self.need(tables.seg_count, "tables.seg_count", torch.int32, (B, 3))

    def cache(self, cache: "PackedCache"):
        self.need(cache.seg_count, "cache.seg_count", torch.int32, (cache.B, 3))
        for k, bits in enumerate(EXPERT_BITS):
            if cache.caps[k] > 0:
                self.need_bytes(cache.pools[k], f"cache.pools[{k}]",
                                pool_bytes(bits, cache.B, cache.Hkv, cache.caps[k], cache.d, cache.C))
        self.need(cache.overflow, "cache.overflow", torch.int32, optional=True)

    def on_gpu(self):
        dev = None
        for name, t in self.seen:
            if t.device.type != "cuda":
                raise ValueError(f"{name} must be on the GPU, got a tensor on {t.device}")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{name} is on {t.device}, other arguments on {dev}")


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def group_bytes(bits: int, d: int) -> int:
    return int(lib().mkv_group_bytes(bits, d))


def pool_bytes(bits: int, B: int, Hkv: int, cap: int, d: int, C: int) -> int:
    return int(lib().mkv_pool_bytes(bits, B, Hkv, cap, d, C))


def workspace_bytes_route(B: int, T: int, D: int, I: int) -> int:
    return int(lib().mkv_workspace_bytes(MKV_OP_ROUTE, B, T, D, I, 0, None))


def workspace_bytes_similarity(B: int, T: int, D: int, C: int) -> int:
    return int(lib().mkv_workspace_bytes(MKV_OP_SIMILARITY, B, T, D, C, 0, None))


def workspace_bytes_attention(B: int, Hq: int, Hkv: int, d: int, C: int, caps: Sequence[int]) -> int:
    arr = (ctypes.c_int * 3)(*caps)
    return int(lib().mkv_workspace_bytes(MKV_OP_ATTENTION, B, Hq, Hkv, d, C, arr))


class RouteTables:
    """Device routing tables of B sequences with room for n_max chunks."""

    def __init__(self, B: int, n_max: int, device="cuda"):
        self.B, self.n_max = B, n_max
        self.chunk_bits = torch.zeros((B, n_max), dtype=torch.uint8, device=device)
        self.chunk_rank = torch.zeros((B, n_max), dtype=torch.int32, device=device)
        self.perm = torch.zeros((B, n_max), dtype=torch.int32, device=device)
        self.seg_count = torch.zeros((B, 3), dtype=torch.int32, device=device)

    def c(self) -> MkvTables:
        return MkvTables(self.chunk_bits.data_ptr(), self.chunk_rank.data_ptr(), self.perm.data_ptr(),
                         self.seg_count.data_ptr(), self.n_max)


class PackedCache:
    """One layer's packed pools.  caps[k] = slots per (sequence, head) in the
    FP16 / INT4 / INT2 pool.  seg_count is the routing tables' (shared by
    every layer: routing sharing)."""

    def __init__(self, B: int, Hkv: int, d: int, C: int, caps: Sequence[int],
                 seg_count: torch.Tensor, device="cuda"):
        self.B, self.Hkv, self.d, self.C = B, Hkv, d, C
        self.caps = [int(c) for c in caps]
        self.pools = []
        for k, bits in enumerate(EXPERT_BITS):
            nbytes = pool_bytes(bits, B, Hkv, self.caps[k], d, C)
            self.pools.append(torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device))
        self.seg_count = seg_count
        self.overflow = torch.zeros(4, dtype=torch.int32, device=device)

    def c(self) -> MkvCache:
        cc = MkvCache()
        cc.B, cc.Hkv, cc.d, cc.C = self.B, self.Hkv, self.d, self.C
        for k in range(3):
            cc.cap[k] = self.caps[k]
            cc.pool[k] = self.pools[k].data_ptr()
        cc.seg_count = self.seg_count.data_ptr()
        cc.overflow = self.overflow.data_ptr()
        return cc

    def nbytes(self) -> int:
        return sum(p.numel() for p in self.pools)


def route_chunks(tables: RouteTables, C: int, *, x: torch.Tensor = None, w12: torch.Tensor = None,
                 w3: torch.Tensor = None, b3: torch.Tensor = None, logits: torch.Tensor = None,
                 logits_in: bool = False, freeze_first: bool = True, chunk_offset: int = 0,
                 append: bool = False, token_expert: torch.Tensor = None,
                 workspace: torch.Tensor = None, stream=None):
    """mkv_route_chunks.  Router mode: x [B,T,D] bf16, w12 [2I,D] bf16, w3 [3,I]
    f32, b3 [3] f32; logits (optional) receives [B,T,3].  Logits-in mode:
    logits [B,T,3] f32 is the input."""
    flags = (MKV_FREEZE_FIRST if freeze_first else 0) | (MKV_LOGITS_IN if logits_in else 0) \
        | (MKV_APPEND if append else 0)
    a = _Args()
    if logits_in:
        a.need(logits, "logits", torch.float32, (tables.B, None, 3))
        B, T = logits.shape[0], logits.shape[1]
        D = I = 0
    else:
        a.need(x, "x", torch.bfloat16, (tables.B, None, None))
        B, T, D = x.shape
        a.need(w12, "w12", torch.bfloat16, (None, D))
        I = w12.shape[0] // 2
        if w12.shape[0] != 2 * I:
            raise ValueError(f"w12 must have an even number of rows (W1 then W2), got {w12.shape[0]}")
        a.need(w3, "w3", torch.float32, (3, I))
        a.need(b3, "b3", torch.float32, (3,))
        a.need(logits, "logits", torch.float32, (B, T, 3), optional=True)
        if workspace is None:
            workspace = torch.empty(workspace_bytes_route(B, T, D, I), dtype=torch.uint8, device=x.device)
        a.need(workspace, "workspace", torch.uint8)
    a.need(token_expert, "token_expert", torch.uint8, (B, T), optional=True)
    a.tables(tables, B)
    tab = tables.c()
    a.on_gpu()
    st = lib().mkv_route_chunks(_ptr(x), _ptr(w12), _ptr(w3), _ptr(b3), _ptr(logits), B, T, D, I, C, flags,
                                _ptr(token_expert), ctypes.byref(tab), chunk_offset, _ptr(workspace),
                                0 if workspace is None else workspace.numel() * workspace.element_size(),
                                _stream(stream))
    _check(st, "mkv_route_chunks")


def select_chunks_by_similarity(tables: RouteTables, C: int, x: torch.Tensor, qe: torch.Tensor,
                                tau_hi: float, tau_lo: float, *, sim: torch.Tensor = None,
                                freeze_first: bool = True, chunk_offset: int = 0, append: bool = False,
                                workspace: torch.Tensor = None, stream=None):
    """mkv_select_chunks_by_similarity: x [B,T,D] bf16 token embeddings, qe
    [B,D] bf16 query embeddings; sim (optional) receives [B, T/C] f32."""
    flags = (MKV_FREEZE_FIRST if freeze_first else 0) | (MKV_APPEND if append else 0)
    a = _Args()
    a.need(x, "x", torch.bfloat16, (tables.B, None, None))
    B, T, D = x.shape
    a.need(qe, "qe", torch.bfloat16, (B, D))
    a.need(sim, "sim", torch.float32, (B, T // C if C > 0 else None), optional=True)
    a.tables(tables, B)
    if workspace is None:
        workspace = torch.empty(workspace_bytes_similarity(B, T, D, C), dtype=torch.uint8, device=x.device)
    a.need(workspace, "workspace", torch.uint8)
    tab = tables.c()
    a.on_gpu()
    st = lib().mkv_select_chunks_by_similarity(_ptr(x), _ptr(qe), B, T, D, C, float(tau_hi), float(tau_lo),
                                               flags, _ptr(sim), ctypes.byref(tab), chunk_offset,
                                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                                               _stream(stream))
    _check(st, "mkv_select_chunks_by_similarity")


def workspace_bytes_prefill(B: int, Hq: int, P: int, d: int, C: int, caps: Sequence[int]) -> int:
    arr = (ctypes.c_int * 3)(*[int(c) for c in caps])
    return int(lib().mkv_workspace_bytes(MKV_OP_PREFILL, B, Hq, P, d, C, arr))


def mixed_kv_prefill_attention(q: torch.Tensor, cache: PackedCache, k_new: torch.Tensor, v_new: torch.Tensor,
                               out: torch.Tensor = None, workspace: torch.Tensor = None, stream=None) -> torch.Tensor:
    """mkv_mixed_kv_prefill_attention: q [B, Hq, P, d] fp16, k_new/v_new
    [B, Hkv, P, d] fp16 -> out [B, Hq, P, d] f32."""
    a = _Args()
    a.need(q, "q", torch.float16, (cache.B, None, None, cache.d))
    B, Hq, P, d = q.shape
    a.need(k_new, "k_new", torch.float16, (B, cache.Hkv, P, d))
    a.need(v_new, "v_new", torch.float16, (B, cache.Hkv, P, d))
    a.cache(cache)
    if out is None:
        out = torch.empty((B, Hq, P, d), dtype=torch.float32, device=q.device)
    a.need(out, "out", torch.float32, (B, Hq, P, d))
    if workspace is None:
        workspace = torch.empty(workspace_bytes_prefill(B, Hq, P, d, cache.C, cache.caps), dtype=torch.uint8,
                                device=q.device)
    a.need(workspace, "workspace", torch.uint8)
    cc = cache.c()
    a.on_gpu()
    st = lib().mkv_mixed_kv_prefill_attention(_ptr(q), Hq, P, ctypes.byref(cc), _ptr(k_new), _ptr(v_new), _ptr(out),
                                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                                              _stream(stream))
    _check(st, "mkv_mixed_kv_prefill_attention")
    return out


def append_tail_rows(a_new: torch.Tensor, a_tail: torch.Tensor, pos: int, b_new: torch.Tensor = None,
                     b_tail: torch.Tensor = None, stream=None):
    """mkv_append_tail_rows: a_new [..., W] (rows = all leading dims) into
    token `pos` of a_tail [..., S, W]; the same for the b pair if given."""
    a = _Args()
    if a_new is None or a_tail is None:
        raise ValueError("a_new and a_tail are required")
    if a_new.element_size() != 2 or a_tail.dtype != a_new.dtype:
        raise TypeError(f"a_new and a_tail must share one 2-byte dtype, got {a_new.dtype} and {a_tail.dtype}")
    W = a_new.shape[-1]
    rows = a_new.numel() // W
    a.need(a_new, "a_new", a_new.dtype)
    a.need(a_tail, "a_tail", a_new.dtype, (*a_new.shape[:-1], None, W))
    if (b_new is None) != (b_tail is None):
        raise ValueError("b_new and b_tail go together")
    if b_new is not None:
        a.need(b_new, "b_new", a_new.dtype, tuple(a_new.shape))
        a.need(b_tail, "b_tail", a_new.dtype, tuple(a_tail.shape))
    if not 0 <= pos < a_tail.shape[-2]:
        raise ValueError(f"pos {pos} outside the tail's {a_tail.shape[-2]} rows")
    a.on_gpu()
    st = lib().mkv_append_tail_rows(_ptr(a_new), _ptr(b_new), _ptr(a_tail), _ptr(b_tail), rows, W,
                                    a_tail.shape[-2], pos, _stream(stream))
    _check(st, "mkv_append_tail_rows")


def grow_pool(src: torch.Tensor, dst: torch.Tensor, bits: int, B: int, Hkv: int, cap_old: int, cap_new: int,
              d: int, C: int, stream=None):
    """mkv_grow_pool: re-lay a pool of cap_old slots into one of cap_new."""
    a = _Args()
    a.need_bytes(src, "src", pool_bytes(bits, B, Hkv, cap_old, d, C))
    a.need_bytes(dst, "dst", pool_bytes(bits, B, Hkv, cap_new, d, C))
    a.on_gpu()
    st = lib().mkv_grow_pool(_ptr(src), _ptr(dst), bits, B, Hkv, cap_old, cap_new, d, C, _stream(stream))
    _check(st, "mkv_grow_pool")


def quantize_pack_kv(k: torch.Tensor, v: torch.Tensor, tables: RouteTables, cache: PackedCache,
                     chunk_offset: int = 0, stream=None):
    """mkv_quantize_pack_kv: k, v [B, Hkv, T, d] fp16 (T = new chunks * C)."""
    a = _Args()
    a.need(k, "k", torch.float16, (cache.B, cache.Hkv, None, cache.d))
    T = k.shape[2]
    a.need(v, "v", torch.float16, (cache.B, cache.Hkv, T, cache.d))
    a.tables(tables, cache.B)
    a.cache(cache)
    tab = tables.c()
    cc = cache.c()
    a.on_gpu()
    st = lib().mkv_quantize_pack_kv(_ptr(k), _ptr(v), T, chunk_offset, ctypes.byref(tab),
                                    ctypes.byref(cc), _stream(stream))
    _check(st, "mkv_quantize_pack_kv")


def attention_workspace(B: int, Hq: int, cache: "PackedCache", device="cuda") -> torch.Tensor:
    """Workspace (tile partials) for mixed_kv_decode_attention."""
    return torch.empty(workspace_bytes_attention(B, Hq, cache.Hkv, cache.d, cache.C, cache.caps),
                       dtype=torch.uint8, device=device)


def mixed_kv_decode_attention(q: torch.Tensor, cache: PackedCache, out: torch.Tensor = None,
                              tail_k: torch.Tensor = None, tail_v: torch.Tensor = None,
                              tail_len: int = None, workspace: torch.Tensor = None, stream=None) -> torch.Tensor:
    """mkv_mixed_kv_decode_attention: q [B, Hq, d] fp16 -> out [B, Hq, d] f32.
    tail_k, tail_v: [B, Hkv, S, d] fp16 tails of S rows; tokens 0 .. tail_len-1
    of each row are attended (tail_len defaults to S)."""
    a = _Args()
    a.need(q, "q", torch.float16, (cache.B, None, cache.d))
    B, Hq, d = q.shape
    a.cache(cache)
    if (tail_k is None) != (tail_v is None):
        raise ValueError("tail_k and tail_v go together")
    a.need(tail_k, "tail_k", torch.float16, (B, cache.Hkv, None, d), optional=True)
    stride = 0 if tail_k is None else tail_k.shape[2]
    a.need(tail_v, "tail_v", torch.float16, (B, cache.Hkv, stride, d), optional=True)
    if tail_len is None:
        tail_len = stride
    if not 0 <= tail_len <= stride:
        raise ValueError(f"tail_len {tail_len} outside the tail's {stride} rows")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    a.need(out, "out", torch.float32, (B, Hq, d))
    if workspace is None:
        workspace = attention_workspace(B, Hq, cache, q.device)
    a.need(workspace, "workspace", torch.uint8)
    cc = cache.c()
    a.on_gpu()
    st = lib().mkv_mixed_kv_decode_attention(_ptr(q), Hq, ctypes.byref(cc), _ptr(tail_k), _ptr(tail_v),
                                             tail_len, stride, _ptr(out), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "mkv_mixed_kv_decode_attention")
    return out


def mixed_kv_decode_attention_noalloc(q: torch.Tensor, cache: PackedCache, out: torch.Tensor,
                                      tail_k: torch.Tensor = None, tail_v: torch.Tensor = None,
                                      tail_len: int = None, stream=None) -> torch.Tensor:
    """mkv_mixed_kv_decode_attention_noalloc: as mixed_kv_decode_attention,
    with the tile partials in the library's fixed per-GPU scratch instead of
    a workspace.  `out` [B, Hq, d] f32 must be given: nothing is allocated."""
    a = _Args()
    a.need(q, "q", torch.float16, (cache.B, None, cache.d))
    B, Hq, d = q.shape
    a.cache(cache)
    if (tail_k is None) != (tail_v is None):
        raise ValueError("tail_k and tail_v go together")
    a.need(tail_k, "tail_k", torch.float16, (B, cache.Hkv, None, d), optional=True)
    stride = 0 if tail_k is None else tail_k.shape[2]
    a.need(tail_v, "tail_v", torch.float16, (B, cache.Hkv, stride, d), optional=True)
    if tail_len is None:
        tail_len = stride
    if not 0 <= tail_len <= stride:
        raise ValueError(f"tail_len {tail_len} outside the tail's {stride} rows")
    a.need(out, "out", torch.float32, (B, Hq, d))
    cc = cache.c()
    a.on_gpu()
    st = lib().mkv_mixed_kv_decode_attention_noalloc(_ptr(q), Hq, ctypes.byref(cc), _ptr(tail_k), _ptr(tail_v),
                                                     tail_len, stride, _ptr(out), _stream(stream))
    _check(st, "mkv_mixed_kv_decode_attention_noalloc")
    return out
