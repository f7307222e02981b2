"""Test-side reader of the packed-cache layout documented in include/mkv.h,
written from that documentation in numpy.  It shares no code with the HIP
library: it turns pool bytes back into logical codes, scales and minima so
that tests can compare them with the oracle.
"""
from __future__ import annotations

import functools

import numpy as np

GROUP = 32


def tok_xor(S: int, L: int) -> int:
    b = [(L >> i) & 1 for i in range(4)]
    if S == 16:
        return (1 * b[0]) ^ (2 * b[1]) ^ (7 * b[2]) ^ (12 * b[3])
    if S == 8:
        return (2 * b[0]) ^ (4 * b[1]) ^ (14 * b[2])
    raise ValueError(S)


def tok_of(S: int, L: int, r: int) -> int:
    """Token held by key field position r (0..31) of lane slot L."""
    return (r & 16) | ((r & 15) ^ tok_xor(S, L))


def section_rows(bits: int):
    """(key meta, key codes, value meta, value codes) rows of a group block."""
    if bits == 16:
        return 0, 32, 0, 32
    return 4, 2 * bits, 4, 2 * bits


def group_bytes(bits: int, d: int) -> int:
    return sum(section_rows(bits)) * (d // 8) * 16


def chunk_bytes(bits: int, d: int, C: int) -> int:
    return group_bytes(bits, d) * (C // GROUP)


@functools.lru_cache(maxsize=None)
def _maps(bits: int, d: int):
    """Index maps from (row, lane slot, dword, field) to (token, channel)."""
    S, NG = d // 8, d // 32
    KM, KC, VM, VC = section_rows(bits)
    m = {}
    if bits == 16:
        # K: row r, slot L, half-word e8 (0..7) -> token r^f(L), channel 8L+e8
        kt = np.zeros((32, S, 8), np.int64)
        kc = np.zeros((32, S, 8), np.int64)
        vt = np.zeros((32, S, 8), np.int64)
        vc = np.zeros((32, S, 8), np.int64)
        for r in range(32):
            for L in range(S):
                G, tq = L % NG, L // NG
                for e in range(8):
                    kt[r, L, e] = tok_of(S, L, r)
                    kc[r, L, e] = 8 * L + e
                    vt[r, L, e] = tq + 4 * (r >> 2)
                    vc[r, L, e] = 32 * G + 8 * (r & 3) + e
        m.update(kt=kt, kc=kc, vt=vt, vc=vc)
        return m
    F = 32 // bits
    kt = np.zeros((KC, S, 4, F), np.int64)
    kc = np.zeros((KC, S, 4, F), np.int64)
    for row in range(KC):
        for L in range(S):
            for e in range(4):
                for i in range(F):
                    kt[row, L, e, i] = tok_of(S, L, F * (row >> 1) + i)
                    kc[row, L, e, i] = 8 * L + 4 * (row & 1) + e
    vt = np.zeros((VC, S, 4, F), np.int64)
    vc = np.zeros((VC, S, 4, F), np.int64)
    for row in range(VC):
        for L in range(S):
            G, tq = L % NG, L // NG
            for dw in range(4):
                for i in range(F):
                    if bits == 4:
                        mm, u = row, dw
                        vt[row, L, dw, i] = tq + 4 * mm
                        vc[row, L, dw, i] = 32 * G + 8 * u + i
                    else:
                        mm, u = 2 * row + (dw >> 1), dw & 1
                        vt[row, L, dw, i] = tq + 4 * mm
                        vc[row, L, dw, i] = 32 * G + 16 * u + i
    # meta: row mr, slot L, float f4 (0..3) -> token, group, is_min
    mt = np.zeros((4, S, 4), np.int64)
    mg = np.zeros((4, S, 4), np.int64)
    for mr in range(4):
        for L in range(S):
            G, tq = L % NG, L // NG
            for f4 in range(4):
                mt[mr, L, f4] = tq + 4 * (2 * mr + (f4 >> 1))
                mg[mr, L, f4] = G
    m.update(kt=kt, kc=kc, vt=vt, vc=vc, mt=mt, mg=mg)
    return m


def decode_blocks(blocks: np.ndarray, bits: int, d: int) -> dict:
    """Group blocks uint8 [N, group_bytes] -> logical contents with a leading N.
    INT-b: kq [N,32,d], ks [N,d], km [N,d], vq [N,32,d], vs [N,32,d/32], vm.
    FP16:  k [N,32,d], v [N,32,d] float16."""
    S, NG = d // 8, d // 32
    KM, KC, VM, VC = section_rows(bits)
    N = blocks.shape[0]
    cells = np.ascontiguousarray(blocks).reshape(N, KM + KC + VM + VC, S, 16)
    m = _maps(bits, d)
    if bits == 16:
        kh = cells[:, :KC].copy().view(np.float16).reshape(N, KC, S, 8)
        vh = cells[:, KC:].copy().view(np.float16).reshape(N, VC, S, 8)
        k = np.zeros((N, 32, d), np.float16)
        v = np.zeros((N, 32, d), np.float16)
        k[:, m["kt"], m["kc"]] = kh
        v[:, m["vt"], m["vc"]] = vh
        return {"bits": 16, "k": k, "v": v}
    F = 32 // bits
    mask = np.uint32((1 << bits) - 1)
    shifts = (np.arange(F, dtype=np.uint32) * np.uint32(bits))
    kmeta = cells[:, 0:KM].copy().view(np.float32).reshape(N, 4, S, 4)
    kw = cells[:, KM:KM + KC].copy().view(np.uint32).reshape(N, KC, S, 4)
    vmeta = cells[:, KM + KC:KM + KC + VM].copy().view(np.float32).reshape(N, 4, S, 4)
    vw = cells[:, KM + KC + VM:].copy().view(np.uint32).reshape(N, VC, S, 4)
    kfield = (kw[..., None] >> shifts) & mask
    kq = np.zeros((N, 32, d), np.uint8)
    kq[:, m["kt"], m["kc"]] = kfield.astype(np.uint8)
    ks = np.concatenate([kmeta[:, 0], kmeta[:, 1]], axis=-1).reshape(N, d)      # [N, S, 8] -> [N, d]
    km = np.concatenate([kmeta[:, 2], kmeta[:, 3]], axis=-1).reshape(N, d)
    vfield = (vw[..., None] >> shifts) & mask
    vq = np.zeros((N, 32, d), np.uint8)
    vq[:, m["vt"], m["vc"]] = vfield.astype(np.uint8)
    vs = np.zeros((N, 32, NG), np.float32)
    vm = np.zeros((N, 32, NG), np.float32)
    is_scale = (np.arange(4) % 2 == 0)
    mt, mg = m["mt"], m["mg"]
    vs[:, mt[..., is_scale], mg[..., is_scale]] = vmeta[..., is_scale]
    vm[:, mt[..., ~is_scale], mg[..., ~is_scale]] = vmeta[..., ~is_scale]
    return {"bits": bits, "kq": kq, "ks": ks, "km": km, "vq": vq, "vs": vs, "vm": vm}


def decode_chunks(pool: np.ndarray, bits: int, Hkv: int, cap: int, d: int, C: int,
                  bh_slots) -> list:
    """Decode the chunks at (b, h, slot) triples; returns dicts shaped like the
    oracle's quantize_chunk output: kq [C,d], ks [C/32,d], km, vq [C,d],
    vs [C,d/32], vm  (FP16: k, v [C,d])."""
    gb = group_bytes(bits, d)
    gpc = C // GROUP
    idx = []
    for (b, h, slot) in bh_slots:
        base = ((b * Hkv + h) * cap + slot) * gpc
        idx.extend(range(base, base + gpc))
    if not idx:
        return []
    blocks = pool.reshape(-1, gb)[np.asarray(idx)]
    dec = decode_blocks(blocks, bits, d)
    out = []
    for n in range(len(bh_slots)):
        sl = slice(n * gpc, (n + 1) * gpc)
        if bits == 16:
            out.append({"bits": 16, "k": dec["k"][sl].reshape(C, d), "v": dec["v"][sl].reshape(C, d)})
        else:
            out.append({"bits": bits,
                        "kq": dec["kq"][sl].reshape(C, d), "ks": dec["ks"][sl], "km": dec["km"][sl],
                        "vq": dec["vq"][sl].reshape(C, d),
                        "vs": dec["vs"][sl].reshape(C, d // 32), "vm": dec["vm"][sl].reshape(C, d // 32)})
    return out
