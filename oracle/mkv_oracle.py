"""Plain CPU oracle for the chunk-adaptive mixed-precision KV-cache path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module.  The product path (the HIP library and its Python binding) never
calls it, and this module imports nothing from that path.

Sources (web pages, cited by title and section):
  [MoQAE]    "MoQAE: Mixed-Precision Quantization for Long-Context LLM
             Inference via Mixture of Quantization-Aware Experts", Paper-Notes
             page (ACL 2025): sections "Overall framework" (整体框架) and
             "Key designs" (关键设计: Quantization-Aware Experts, Routing
             Freezing, Routing Sharing), "Related work" (KIVI note).
  [Cocktail] scholarfeed author page, Cocktail abstract (chunk-level
             quantization search; chunk-level KV cache computation that
             reorders chunks before quantization).

Every step is written out in the order the pages give it, in plain numpy.
Floating point: the router and attention run in float64; the quantizer runs
in IEEE float32, one rounded operation at a time (numpy float32 element-wise
arithmetic never contracts a*b+c into an FMA), because the codes, scales and
minima must be reproduced bit for bit.

Readings taken where the pages are silent or garbled:
  R1  The router formula on the MoQAE page lost its operators in extraction.
      It is read as z = f((X W1^T) * (X W2^T)) W3^T + b3 with "*" the
      element-wise product and f = SiLU applied to that product.  Only the
      last layer has a bias (b3).  parity unpinned against the authors'
      router (no code or weights exist).
  R2  "Probabilities": the softmax is monotone, so the argmax is taken on the
      logits.  Exact ties go to the lowest expert index (higher precision).
  R3  The chunk vote is a plurality vote; a tie between counts goes to the
      lowest expert index (higher precision).
  R4  Routing freezing pins chunk 0 of every sequence to FP16.
  R5  Routing sharing: one table per sequence serves every layer and head.
  R6  Cocktail's reorder is a stable partition of a sequence's chunks into
      the segment order FP16, INT4, INT2.
  R7  Quantizer: asymmetric min-max with a float minimum, groups of 32 along
      each tensor's quantization axis (keys: 32 tokens of one channel,
      values: 32 channels of one token, following the KIVI note).
      s = fl((mx - mn) / L), r = fl(1 / s), code = clamp(rne(fl(fl(x - mn) * r)), 0, L),
      a -0 extreme (mn or mx) is canonicalised to +0, so s and mn never carry
      a sign that depends on reduction order; s == 0 gives all-zero codes.
  R8  Attention is ordinary softmax attention over the dequantized cache
      (x_hat = code * s + mn), no mask, keys already position-encoded.
  R9  Cocktail's chunk-level quantization search gives each chunk a bitwidth
      from the similarity between the chunk and the query.  The page names no
      measure, summary or rule.  Plainest reading: the chunk is summarised by
      the mean of its tokens' embeddings, the similarity is the cosine
      between that mean and the query embedding (a zero vector gives 0), and
      two thresholds split the range: sim >= tau_hi -> FP16,
      tau_lo <= sim < tau_hi -> INT4, sim < tau_lo -> INT2 (more similar
      chunks matter more to the query and keep more bits).  Routing freezing
      may pin chunk 0 as for the router.  parity unpinned against the
      authors' search (no code or constants exist).
  R10 Chunked prefill: a chunk of P new tokens is attended before it is
      quantized.  Query i of the chunk sees every cached token (dequantized)
      and the new chunk's own fp16 tokens 0..i (causal), in ordinary softmax
      attention.
"""
from __future__ import annotations

import numpy as np

# Expert index -> bitwidth.  Index order is also the precision order
# (MoQAE "Key designs": the experts are FP16, INT4 and INT2 settings).
EXPERT_BITS = (16, 4, 2)
GROUP = 32  # quantization group size along each tensor's quantization axis


# --------------------------------------------------------------------------
# input decoding (bit patterns -> exact values); no method arithmetic
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16/int16) -> exact float64 values."""
    u32 = bits.astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# router  [MoQAE, "Key designs" — Quantization-Aware Experts]
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, w12: np.ndarray, w3: np.ndarray,
                  b3: np.ndarray, inner: int) -> np.ndarray:
    """Per-token expert scores, float64.

    x   [N, D] hidden states (float64 values, already exact bf16 values)
    w12 [2*inner, D] rows 0..inner-1 = W1, rows inner..2*inner-1 = W2
    w3  [3, inner], b3 [3]
    Returns z [N, 3] = SiLU((x W1^T) * (x W2^T)) W3^T + b3  (reading R1).
    """
    x = np.asarray(x, dtype=np.float64)
    w12 = np.asarray(w12, dtype=np.float64)
    h1 = x @ w12[:inner].T
    h2 = x @ w12[inner:].T
    u = h1 * h2
    with np.errstate(over="ignore"):
        a = u / (1.0 + np.exp(-u))          # SiLU(u) = u * sigmoid(u)
    return a @ np.asarray(w3, dtype=np.float64).T + np.asarray(b3, dtype=np.float64)


def token_experts(z: np.ndarray) -> np.ndarray:
    """Each token picks its highest-scoring expert; ties -> lowest index (R2).
    np.argmax returns the first maximal index, which is that rule."""
    return np.argmax(z, axis=-1).astype(np.uint8)


# --------------------------------------------------------------------------
# chunk vote, routing freezing, routing sharing  [MoQAE, "Key designs"]
# --------------------------------------------------------------------------
def chunk_vote(experts: np.ndarray, chunk: int, freeze_first: bool = True,
               chunk_offset: int = 0) -> np.ndarray:
    """Plurality vote of the token experts inside each chunk (R3), then
    routing freezing (R4).

    experts [B, T] expert index per token, T a multiple of ``chunk``.
    chunk_offset: index of the first chunk in ``experts`` within its sequence
    (freezing only touches the chunk whose index is 0).
    Returns the winning expert index per chunk, [B, T // chunk] uint8.
    """
    B, T = experts.shape
    n = T // chunk
    out = np.zeros((B, n), dtype=np.uint8)
    for b in range(B):
        for c in range(n):
            seg = experts[b, c * chunk:(c + 1) * chunk]
            counts = [int(np.count_nonzero(seg == k)) for k in range(3)]
            best = max(counts)
            out[b, c] = min(k for k in range(3) if counts[k] == best)
    if freeze_first and chunk_offset == 0 and n > 0:
        out[:, 0] = 0
    return out


def bits_of(expert_idx: np.ndarray) -> np.ndarray:
    return np.asarray(EXPERT_BITS, dtype=np.uint8)[expert_idx]


def expert_of_bits(bits: np.ndarray) -> np.ndarray:
    lut = np.full(256, 255, dtype=np.uint8)
    lut[16], lut[4], lut[2] = 0, 1, 2
    out = lut[np.asarray(bits, dtype=np.uint8)]
    if np.any(out == 255):
        raise ValueError("bitwidth outside {16, 4, 2}")
    return out


# --------------------------------------------------------------------------
# reorder  [Cocktail abstract: chunks reordered before quantization]
# --------------------------------------------------------------------------
def reorder(expert_idx: np.ndarray):
    """Stable partition of each sequence's chunks by expert (R6).

    expert_idx [B, n].  Returns
      perm      [B, n] int32: position in segment order -> chunk index
      rank      [B, n] int32: slot of each chunk inside its own segment
      seg_count [B, 3] int32: chunks per expert
    """
    B, n = expert_idx.shape
    perm = np.zeros((B, n), dtype=np.int32)
    rank = np.zeros((B, n), dtype=np.int32)
    seg = np.zeros((B, 3), dtype=np.int32)
    for b in range(B):
        pos = 0
        for k in range(3):
            for c in range(n):
                if expert_idx[b, c] == k:
                    perm[b, pos] = c
                    rank[b, c] = seg[b, k]
                    seg[b, k] += 1
                    pos += 1
    return perm, rank, seg


# --------------------------------------------------------------------------
# quantizer  [MoQAE "Overall framework": the KV cache is quantized at the
# chosen bitwidth; "Related work": keys per channel (KIVI)]
# --------------------------------------------------------------------------
def quantize_groups(g: np.ndarray, bits: int):
    """Asymmetric min-max quantization of groups along the last axis (R7).

    g [..., 32] float16 (or float32 holding fp16 values).  All arithmetic is
    float32, one rounding per operation.  Returns (codes uint8 [..., 32],
    scale float32 [...], minimum float32 [...]).
    """
    assert bits in (2, 4)
    L = np.float32((1 << bits) - 1)
    x = np.asarray(g).astype(np.float32)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    mn = (mn + np.float32(0.0)).astype(np.float32)      # -0 -> +0
    mx = (mx + np.float32(0.0)).astype(np.float32)      # -0 -> +0
    s = ((mx - mn).astype(np.float32) / L).astype(np.float32)
    zero = s == np.float32(0.0)
    safe = np.where(zero, np.float32(1.0), s).astype(np.float32)
    r = (np.float32(1.0) / safe).astype(np.float32)
    t = (x - mn[..., None]).astype(np.float32)
    t = (t * r[..., None]).astype(np.float32)
    q = np.rint(t)                                      # round half to even
    q = np.clip(q, 0, L)
    q[zero] = 0
    return q.astype(np.uint8), s, mn


def quantize_chunk_k(k: np.ndarray, bits: int):
    """Keys of one chunk, [C, d] fp16: groups are 32 consecutive tokens of
    one channel.  Returns codes [C, d], scale [C/32, d], min [C/32, d]."""
    C, d = k.shape
    g = np.asarray(k).reshape(C // GROUP, GROUP, d).transpose(0, 2, 1)   # [G, d, 32]
    q, s, mn = quantize_groups(g, bits)
    return q.transpose(0, 2, 1).reshape(C, d), s, mn


def quantize_chunk_v(v: np.ndarray, bits: int):
    """Values of one chunk, [C, d] fp16: groups are 32 consecutive channels
    of one token.  Returns codes [C, d], scale [C, d/32], min [C, d/32]."""
    C, d = v.shape
    g = np.asarray(v).reshape(C, d // GROUP, GROUP)
    q, s, mn = quantize_groups(g, bits)
    return q.reshape(C, d), s, mn


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack a 1-D run of codes into 32-bit words, least significant field
    first: code i goes to word i // (32/bits) at bit bits*(i % (32/bits))."""
    per = 32 // bits
    c = np.asarray(codes, dtype=np.uint64).reshape(-1, per)
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
    return (c << shifts).sum(axis=1).astype(np.uint32)


def unpack_codes(words: np.ndarray, bits: int) -> np.ndarray:
    per = 32 // bits
    w = np.asarray(words, dtype=np.uint64).reshape(-1, 1)
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
    return ((w >> shifts) & np.uint64((1 << bits) - 1)).astype(np.uint8).reshape(-1)


def dequant_k(codes: np.ndarray, scale: np.ndarray, mn: np.ndarray) -> np.ndarray:
    """x_hat = code * s + mn in float64, keys (per-channel groups)."""
    C, d = codes.shape
    s = np.repeat(scale.astype(np.float64), GROUP, axis=0)      # [C, d]
    m = np.repeat(mn.astype(np.float64), GROUP, axis=0)
    return codes.astype(np.float64) * s + m


def dequant_v(codes: np.ndarray, scale: np.ndarray, mn: np.ndarray) -> np.ndarray:
    """x_hat = code * s + mn in float64, values (per-token groups)."""
    s = np.repeat(scale.astype(np.float64), GROUP, axis=1)      # [C, d]
    m = np.repeat(mn.astype(np.float64), GROUP, axis=1)
    return codes.astype(np.float64) * s + m


# --------------------------------------------------------------------------
# attention  [MoQAE "Overall framework": ordinary attention on the cache]
# --------------------------------------------------------------------------
def attention(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(d)) v for one query vector, float64.

    q [d], k_hat [T, d], v_hat [T, d]."""
    q = np.asarray(q, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    d = q.shape[0]
    sc = (k_hat @ q) / np.sqrt(d)
    w = np.exp(sc - sc.max())
    return (w @ v_hat) / w.sum()


# --------------------------------------------------------------------------
# whole-path helpers (still step by step; used by tests and the bench's
# CPU-baseline leg)
# --------------------------------------------------------------------------
# --------------------------------------------------------------------------
# similarity-based chunk selection  [Cocktail abstract: chunk-level
# quantization search; reading R9]
# --------------------------------------------------------------------------
def chunk_similarity(x: np.ndarray, qe: np.ndarray, chunk: int) -> np.ndarray:
    """Cosine similarity between each chunk's mean token embedding and the
    query embedding, float64.

    x  [B, T, D] embeddings (float64 values), T a multiple of ``chunk``
    qe [B, D] query embeddings
    Returns sim [B, T/chunk]; 0 where either vector is zero.
    """
    x = np.asarray(x, dtype=np.float64)
    qe = np.asarray(qe, dtype=np.float64)
    B, T, D = x.shape
    n = T // chunk
    sim = np.zeros((B, n))
    for b in range(B):
        qn = np.sqrt(np.dot(qe[b], qe[b]))
        for c in range(n):
            mean = x[b, c * chunk:(c + 1) * chunk].sum(axis=0) / chunk
            mn = np.sqrt(np.dot(mean, mean))
            if mn > 0 and qn > 0:
                sim[b, c] = np.dot(mean, qe[b]) / (mn * qn)
    return sim


def similarity_experts(sim: np.ndarray, tau_hi: float, tau_lo: float,
                       freeze_first: bool = False, chunk_offset: int = 0) -> np.ndarray:
    """Expert index of each chunk from its similarity (reading R9): FP16 at
    or above tau_hi, INT4 at or above tau_lo, INT2 below.  With freezing,
    the sequence's chunk 0 (global index 0, i.e. only when chunk_offset is
    0) is FP16."""
    sim = np.asarray(sim, dtype=np.float64)
    e = np.where(sim >= tau_hi, 0, np.where(sim >= tau_lo, 1, 2)).astype(np.int64)
    if freeze_first and chunk_offset == 0 and e.shape[1] > 0:
        e[:, 0] = 0
    return e


def select_by_similarity(x_bits: np.ndarray, qe_bits: np.ndarray, chunk: int, tau_hi: float,
                         tau_lo: float, freeze_first: bool = False):
    """x_bits [B, T, D] and qe_bits [B, D] bf16 bit patterns.  Returns
    (sim [B, n] f64, chunk expert [B, n], perm, rank, seg_count)."""
    B, T, D = x_bits.shape
    x = bf16_bits_to_f64(x_bits.reshape(B * T, D)).reshape(B, T, D)
    qe = bf16_bits_to_f64(qe_bits)
    sim = chunk_similarity(x, qe, chunk)
    e = similarity_experts(sim, tau_hi, tau_lo, freeze_first)
    perm, rank, seg = reorder(e)
    return sim, e, perm, rank, seg


def prefill_attention(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray,
                      k_new: np.ndarray, v_new: np.ndarray) -> np.ndarray:
    """Chunked-prefill attention of one (sequence, query head), float64
    (reading R10).  q [P, d] queries of the new chunk, k_hat/v_hat [T, d]
    the dequantized cache, k_new/v_new [P, d] the chunk's own keys/values.
    Returns [P, d]: row i attends to the cache and new tokens 0..i."""
    P = q.shape[0]
    out = np.zeros((P, q.shape[1]))
    for i in range(P):
        k = np.concatenate([k_hat, k_new[:i + 1]])
        v = np.concatenate([v_hat, v_new[:i + 1]])
        out[i] = attention(q[i], k, v)
    return out


def route(x_bits: np.ndarray, w12_bits: np.ndarray, w3: np.ndarray,
          b3: np.ndarray, inner: int, chunk: int, freeze_first: bool = True):
    """x_bits [B, T, D] bf16 bit patterns.  Returns (logits [B,T,3] f64,
    token experts [B,T], chunk expert [B,n], perm, rank, seg_count)."""
    B, T, D = x_bits.shape
    z = router_logits(bf16_bits_to_f64(x_bits.reshape(B * T, D)),
                      bf16_bits_to_f64(w12_bits), w3, b3, inner).reshape(B, T, 3)
    e = token_experts(z)
    v = chunk_vote(e, chunk, freeze_first)
    perm, rank, seg = reorder(v)
    return z, e, v, perm, rank, seg


def quantize_chunk(k: np.ndarray, v: np.ndarray, bits: int):
    """One chunk of one head: returns a dict with the logical result.
    FP16 chunks are kept bit for bit."""
    if bits == 16:
        return {"bits": 16, "k": np.asarray(k, np.float16).copy(),
                "v": np.asarray(v, np.float16).copy()}
    kq, ks, km = quantize_chunk_k(k, bits)
    vq, vs, vm = quantize_chunk_v(v, bits)
    return {"bits": bits, "kq": kq, "ks": ks, "km": km, "vq": vq, "vs": vs, "vm": vm}


def dequant_chunk(ch: dict):
    if ch["bits"] == 16:
        return ch["k"].astype(np.float64), ch["v"].astype(np.float64)
    return (dequant_k(ch["kq"], ch["ks"], ch["km"]),
            dequant_v(ch["vq"], ch["vs"], ch["vm"]))
