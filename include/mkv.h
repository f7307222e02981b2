/*
 * mkv.h — C ABI of libmkv.so: chunk-adaptive mixed-precision KV cache on
 * AMD MI355X (gfx950).
 *
 * The method (web sources, cited by page title and section):
 *   - "MoQAE: Mixed-Precision Quantization for Long-Context LLM Inference via
 *     Mixture of Quantization-Aware Experts" (Paper-Notes, ACL 2025):
 *       "Overall framework": text is split into equal-length chunks; a router
 *       scores every token against quantization "experts"; a vote inside each
 *       chunk picks the chunk's bitwidth; the KV cache is quantized at that
 *       bitwidth; attention then runs as usual.
 *       "Key designs": experts are FP16, INT4, INT2; router MLP over a chunk's
 *       hidden states; routing freezing (chunk 0 stays FP16); routing sharing
 *       (one routing for every block).
 *       "Related work" (KIVI): keys have outlier channels, so keys are
 *       quantized per channel.
 *   - Cocktail abstract (scholarfeed author page): chunks are reordered
 *     before quantization so that chunks of one bitwidth are contiguous and
 *     attention runs chunk by chunk without mixed-precision inefficiency.
 *
 * Three calls make the hot path:
 *   mkv_route_chunks              router -> per-token expert -> chunk vote ->
 *                                 freezing -> stable reorder tables
 *   mkv_quantize_pack_kv          K/V of routed chunks -> packed segment pools
 *   mkv_mixed_kv_decode_attention one query per sequence and query head over
 *                                 the packed pools (+ optional fp16 tail)
 *
 * Conventions shared by every call
 *   - Every pointer to tensor data is a DEVICE pointer; structs are passed by
 *     HOST pointer and hold device pointers.  The caller allocates and owns
 *     every buffer and keeps it alive until the stream work is done; the
 *     library allocates nothing and keeps no state between calls (the one
 *     exception, the no-allocation variant of call 3, keeps a fixed device
 *     array per GPU and its address).
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the default stream) and the call returns without synchronising.
 *   - Return value: MKV_OK (0) or a negative MKV_ERR_*.  Arguments are
 *     checked before anything is launched, so an argument error leaves every
 *     output untouched.  MKV_ERR_HIP means a HIP call failed; the HIP error
 *     code of the last such failure on the calling thread is returned by
 *     mkv_last_hip_error().
 *   - Every device buffer must be 16-byte aligned.
 *   - Bitwidths are 16 (FP16 expert, index 0), 4 (INT4, index 1) and
 *     2 (INT2, index 2).  Expert index order is precision order.
 */
#ifndef MKV_H_
#define MKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define MKV_OK               0
#define MKV_ERR_ARG         -1  /* null pointer, bad size, misalignment     */
#define MKV_ERR_UNSUPPORTED -2  /* shape outside what the kernels handle    */
#define MKV_ERR_WORKSPACE   -3  /* workspace missing or too small           */
#define MKV_ERR_HIP         -4  /* a HIP runtime call failed                */
#define MKV_ERR_SCRATCH     -5  /* more than the fixed scratch of the
                                   no-allocation entry point holds           */

/* ---- flags for mkv_route_chunks ---------------------------------------- */
#define MKV_FREEZE_FIRST 0x1u /* routing freezing: chunk 0 of each sequence
                                 becomes FP16 (MoQAE, "Key designs")       */
#define MKV_LOGITS_IN    0x2u /* skip the router: `logits` holds the final
                                 per-token expert scores to vote on        */
#define MKV_APPEND       0x4u /* the routed chunks start at chunk_offset;
                                 tables for chunks [0, chunk_offset) are
                                 kept and the reorder covers them too      */

/* ---- workspace query ops ------------------------------------------------ */
#define MKV_OP_ROUTE      1
#define MKV_OP_ATTENTION  2
#define MKV_OP_SIMILARITY 3
#define MKV_OP_PREFILL    4

/* Routing tables of a batch of sequences (routing sharing: one table serves
 * every layer and head).  All arrays are device memory, row stride n_max:
 *   chunk_bits [B][n_max] u8   16 / 4 / 2 for each chunk (in chunk order)
 *   chunk_rank [B][n_max] i32  slot of the chunk inside its bitwidth segment
 *   perm       [B][n_max] i32  segment-order position -> chunk index
 *                              (FP16 segment, then INT4, then INT2; chunk
 *                              order kept inside a segment)
 *   seg_count  [B][3]     i32  chunks in the FP16, INT4 and INT2 segments   */
typedef struct mkv_tables {
    uint8_t* chunk_bits;
    int32_t* chunk_rank;
    int32_t* perm;
    int32_t* seg_count;
    int n_max;
} mkv_tables;

/* One layer's packed cache.  pool[k] (k = 0 FP16, 1 INT4, 2 INT2) is device
 * memory of mkv_pool_bytes(k-th bitwidth, B, Hkv, cap[k], d, C) bytes, laid
 * out [B][Hkv][cap[k] slots][C/32 groups][group block].  The chunk of
 * sequence b with bitwidth index k and rank r lives at slot r of every head
 * (b, h).  The segment of (b, h, k) is therefore one contiguous run of
 * seg_count[b][k]*C/32 group blocks.
 *
 * A group block holds 32 consecutive tokens of one (sequence, KV head).
 * Let S = d/8 ("lane slots"), NG = d/32 (value groups per token) and let
 * a "row" of a section be S 16-byte cells, cell L belonging to lane slot L.
 * A group block is four sections in this order, each section being a run of
 * rows (row index = "load index"):
 *
 *   INT-b (b = 4 or 2), F = 32/b codes per 32-bit word, LSB first:
 *     K meta    4 rows: row 0 / 1 = scale of channels 8L+0..3 / 8L+4..7,
 *               row 2 / 3 = min of the same channels (float32).  Key groups
 *               run along tokens: one (scale, min) per channel for the 32
 *               tokens of the block.
 *     K codes   rows 0 .. 2b-1: lane slot L owns channels 8L..8L+7; for
 *               channel j = 8L + 4*(row & 1) + e (e = dword in the cell) the
 *               cell holds word w = row >> 1 of that channel.  Field i of word
 *               w of lane slot L is the key code of token tok(L, F*w + i):
 *                 tok(L, r) = (r & 16) | ((r & 15) XOR f_S(L)),
 *                 f_16(L) = 1*L0 ^ 2*L1 ^ 7*L2 ^ 12*L3   (d = 128)
 *                 f_8(L)  = 2*L0 ^ 4*L1 ^ 14*L2           (d = 64)
 *               where Lk is bit k of L.
 *     V meta    4 rows: lane slot L has value group G = L % NG and token
 *               quarter tq = L / NG and covers tokens t_m = tq + 4m,
 *               m = 0..7.  Row m holds (scale, min) of token t_{2m} then
 *               (scale, min) of token t_{2m+1}, for group G (float32).  Value
 *               groups run along channels: one (scale, min) per (token, 32
 *               channels).
 *     V codes   2b rows over channels 32G..32G+31 of the lane's tokens.
 *               INT4: row m holds words u = 0..3 of token t_m, word u =
 *               channels 32G+8u .. +7.  INT2: row m holds the two words of
 *               token t_{2m} then those of t_{2m+1} (word u = channels
 *               32G+16u .. +15).
 *   FP16 (bit-for-bit copies):
 *     K         32 rows: row r holds channels 8L..8L+7 of token tok(L, r).
 *     V         32 rows: row r holds channels 32G + 8*(r & 3) .. +7 of token
 *               t_{r >> 2} (G, t_m as for INT-b values).
 *   Group block bytes: FP16 64*S*16, INT4 24*S*16, INT2 16*S*16.
 * The layout lets each lane of a 64-wide wavefront issue whole-row 16-byte
 * loads that are contiguous across the lane slots of a row.  Quantization
 * itself (which values share a scale) does not depend on the layout.     */
typedef struct mkv_cache {
    int B, Hkv, d, C;
    int cap[3];                 /* slots per (sequence, head) in each pool  */
    void* pool[3];              /* device; pool[k] may be NULL if cap[k]==0 */
    const int32_t* seg_count;   /* device [B][3] (usually tables.seg_count) */
    int32_t* overflow;          /* device i32 or NULL: set to 1 by
                                   mkv_quantize_pack_kv when a chunk's rank
                                   does not fit cap[k] (that chunk is then
                                   not written)                             */
} mkv_cache;

/* ------------------------------------------------------------------------
 * 1. mkv_route_chunks — router, chunk vote, routing freezing, reorder.
 *    MoQAE "Key designs" (Quantization-Aware Experts; routing freezing;
 *    routing sharing) and Cocktail abstract (reorder before quantization).
 *
 * Routes T tokens (= T/C new chunks) of each of B sequences.  Per token:
 *   z = SiLU((x W1^T) .* (x W2^T)) W3^T + b3        (3 logits, fp32)
 * with bf16 inputs and fp32 accumulation (MFMA); the expert is the argmax
 * (ties to the lower index).  Per chunk: plurality vote over its C tokens
 * (ties to the lower index); with MKV_FREEZE_FIRST chunk 0 becomes FP16.
 * The chunk bitwidths land in tab->chunk_bits[b][chunk_offset + c]; then
 * chunk_rank, perm and seg_count are recomputed over chunks
 * [0, chunk_offset + T/C) of each sequence (stable partition FP16, INT4, INT2).
 *
 *   x_bf16     [B][T][D] bf16 hidden states (ignored with MKV_LOGITS_IN)
 *   w12_bf16   [2I][D] bf16, rows 0..I-1 = W1, rows I..2I-1 = W2
 *   w3         [3][I] fp32;   b3 [3] fp32
 *   logits     [B][T][3] fp32: output if non-NULL; with MKV_LOGITS_IN it is
 *              the input (final scores, b3 not added) and must be non-NULL
 *   token_expert [B][T] u8 output (expert index per token) or NULL
 *   chunk_offset must be 0 unless MKV_APPEND is set; chunk_offset + T/C
 *              must not exceed tab->n_max.
 *   workspace  device scratch of at least
 *              mkv_workspace_bytes(MKV_OP_ROUTE, B, T, D, I, ...) bytes.
 * Limits: T % C == 0, C % 32 == 0, 32 <= C <= 1024; D % 64 == 0;
 *         I % 128 == 0 and 2*I*D*2 bytes of W12 < 4 GiB (router mode).
 * ---------------------------------------------------------------------- */
int mkv_route_chunks(const void* x_bf16, const void* w12_bf16,
                     const float* w3, const float* b3, float* logits,
                     int B, int T, int D, int I, int C, unsigned flags,
                     uint8_t* token_expert, const mkv_tables* tab,
                     int chunk_offset, void* workspace,
                     size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * 1b. mkv_select_chunks_by_similarity — bitwidths from query-chunk
 *    similarity instead of the router (Cocktail abstract: chunk-level
 *    quantization search), then the same reorder tables as call 1.
 *
 *   x_bf16     [B][T][D] bf16 embeddings of the T = n_new*C tokens of chunks
 *              chunk_offset .. chunk_offset+n_new-1 of each sequence
 *   qe_bf16    [B][D] bf16 query embedding of each sequence
 *   tau_hi, tau_lo  thresholds, tau_lo <= tau_hi
 *   sim        [B][n_new] fp32 out (optional, may be NULL): each new
 *              chunk's similarity
 *   flags      MKV_FREEZE_FIRST (chunk 0 of each sequence FP16) | MKV_APPEND
 *   tab, chunk_offset   as in call 1 (chunk_offset must be 0 without
 *              MKV_APPEND)
 *   workspace  at least mkv_workspace_bytes(MKV_OP_SIMILARITY, ...) bytes
 * A chunk's similarity is the cosine between the sum (the direction of the
 * mean) of its tokens' embeddings and the query embedding, in fp32, or 0
 * when either vector is zero.  Its bitwidth is 16 when sim >= tau_hi, 4
 * when tau_lo <= sim < tau_hi, 2 otherwise.  The reorder then covers chunks
 * [0, chunk_offset + n_new) exactly as in call 1.
 * Limits: D % 64 == 0; C % 32 == 0, C <= 1024; B, n_new <= 65535.
 * ---------------------------------------------------------------------- */
int mkv_select_chunks_by_similarity(const void* x_bf16, const void* qe_bf16,
                                    int B, int T, int D, int C,
                                    float tau_hi, float tau_lo, unsigned flags,
                                    float* sim, const mkv_tables* tab,
                                    int chunk_offset, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * 2. mkv_quantize_pack_kv — quantize and pack the K/V of routed chunks.
 *    MoQAE "Overall framework" (cache quantized at the voted bitwidth) and
 *    "Related work" (keys per channel); Cocktail abstract (chunks written to
 *    their bitwidth's contiguous segment).
 *
 *   k_fp16, v_fp16  [B][Hkv][T][d] fp16, the T = n_new*C tokens of chunks
 *                   chunk_offset .. chunk_offset+n_new-1 of each sequence
 *   tab             tables from mkv_route_chunks (chunk_bits, chunk_rank)
 *   cache           destination; B, Hkv, d, C are taken from it
 * FP16 chunks are copied bit for bit.  INT-b chunks (b = 4, 2, L = 2^b-1)
 * use asymmetric min-max codes on groups of 32 values (keys: 32 tokens of
 * one channel; values: 32 channels of one token), in float32 with one
 * rounding per operation:
 *   mn = min, mx = max (a -0 extreme becomes +0), s = (mx - mn) / L, r = 1 / s,
 *   code = clamp(round_half_even((x - mn) * r), 0, L); s == 0 -> codes 0.
 * Dequantization is x = code * s + mn.
 * Limits: as for the cache; T % C == 0.
 * ---------------------------------------------------------------------- */
int mkv_quantize_pack_kv(const void* k_fp16, const void* v_fp16, int T,
                         int chunk_offset, const mkv_tables* tab,
                         const mkv_cache* cache, void* stream);

/* ------------------------------------------------------------------------
 * 3. mkv_mixed_kv_decode_attention — one decode step over the mixed cache.
 *    MoQAE "Overall framework" (ordinary attention after quantization) and
 *    Cocktail abstract (chunk-level computation over reordered segments).
 *
 * For each sequence b and query head hq (KV head h = hq / (Hq/Hkv)):
 *   out[b][hq] = softmax(q k^T / sqrt(d)) v
 * over every cached token of (b, h) (all segments, in any order: attention
 * does not depend on key order) plus the tail_len fp16 tokens of the tail.
 * Cached values are dequantized in registers; accumulation is fp32.  One
 * launch splits the whole cache into ranges of equal cost (bytes weighted
 * by each bitwidth's work per byte), one per workgroup, whose wavefronts
 * take single-bitwidth work units dynamically; a second launch merges the
 * partials of each (sequence, KV head) with a log-sum-exp combine.  Because units are handed out dynamically, the fp32
 * summation order (not the result beyond rounding) can differ between calls.
 *
 *   q_fp16      [B][Hq][d] fp16
 *   tail_k/v    [B][Hkv][tail_stride][d] fp16, tokens 0 .. tail_len-1 of
 *               each row used; NULL when tail_len == 0
 *   tail_stride tokens between consecutive (sequence, head) rows of the
 *               tail, >= tail_len; 0 means tail_len (a packed tail).  A
 *               decode loop keeps a tail buffer of C rows and passes C.
 *   out         [B][Hq][d] fp32
 *   workspace   at least mkv_workspace_bytes(MKV_OP_ATTENTION, ...) bytes
 *               (tile partials; no initial contents needed).  Calls that
 *               overlap in time need separate workspaces.
 * Query heads per KV head: any Hq/Hkv up to 64.  The kernels attend the
 * query heads of a KV head in groups of 4, 2 and 1 (as many groups of 4 as
 * fit, then one of 2, then one of 1), one launch pair per group, each
 * reading the KV head's cache: with 1, 2 or 4 heads per KV head the cache is
 * read once, with 8 twice, with 6 (4 + 2) twice, with 3 (2 + 1) twice.
 * Limits: d in {64, 128}; Hq/Hkv <= 64; 0 <= tail_len < 4096; the
 * pools at capacity within 2^31 work-split granules of 512 bytes (weighted
 * by bitwidth: 0.6 to 1 TiB of packed cache), else MKV_ERR_UNSUPPORTED.
 * A (b, h) with no cached token and tail_len == 0 yields zeros.
 * ---------------------------------------------------------------------- */
int mkv_mixed_kv_decode_attention(const void* q_fp16, int Hq,
                                  const mkv_cache* cache,
                                  const void* tail_k_fp16,
                                  const void* tail_v_fp16, int tail_len,
                                  int tail_stride, float* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * 3'. mkv_mixed_kv_decode_attention_noalloc — call 3 without a workspace,
 *    for callers that cannot allocate device memory (code under HIP graph
 *    capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, result and limits as mkv_mixed_kv_decode_attention, minus
 * the workspace: the tile partials go to a fixed device array of
 * MKV_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held from
 * the first call on that GPU until the process ends.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * call on a device looks the array's device address up with that device
 * current.  The stream must belong to the calling thread's current device.
 *   Returns MKV_ERR_SCRATCH, before any launch, when the call would need
 *   more than MKV_NOALLOC_SCRATCH_BYTES of partials, i.e. when
 *   mkv_workspace_bytes(MKV_OP_ATTENTION, ...) exceeds it (for d = 128
 *   about (B*Hkv + 256) * min(Hq/Hkv, 4) <= 15800).
 *   Every call on one GPU shares that GPU's array, so calls that overlap in
 *   time on one GPU (other streams, other threads) race and must not be
 *   issued; calls on one stream are ordered and safe.  No part of the array
 *   needs initial contents: each call writes every partial it reads.
 * ---------------------------------------------------------------------- */
#define MKV_NOALLOC_SCRATCH_BYTES (8u << 20)
int mkv_mixed_kv_decode_attention_noalloc(const void* q_fp16, int Hq,
                                          const mkv_cache* cache,
                                          const void* tail_k_fp16,
                                          const void* tail_v_fp16,
                                          int tail_len, int tail_stride,
                                          float* out, void* stream);

/* ------------------------------------------------------------------------
 * 3b. mkv_mixed_kv_prefill_attention — chunked prefill over the mixed cache:
 *    a chunk of P new tokens attends before it is quantized (MoQAE "Overall
 *    framework": ordinary attention; Cocktail abstract: chunk-level
 *    computation over the bitwidth segments).
 *
 * For each sequence b, query head hq (KV head h = hq / (Hq/Hkv)) and query
 * i < P: out[b][hq][i] = softmax(q k^T / sqrt(d)) v over every cached token
 * of (b, h) and the new tokens 0..i of k_new/v_new (causal).  Cached values
 * are dequantized to fp16 tiles and multiplied on the matrix cores with fp32
 * accumulation; the splits of the cache are merged with a log-sum-exp
 * combine.
 *
 *   q_fp16      [B][Hq][P][d] fp16
 *   k_new/v_new [B][Hkv][P][d] fp16: the chunk's own keys and values
 *   out         [B][Hq][P][d] fp32
 *   workspace   at least mkv_workspace_bytes(MKV_OP_PREFILL, ...) bytes
 * Limits: d in {64, 128}; Hq % Hkv == 0; 1 <= P <= 65535; B*Hq <= 65535.
 * ---------------------------------------------------------------------- */
int mkv_mixed_kv_prefill_attention(const void* q_fp16, int Hq, int P,
                                   const mkv_cache* cache,
                                   const void* k_new_fp16,
                                   const void* v_new_fp16, float* out,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/* ------------------------------------------------------------------------
 * Streaming decode helpers: the step either side of the path (MoQAE
 * "Overall framework": the context is cut into equal chunks as it grows).
 * Tokens of a partial chunk wait in an fp16 tail that attention reads
 * directly; a full tail is routed, quantized and appended as one chunk.
 *
 * mkv_append_tail_rows: copy row r of `a_new` (and of `b_new`, if not NULL)
 * into row r, token `pos` of the tail `a_tail` (`b_tail`), for r < rows:
 *   a_new, b_new    [rows][width] 2-byte elements (fp16 K/V of one token
 *                   per (sequence, head): rows = B*Hkv, width = d; or bf16
 *                   hidden states: rows = B, width = D)
 *   a_tail, b_tail  [rows][tail_stride][width]
 * 0 <= pos < tail_stride.  width % 8 == 0; buffers 16-byte aligned.
 *
 * mkv_grow_pool: copy a pool of `bits` laid out for cap_old slots per
 * (sequence, head) into a pool laid out for cap_new >= cap_old slots (see
 * mkv_cache).  Slots cap_old .. cap_new-1 of dst are left as they were.
 * src and dst must not overlap.
 * ---------------------------------------------------------------------- */
int mkv_append_tail_rows(const void* a_new, const void* b_new, void* a_tail,
                         void* b_tail, int rows, int width, int tail_stride,
                         int pos, void* stream);
int mkv_grow_pool(const void* src, void* dst, int bits, int B, int Hkv,
                  int cap_old, int cap_new, int d, int C, void* stream);

/* ---- helpers -------------------------------------------------------------
 * mkv_workspace_bytes: scratch needed by an op.
 *   MKV_OP_ROUTE:     a = B, b = T, c = D, e = I (f, g unused)
 *   MKV_OP_ATTENTION: a = B, b = Hq, c = Hkv, e = d, f = C, and `cache_caps`
 *                     points to the cache's cap[3] (host memory)
 *   MKV_OP_SIMILARITY: a = B, b = T, c = D, e = C (f, cache_caps unused)
 *   MKV_OP_PREFILL:   a = B, b = Hq, c = P, e = d, f = C, and `cache_caps`
 *                     points to the cache's cap[3] (host memory)
 * Returns 0 for an unknown op or invalid sizes.                          */
size_t mkv_workspace_bytes(int op, int a, int b, int c, int e, int f,
                           const int* cache_caps);

/* Bytes of one group block (32 tokens of one head) and of one pool. */
size_t mkv_group_bytes(int bits, int d);
size_t mkv_pool_bytes(int bits, int B, int Hkv, int cap, int d, int C);

const char* mkv_status_string(int status);
int mkv_last_hip_error(void);
int mkv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MKV_H_ */
