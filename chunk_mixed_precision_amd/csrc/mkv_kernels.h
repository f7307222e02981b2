// Kernel parameter blocks and kernel declarations of libmkv.so (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace mkv {

// ---------------------------------------------------------------- router
constexpr int kRouterBM = 256;   // tokens per workgroup tile
constexpr int kRouterBI = 128;   // inner indices per workgroup tile (128 W1 + 128 W2 rows)
constexpr int kRouterBK = 64;    // K step staged in LDS
constexpr int kRouterWaves = 8;  // wavefronts per router workgroup
constexpr int kRouterStages = 2; // LDS ring depth of the router GEMM

struct RouterParams {
    const uint16_t* x;      // [M][D] bf16 bits
    const uint16_t* w12;    // [2I][D] bf16 bits
    const float* w3;        // [3][I]
    float* zpart;           // [I/kRouterBI][M][3] partial logits
    int M, D, I;
};

struct VoteParams {
    const float* zpart;     // router mode: [ntile][M][3]; NULL in logits-in mode
    int ntile;
    const float* b3;        // [3] (router mode)
    const float* logits_in; // logits-in mode: [B][T][3]
    float* logits_out;      // router mode, optional
    uint8_t* token_expert;  // optional [B][T]
    uint8_t* chunk_bits;    // [B][n_max]
    int B, T, C, n_max, chunk_offset;
    int freeze_first;
};

// Optional first step of the reorder: chunk bitwidths from the similarity
// partials (sel_part == nullptr: the bitwidths are already in the table).
struct SelectStep {
    const float4* sel_part; // [B][n_new][ds] partials of sim_partial_kernel
    float* sim;             // [B][n_new] out, optional
    uint8_t* chunk_bits;    // the table's bitwidths (written for the new chunks)
    int first, n_new, ds;   // new chunks first .. first + n_new - 1
    float tau_hi, tau_lo;
    int freeze_first;
};

struct ReorderParams {
    const uint8_t* chunk_bits;
    int32_t* chunk_rank;
    int32_t* perm;
    int32_t* seg_count;
    int n_total, n_max;
    int32_t* bad;           // optional: set when a chunk's bitwidth is invalid
    SelectStep sel;
};

// ---------------------------------------------------------------- similarity selection
constexpr int kSimSlice = 512;          // embedding dims per partial-sum workgroup (64 lanes x 8)

struct SimParams {
    const uint16_t* x;      // [B][T][D] bf16 embeddings of the new chunks' tokens
    const uint16_t* qe;     // [B][D] bf16 query embeddings
    float4* part;           // [B][n_new][ds]: (q.S, |S|^2, |q|^2, 0) per dim slice
    int B, T, D, C, ds;
};

// ---------------------------------------------------------------- chunked prefill
struct PrefillParams {
    const uint16_t* q;      // [B][Hq][P][d] fp16 queries of the new chunk
    const uint8_t* pool[3];
    int cap[3];
    const int32_t* seg_count;
    const uint16_t* k_new;  // [B][Hkv][P][d] fp16: the chunk's own keys / values
    const uint16_t* v_new;
    float* part;            // [B][Hq][P][NS][d+4]: o[d], m (log2 domain), l, 0, 0
    float* out;             // [B][Hq][P][d]
    int B, Hq, Hkv, C, P, NS;
    float qscale;           // log2(e) / sqrt(d)
};

// ---------------------------------------------------------------- quantize
struct QuantParams {
    const uint16_t* k;      // [B][Hkv][T][d] fp16 bits
    const uint16_t* v;
    int B, Hkv, T, C, chunk_offset, n_max;
    const uint8_t* chunk_bits;
    const int32_t* chunk_rank;
    int cap[3];
    uint8_t* pool[3];
    int32_t* overflow;
};

// ---------------------------------------------------------------- attention
constexpr int kAttnWaves = 8;             // wavefronts per attention workgroup (2 per SIMD)
constexpr long long kAttnMinWgCost = 128 << 10;  // smallest cost range given to one workgroup
// The split counts costs in granules of this many bytes, in 32-bit integers;
// every unit's cost is a whole number of granules.
constexpr int kAttnGranule = 512;
// Largest whole-cache cost, in granules, that the split handles.
constexpr long long kAttnMaxGranules = (1LL << 31) - 1;
// Cost of a unit per byte, in sixteenths, for segment k (FP16, INT4, INT2)
// and hb query heads per KV head: the time per byte of a cache of that
// segment alone relative to INT4, measured per kernel variant.  With one head
// per KV head the kernel streams at the same rate on every segment; with
// grouped-query heads the arithmetic per byte counts (an INT2 byte holds
// twice the codes of an INT4 byte, an FP16 byte needs no unpacking).
// Equal-cost ranges finish together.
constexpr int attn_cost16(int hb, int k) {
    return hb == 1 ? 16
         : hb == 2 ? (k == 0 ? 11 : k == 1 ? 16 : 22)
                   : (k == 0 ? 9 : k == 1 ? 16 : 21);
}
// Rows of lanes per group block and heads per row, as the unit geometry
// sees them: with two query heads per KV head a row serves both (each code
// word is unpacked once for both); with four, a row pair shares a group
// block (split by data, both rows serving all four heads), which gives the
// same group blocks per wavefront iteration as two heads per row.
constexpr int attn_heads_per_row(int hb) { return hb == 1 ? 1 : 2; }

struct AttnParams {
    const uint16_t* q;      // [B][Hq][d]
    const uint8_t* pool[3];
    int cap[3];
    const int32_t* seg_count;
    int B, Hkv, Hq, C;
    int hpk;                // query heads per KV head in q and out (Hq / Hkv)
    int hoff;               // first query head of this launch's group within a KV head's heads
    int G;                  // workgroups launched (the device may use fewer)
    float* part;            // [B*Hkv + G][HB][d+4]: o[d], m (log2 domain), l, 0, 0
    const uint16_t* tail_k; // [B][Hkv][tail_stride][d] or NULL; tokens 0..tail_len-1 are used
    const uint16_t* tail_v;
    int tail_len;
    int tail_stride;        // tokens between consecutive (sequence, head) rows of the tail
    float* out;             // [B][Hq][d]
    float qscale;           // log2(e) / sqrt(d)
};

// Host-side launchers (each defined next to its kernels).
hipError_t launch_router(const RouterParams& rp, hipStream_t st);
hipError_t launch_vote(const VoteParams& vp, int n_new, hipStream_t st);
hipError_t launch_reorder(const ReorderParams& rp, int B, hipStream_t st);
hipError_t launch_quant(const QuantParams& qp, int D, int ngroups, hipStream_t st);
hipError_t launch_similarity(const SimParams& sp, hipStream_t st);
hipError_t launch_prefill(const PrefillParams& pp, int D, hipStream_t st);
hipError_t launch_copy_rows(const void* src, size_t spitch, void* dst, size_t dpitch, size_t row_bytes, int rows,
                            hipStream_t st);
hipError_t launch_attention(const AttnParams& ap, int D, int HB, hipStream_t st);

}  // namespace mkv
