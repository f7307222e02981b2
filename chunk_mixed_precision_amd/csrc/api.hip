// C ABI of libmkv.so: argument checks, workspace sizing and launches.
// Nothing here allocates device memory or keeps state between calls; every
// argument error is reported before the first launch.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mkv.h"
#include "mkv_internal.h"
#include "mkv_kernels.h"

namespace mkv {
int prefill_query_tile(int P);   // queries per prefill workgroup (defined with the kernels)
}

namespace {

thread_local int g_last_hip = 0;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline int hip_status(hipError_t e) {
    if (e == hipSuccess) return MKV_OK;
    g_last_hip = (int)e;
    return MKV_ERR_HIP;
}

// Attention work split: persistent workgroups of mkv::kAttnWaves wavefronts,
// one per CU (256 on MI355X), each taking an equal cost range of the cache;
// fewer when the cache at capacity is small (here counted in bytes: every
// range at least mkv::kAttnMinWgCost).  The device recomputes the split from
// the actual segment counts and unit costs and never uses more than this.  Partials: one record per
// (sequence, head) plus one per workgroup boundary.
constexpr long long kAttnWorkgroups = 256;

inline int attn_workgroups(int B, int Hkv, int d, const int* cap, int C) {
    const int bits[3] = {16, 4, 2};
    long long bh_bytes = 0;
    for (int k = 0; k < 3; ++k) bh_bytes += (long long)cap[k] * (C / mkv::kGroup) * (long long)mkv::group_bytes(bits[k], d);
    const long long total = bh_bytes * B * Hkv;
    long long g = total / mkv::kAttnMinWgCost;
    if (g > kAttnWorkgroups) g = kAttnWorkgroups;
    if (g < 1) g = 1;
    return (int)g;
}

// Chunked prefill: splits of each (sequence, query head)'s cached group
// blocks.  One 8-wavefront workgroup fits a CU at a time, so the grid runs in
// rounds of 256: take at least enough splits for one round, and more while
// the last round would be less than 90 % full; none shorter than 4 group
// blocks (counted at capacity), at most 32.
inline int prefill_splits(int B, int Hq, int P, const int* cap, int C) {
    const int qt = mkv::prefill_query_tile(P);
    const long long tiles = (long long)B * Hq * ((P + qt - 1) / qt);
    const long long gcap = ((long long)cap[0] + cap[1] + cap[2]) * (C / mkv::kGroup);
    long long lim = gcap / 4 < 32 ? gcap / 4 : 32;
    if (lim < 1) lim = 1;
    long long ns = (256 + tiles - 1) / tiles;
    if (ns > lim) ns = lim;
    while (ns < lim) {
        const long long wg = tiles * ns, rounds = (wg + 255) / 256;
        if (wg * 10 >= rounds * 256 * 9) break;
        ++ns;
    }
    return (int)ns;
}

inline bool valid_cache(const mkv_cache* c) {
    if (!c) return false;
    if (c->B <= 0 || c->Hkv <= 0 || c->C <= 0 || c->d <= 0) return false;
    for (int k = 0; k < 3; ++k) {
        if (c->cap[k] < 0) return false;
        if (c->cap[k] > 0 && (!c->pool[k] || !aligned16(c->pool[k]))) return false;
    }
    if (!c->seg_count) return false;
    return true;
}

inline int check_cache_shape(const mkv_cache* c) {
    if (c->d != 64 && c->d != 128) return MKV_ERR_UNSUPPORTED;
    if (c->C % 32 != 0 || c->C < 32 || c->C > 1024) return MKV_ERR_UNSUPPORTED;
    if ((long)c->B * c->Hkv > 65535) return MKV_ERR_UNSUPPORTED;
    return MKV_OK;
}


// The query heads of a KV head are attended in groups of 4, 2 and 1 (the
// kernels' shapes): as many groups of 4 as fit, then one of 2, then one of
// 1.  Each group is one tile + combine launch pair that reads the KV head's
// cache; with 1, 2 or 4 heads per KV head that is a single pair.  Returns
// the group count, sizes in hb[] and first heads in off[].
int attention_head_groups(int g, int* hb, int* off) {
    int n = 0, h = 0;
    while (g - h >= 4) { hb[n] = 4; off[n++] = h; h += 4; }
    if (g - h >= 2) { hb[n] = 2; off[n++] = h; h += 2; }
    if (g - h >= 1) { hb[n] = 1; off[n++] = h; h += 1; }
    return n;
}

// Decode attention: the argument checks shared by both entry points (no
// launch, no HIP call).  Resolves a tail_stride of 0 to tail_len.
int attention_args(const void* q_fp16, int Hq, const mkv_cache* cache, const void* tail_k_fp16,
                   const void* tail_v_fp16, int tail_len, int* tail_stride, const float* out) {
    if (!q_fp16 || !out || !aligned16(q_fp16) || !aligned16(out)) return MKV_ERR_ARG;
    if (!valid_cache(cache)) return MKV_ERR_ARG;
    int s = check_cache_shape(cache);
    if (s) return s;
    if (Hq <= 0 || Hq % cache->Hkv != 0) return MKV_ERR_ARG;
    const int g = Hq / cache->Hkv;
    if (g > 64) return MKV_ERR_UNSUPPORTED;
    if ((long)cache->B * Hq > 2147483647L) return MKV_ERR_UNSUPPORTED;
    if (tail_len < 0 || tail_len >= 4096) return MKV_ERR_ARG;
    if (tail_len > 0 && (!tail_k_fp16 || !tail_v_fp16)) return MKV_ERR_ARG;
    if (*tail_stride == 0) *tail_stride = tail_len;
    if (*tail_stride < tail_len) return MKV_ERR_ARG;
    // the work split counts the cost of the whole cache at capacity in
    // 32-bit granules (for each head group shape used)
    int hb[32], off[32];
    const int ngroups = attention_head_groups(g, hb, off);
    for (int i = 0; i < ngroups; ++i) {
        const int gg = hb[i];
        const int gpi = (512 / cache->d) * mkv::attn_heads_per_row(gg) / gg;   // group blocks per unit
        const int bits[3] = {16, 4, 2};
        long long gran = 0;
        for (int k = 0; k < 3; ++k) {
            const long long units = ((long long)cache->cap[k] * (cache->C / mkv::kGroup) + gpi - 1) / gpi;
            gran += units * ((long long)gpi * mkv::group_bytes(bits[k], cache->d) * mkv::attn_cost16(gg, k) /
                             (16 * mkv::kAttnGranule));
        }
        if (gran * cache->B * cache->Hkv > mkv::kAttnMaxGranules) return MKV_ERR_UNSUPPORTED;
    }
    return MKV_OK;
}

// Decode attention: the launch pairs (tile kernel, combine), one per head
// group, on checked arguments; `workspace` holds the tile partials of one
// pair at a time (the pairs run in stream order).
int attention_launch(const void* q_fp16, int Hq, const mkv_cache* cache, const void* tail_k_fp16,
                     const void* tail_v_fp16, int tail_len, int tail_stride, float* out, void* workspace,
                     hipStream_t st) {
    mkv::AttnParams ap{};
    ap.q = static_cast<const uint16_t*>(q_fp16);
    for (int k = 0; k < 3; ++k) {
        ap.pool[k] = static_cast<const uint8_t*>(cache->pool[k]);
        ap.cap[k] = cache->cap[k];
    }
    ap.seg_count = cache->seg_count;
    ap.B = cache->B; ap.Hkv = cache->Hkv; ap.Hq = Hq; ap.C = cache->C;
    ap.G = attn_workgroups(cache->B, cache->Hkv, cache->d, cache->cap, cache->C);
    ap.part = static_cast<float*>(workspace);
    ap.tail_k = static_cast<const uint16_t*>(tail_k_fp16);
    ap.tail_v = static_cast<const uint16_t*>(tail_v_fp16);
    ap.tail_len = tail_len;
    ap.tail_stride = tail_stride;
    ap.out = out;
    ap.qscale = (float)(1.4426950408889634 / sqrt((double)cache->d));
    ap.hpk = Hq / cache->Hkv;
    int hb[32], off[32];
    const int ngroups = attention_head_groups(ap.hpk, hb, off);
    for (int i = 0; i < ngroups; ++i) {
        ap.hoff = off[i];
        const int s = hip_status(mkv::launch_attention(ap, cache->d, hb[i], st));
        if (s) return s;
    }
    return MKV_OK;
}

// ---- the no-allocation variant of decode attention ----------------------
// Its tile partials live in `scratch`, a fixed device array that every GPU
// the library runs on holds until the process ends.  In host code the
// array's name is only a host-side stand-in, so kernels get the device
// address that hipGetSymbolAddress reports, looked up once per device (with
// that device current) on the first call there and kept per device.
constexpr size_t kScratchBytes = MKV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[MKV_NOALLOC_SCRATCH_BYTES];

namespace {

int scratch_of_current_device(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return MKV_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!p) return MKV_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MKV_OK;
}

}  // namespace

extern "C" {

int mkv_version(void) { return 1; }

int mkv_last_hip_error(void) { return g_last_hip; }

const char* mkv_status_string(int status) {
    switch (status) {
        case MKV_OK: return "ok";
        case MKV_ERR_ARG: return "invalid argument (null pointer, bad size or misaligned buffer)";
        case MKV_ERR_UNSUPPORTED: return "shape not supported by the kernels";
        case MKV_ERR_WORKSPACE: return "workspace missing or too small";
        case MKV_ERR_HIP: return "HIP runtime error (see mkv_last_hip_error)";
        case MKV_ERR_SCRATCH:
            return "the call needs more tile-partial space than the no-allocation entry point's fixed "
                   "device scratch holds (use mkv_mixed_kv_decode_attention with a workspace)";
        default: return "unknown status";
    }
}

size_t mkv_group_bytes(int bits, int d) {
    if ((bits != 16 && bits != 4 && bits != 2) || (d != 64 && d != 128)) return 0;
    return mkv::group_bytes(bits, d);
}

size_t mkv_pool_bytes(int bits, int B, int Hkv, int cap, int d, int C) {
    const size_t gb = mkv_group_bytes(bits, d);
    if (!gb || B < 0 || Hkv < 0 || cap < 0 || C <= 0 || C % 32) return 0;
    return (size_t)B * Hkv * cap * (C / 32) * gb;
}

size_t mkv_workspace_bytes(int op, int a, int b, int c, int e, int f, const int* caps) {
    if (op == MKV_OP_ROUTE) {
        const int B = a, T = b, I = e;
        if (B <= 0 || T <= 0 || I <= 0 || I % mkv::kRouterBI) return 0;
        return (size_t)(I / mkv::kRouterBI) * B * T * 3 * sizeof(float);
    }
    if (op == MKV_OP_SIMILARITY) {
        const int B = a, T = b, D = c, C = e;
        if (B <= 0 || T <= 0 || D <= 0 || C <= 0 || T % C) return 0;
        const size_t ds = ((size_t)D + mkv::kSimSlice - 1) / mkv::kSimSlice;
        return (size_t)B * (T / C) * ds * 16;
    }
    if (op == MKV_OP_PREFILL) {
        const int B = a, Hq = b, P = c, d = e, C = f;
        if (!caps || B <= 0 || Hq <= 0 || P <= 0 || (d != 64 && d != 128) || C <= 0 || C % 32) return 0;
        const int ns = prefill_splits(B, Hq, P, caps, C);
        return (size_t)B * Hq * P * ns * (d + 4) * sizeof(float) + 16;
    }
    if (op == MKV_OP_ATTENTION) {
        const int B = a, Hq = b, Hkv = c, d = e, C = f;
        if (!caps || B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || (d != 64 && d != 128) || C <= 0 || C % 32) return 0;
        const int G = attn_workgroups(B, Hkv, d, caps, C);
        // records of one head group at a time: at most 4 heads
        const int hb = Hq / Hkv < 4 ? Hq / Hkv : 4;
        return ((size_t)B * Hkv + G) * hb * (d + 4) * sizeof(float) + 16;
    }
    return 0;
}

int mkv_route_chunks(const void* x_bf16, const void* w12_bf16, const float* w3, const float* b3,
                     float* logits, int B, int T, int D, int I, int C, unsigned flags,
                     uint8_t* token_expert, const mkv_tables* tab, int chunk_offset,
                     void* workspace, size_t workspace_bytes, void* stream) {
    const bool logits_in = (flags & MKV_LOGITS_IN) != 0;
    const bool append = (flags & MKV_APPEND) != 0;
    if (flags & ~(MKV_FREEZE_FIRST | MKV_LOGITS_IN | MKV_APPEND)) return MKV_ERR_ARG;
    if (!tab || !tab->chunk_bits || !tab->chunk_rank || !tab->perm || !tab->seg_count) return MKV_ERR_ARG;
    if (B <= 0 || T <= 0 || C <= 0) return MKV_ERR_ARG;
    if (C % 32 != 0 || C > 1024 || T % C != 0) return MKV_ERR_UNSUPPORTED;
    if (chunk_offset < 0 || (!append && chunk_offset != 0)) return MKV_ERR_ARG;
    const int n_new = T / C;
    if (tab->n_max <= 0 || chunk_offset + n_new > tab->n_max) return MKV_ERR_ARG;
    if (B > 65535 || n_new > 2147483647 / 1) return MKV_ERR_UNSUPPORTED;
    if (logits_in) {
        if (!logits || !aligned16(logits)) return MKV_ERR_ARG;
    } else {
        if (!x_bf16 || !w12_bf16 || !w3 || !b3) return MKV_ERR_ARG;
        if (!aligned16(x_bf16) || !aligned16(w12_bf16) || !aligned16(w3)) return MKV_ERR_ARG;
        if (logits && !aligned16(logits)) return MKV_ERR_ARG;
        if (D <= 0 || I <= 0) return MKV_ERR_ARG;
        if (D % 64 != 0 || I % mkv::kRouterBI != 0) return MKV_ERR_UNSUPPORTED;
        // the GEMM addresses the 2I weight rows with 32-bit byte offsets
        if ((size_t)2 * I * D * sizeof(uint16_t) > 0xFFFFFFFFull) return MKV_ERR_UNSUPPORTED;
        const size_t need = mkv_workspace_bytes(MKV_OP_ROUTE, B, T, D, I, 0, nullptr);
        if (!workspace || !aligned16(workspace) || workspace_bytes < need) return MKV_ERR_WORKSPACE;
        if ((long)B * T > 2147483647L) return MKV_ERR_UNSUPPORTED;
    }
    hipStream_t st = (hipStream_t)stream;
    const int M = B * T;
    if (!logits_in) {
        mkv::RouterParams rp{static_cast<const uint16_t*>(x_bf16), static_cast<const uint16_t*>(w12_bf16), w3,
                             static_cast<float*>(workspace), M, D, I};
        int s = hip_status(mkv::launch_router(rp, st));
        if (s) return s;
    }
    mkv::VoteParams vp{};
    vp.zpart = logits_in ? nullptr : static_cast<const float*>(workspace);
    vp.ntile = logits_in ? 0 : I / mkv::kRouterBI;
    vp.b3 = b3;
    vp.logits_in = logits_in ? logits : nullptr;
    vp.logits_out = logits_in ? nullptr : logits;
    vp.token_expert = token_expert;
    vp.chunk_bits = tab->chunk_bits;
    vp.B = B; vp.T = T; vp.C = C; vp.n_max = tab->n_max; vp.chunk_offset = chunk_offset;
    vp.freeze_first = (flags & MKV_FREEZE_FIRST) ? 1 : 0;
    int s = hip_status(mkv::launch_vote(vp, n_new, st));
    if (s) return s;
    mkv::ReorderParams op{tab->chunk_bits, tab->chunk_rank, tab->perm, tab->seg_count,
                          chunk_offset + n_new, tab->n_max, nullptr};
    return hip_status(mkv::launch_reorder(op, B, st));
}

int mkv_select_chunks_by_similarity(const void* x_bf16, const void* qe_bf16, int B, int T, int D, int C,
                                    float tau_hi, float tau_lo, unsigned flags, float* sim,
                                    const mkv_tables* tab, int chunk_offset, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    const bool append = (flags & MKV_APPEND) != 0;
    if (flags & ~(MKV_FREEZE_FIRST | MKV_APPEND)) return MKV_ERR_ARG;
    if (!tab || !tab->chunk_bits || !tab->chunk_rank || !tab->perm || !tab->seg_count) return MKV_ERR_ARG;
    if (!x_bf16 || !qe_bf16 || !aligned16(x_bf16) || !aligned16(qe_bf16)) return MKV_ERR_ARG;
    if (sim && !aligned16(sim)) return MKV_ERR_ARG;
    if (B <= 0 || T <= 0 || C <= 0 || D <= 0) return MKV_ERR_ARG;
    if (!(tau_lo <= tau_hi)) return MKV_ERR_ARG;   // also rejects NaN thresholds
    if (C % 32 != 0 || C > 1024 || T % C != 0 || D % 64 != 0) return MKV_ERR_UNSUPPORTED;
    if (chunk_offset < 0 || (!append && chunk_offset != 0)) return MKV_ERR_ARG;
    const int n_new = T / C;
    if (tab->n_max <= 0 || chunk_offset + n_new > tab->n_max) return MKV_ERR_ARG;
    if (B > 65535 || n_new > 65535) return MKV_ERR_UNSUPPORTED;
    const size_t need = mkv_workspace_bytes(MKV_OP_SIMILARITY, B, T, D, C, 0, nullptr);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need) return MKV_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    mkv::SimParams sp{};
    sp.x = static_cast<const uint16_t*>(x_bf16);
    sp.qe = static_cast<const uint16_t*>(qe_bf16);
    sp.part = static_cast<float4*>(workspace);
    sp.B = B; sp.T = T; sp.D = D; sp.C = C;
    sp.ds = (D + mkv::kSimSlice - 1) / mkv::kSimSlice;
    int s = hip_status(mkv::launch_similarity(sp, st));
    if (s) return s;
    mkv::ReorderParams op{tab->chunk_bits, tab->chunk_rank, tab->perm, tab->seg_count,
                          chunk_offset + n_new, tab->n_max, nullptr, {}};
    op.sel = mkv::SelectStep{sp.part, sim, tab->chunk_bits, chunk_offset, n_new, sp.ds, tau_hi, tau_lo,
                             (flags & MKV_FREEZE_FIRST) ? 1 : 0};
    return hip_status(mkv::launch_reorder(op, B, st));
}

int mkv_quantize_pack_kv(const void* k_fp16, const void* v_fp16, int T, int chunk_offset,
                         const mkv_tables* tab, const mkv_cache* cache, void* stream) {
    if (!k_fp16 || !v_fp16 || !aligned16(k_fp16) || !aligned16(v_fp16)) return MKV_ERR_ARG;
    if (!tab || !tab->chunk_bits || !tab->chunk_rank) return MKV_ERR_ARG;
    if (!valid_cache(cache)) return MKV_ERR_ARG;
    int s = check_cache_shape(cache);
    if (s) return s;
    if (T <= 0 || T % cache->C != 0) return MKV_ERR_ARG;
    if (chunk_offset < 0 || chunk_offset + T / cache->C > tab->n_max) return MKV_ERR_ARG;
    if ((long)T / 32 > 2147483647L) return MKV_ERR_UNSUPPORTED;
    mkv::QuantParams qp{};
    qp.k = static_cast<const uint16_t*>(k_fp16);
    qp.v = static_cast<const uint16_t*>(v_fp16);
    qp.B = cache->B; qp.Hkv = cache->Hkv; qp.T = T; qp.C = cache->C;
    qp.chunk_offset = chunk_offset; qp.n_max = tab->n_max;
    qp.chunk_bits = tab->chunk_bits; qp.chunk_rank = tab->chunk_rank;
    for (int k = 0; k < 3; ++k) {
        qp.cap[k] = cache->cap[k];
        qp.pool[k] = static_cast<uint8_t*>(cache->pool[k]);
    }
    qp.overflow = cache->overflow;
    return hip_status(mkv::launch_quant(qp, cache->d, T / 32, (hipStream_t)stream));
}

int mkv_mixed_kv_decode_attention(const void* q_fp16, int Hq, const mkv_cache* cache,
                                  const void* tail_k_fp16, const void* tail_v_fp16, int tail_len, int tail_stride,
                                  float* out, void* workspace, size_t workspace_bytes, void* stream) {
    int s = attention_args(q_fp16, Hq, cache, tail_k_fp16, tail_v_fp16, tail_len, &tail_stride, out);
    if (s) return s;
    const size_t need = mkv_workspace_bytes(MKV_OP_ATTENTION, cache->B, Hq, cache->Hkv, cache->d, cache->C, cache->cap);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need) return MKV_ERR_WORKSPACE;
    return attention_launch(q_fp16, Hq, cache, tail_k_fp16, tail_v_fp16, tail_len, tail_stride, out, workspace,
                            (hipStream_t)stream);
}

int mkv_mixed_kv_decode_attention_noalloc(const void* q_fp16, int Hq, const mkv_cache* cache,
                                          const void* tail_k_fp16, const void* tail_v_fp16, int tail_len,
                                          int tail_stride, float* out, void* stream) {
    int s = attention_args(q_fp16, Hq, cache, tail_k_fp16, tail_v_fp16, tail_len, &tail_stride, out);
    if (s) return s;
    const size_t need = mkv_workspace_bytes(MKV_OP_ATTENTION, cache->B, Hq, cache->Hkv, cache->d, cache->C, cache->cap);
    if (need == 0 || need > kScratchBytes) return MKV_ERR_SCRATCH;
    void* ws = nullptr;
    s = scratch_of_current_device(&ws);
    if (s) return s;
    return attention_launch(q_fp16, Hq, cache, tail_k_fp16, tail_v_fp16, tail_len, tail_stride, out, ws,
                            (hipStream_t)stream);
}

int mkv_mixed_kv_prefill_attention(const void* q_fp16, int Hq, int P, const mkv_cache* cache,
                                   const void* k_new_fp16, const void* v_new_fp16, float* out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    if (!q_fp16 || !out || !k_new_fp16 || !v_new_fp16) return MKV_ERR_ARG;
    if (!aligned16(q_fp16) || !aligned16(out) || !aligned16(k_new_fp16) || !aligned16(v_new_fp16)) return MKV_ERR_ARG;
    if (!valid_cache(cache)) return MKV_ERR_ARG;
    int s = check_cache_shape(cache);
    if (s) return s;
    if (Hq <= 0 || Hq % cache->Hkv != 0 || P <= 0) return MKV_ERR_ARG;
    if (P > 65535 || (long long)cache->B * Hq > 65535) return MKV_ERR_UNSUPPORTED;
    const size_t need = mkv_workspace_bytes(MKV_OP_PREFILL, cache->B, Hq, P, cache->d, cache->C, cache->cap);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need) return MKV_ERR_WORKSPACE;
    mkv::PrefillParams pp{};
    pp.q = static_cast<const uint16_t*>(q_fp16);
    for (int k = 0; k < 3; ++k) {
        pp.pool[k] = static_cast<const uint8_t*>(cache->pool[k]);
        pp.cap[k] = cache->cap[k];
    }
    pp.seg_count = cache->seg_count;
    pp.k_new = static_cast<const uint16_t*>(k_new_fp16);
    pp.v_new = static_cast<const uint16_t*>(v_new_fp16);
    pp.part = static_cast<float*>(workspace);
    pp.out = out;
    pp.B = cache->B; pp.Hq = Hq; pp.Hkv = cache->Hkv; pp.C = cache->C; pp.P = P;
    pp.NS = prefill_splits(cache->B, Hq, P, cache->cap, cache->C);
    pp.qscale = (float)(1.4426950408889634 / sqrt((double)cache->d));
    return hip_status(mkv::launch_prefill(pp, cache->d, (hipStream_t)stream));
}

int mkv_append_tail_rows(const void* a_new, const void* b_new, void* a_tail, void* b_tail, int rows, int width,
                         int tail_stride, int pos, void* stream) {
    if (!a_new || !a_tail || (b_new == nullptr) != (b_tail == nullptr)) return MKV_ERR_ARG;
    if (!aligned16(a_new) || !aligned16(a_tail) || (b_new && (!aligned16(b_new) || !aligned16(b_tail))))
        return MKV_ERR_ARG;
    if (rows <= 0 || width <= 0 || tail_stride <= 0 || pos < 0 || pos >= tail_stride) return MKV_ERR_ARG;
    if (width % 8) return MKV_ERR_UNSUPPORTED;
    hipStream_t st = (hipStream_t)stream;
    const size_t rb = (size_t)width * 2, pitch = (size_t)tail_stride * rb;
    int s = hip_status(mkv::launch_copy_rows(a_new, rb, static_cast<char*>(a_tail) + (size_t)pos * rb, pitch, rb,
                                             rows, st));
    if (s || !b_new) return s;
    return hip_status(mkv::launch_copy_rows(b_new, rb, static_cast<char*>(b_tail) + (size_t)pos * rb, pitch, rb,
                                            rows, st));
}

int mkv_grow_pool(const void* src, void* dst, int bits, int B, int Hkv, int cap_old, int cap_new, int d, int C,
                  void* stream) {
    if (!src || !dst || !aligned16(src) || !aligned16(dst)) return MKV_ERR_ARG;
    if (B <= 0 || Hkv <= 0 || cap_old < 0 || cap_new < cap_old || C <= 0 || C % mkv::kGroup) return MKV_ERR_ARG;
    const size_t slot = mkv_pool_bytes(bits, 1, 1, 1, d, C);
    if (!slot) return MKV_ERR_UNSUPPORTED;
    if ((long long)B * Hkv > 2147483647LL) return MKV_ERR_UNSUPPORTED;
    const char* s8 = static_cast<const char*>(src);
    char* d8 = static_cast<char*>(dst);
    const size_t old_bytes = (size_t)B * Hkv * cap_old * slot, new_bytes = (size_t)B * Hkv * cap_new * slot;
    if (s8 < d8 + new_bytes && d8 < s8 + old_bytes) return MKV_ERR_ARG;   // overlap
    return hip_status(mkv::launch_copy_rows(src, (size_t)cap_old * slot, dst, (size_t)cap_new * slot,
                                            (size_t)cap_old * slot, B * Hkv, (hipStream_t)stream));
}

}  // extern "C"
