// Chunked-prefill attention over the mixed-bitwidth cache.  A chunk of P new
// tokens is attended before it is quantized (MoQAE "Overall framework":
// ordinary attention over the cache; Cocktail abstract: chunk-level
// computation over bitwidth-contiguous segments): query i of the chunk sees
// every cached token and the chunk's own fp16 tokens 0..i.
//
// Unlike a decode step this is a dense contraction (P queries x T tokens x
// d), so it runs on the matrix cores.  A workgroup holds 256 queries of one
// query head (32 per wavefront) and one split of the cached group blocks.
// Each 32-token group block is dequantized once into LDS as fp16 -- keys
// token-major, values channel-major -- and shared by the eight wavefronts;
// each wavefront then computes S^T = K Q^T with v_mfma_f32_32x32x16_f16
// (lane = query, so the online softmax is lane-local), and O^T += V^T P^T
// with the probabilities fed from its own accumulator registers.  Splits are
// merged by a log-sum-exp combine.
#include "mkv_internal.h"
#include "mkv_kernels.h"

namespace mkv {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // a 16-byte cell as a value type

constexpr int NWAVE = 8;                // wavefronts per workgroup (2 per SIMD)
constexpr int PT = 64 * NWAVE;          // threads per workgroup
constexpr int QPW = 32;                 // queries per wavefront
constexpr int QT = QPW * NWAVE;         // queries per workgroup
constexpr int RING_CELLS = 6144;        // 96 KB ring of raw group blocks (16-byte cells)

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glob_void;

// s_waitcnt immediate waiting until at most n vector memory operations are
// outstanding (gfx9 encoding: vmcnt [3:0] and [15:14]; the other counters
// left at their maximum).
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Workgroup barrier for LDS written by ds_write only: wait for this
// wavefront's LDS operations, then s_barrier.  Unlike __syncthreads() it does
// not wait for outstanding global->LDS loads of later blocks.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0); vmcnt and expcnt at their maximum
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
struct PfTile {
    _Float16 k[32][D + 8];                 // keys of a block, token-major (rows padded by 16 bytes)
    _Float16 vt[D][36];                    // values, channel-major: 32 tokens + 4 pad (72-byte rows);
                                           // the 4-token chunk c of channel ch sits at chunk
                                           // c ^ vt_swz(ch), spreading the writes over the banks
};

// Chunk swizzle of the value tile: the channel's 32-channel group.
__device__ __forceinline__ constexpr int vt_swz(int ch) { return (ch >> 5) & 7; }

template <int D>
struct PfLds {
    u32x4 ring[RING_CELLS];                // raw group blocks in flight (slots sized per bitwidth)
    PfTile<D> tile[2];                     // fp16 blocks: one being consumed, one being filled
};

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}
__device__ __forceinline__ uint32_t lo16(uint32_t x) { return x & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t x) { return x >> 16; }

// Packed group block (raw, 16-byte cells as laid out in the pool) -> fp16
// keys and values in LDS.  Every thread writes whole 8-byte runs: four
// channels of one token for the keys, four consecutive tokens of one channel
// for the values (gathered from the four lane slots that hold tokens
// 4m .. 4m+3 of a value group).
template <int D, int BITS>
__device__ __forceinline__ void dequant_block(PfTile<D>& s, const u32x4* raw) {
    constexpr int S = D / 8, NG = D / 32;
    const int tid = threadIdx.x;
    if constexpr (BITS == 16) {
        // keys: row r, lane slot L: channels 8L..8L+7 of token tok(L, r)
        for (int c = tid; c < 32 * S; c += PT) {
            const int r = c / S, L = c % S;
            *reinterpret_cast<u32x4*>(&s.k[tok_of(S, L, r)][8 * L]) = raw[c];
        }
        // values: item (m, G, octet o, half h): channels 32G + 8o + 4h .. +3 of
        // tokens 4m .. 4m+3, i.e. of token m of the slots tq*NG + G, tq = 0..3
        // (row 4m + o holds channels 32G + 8o .. +7 of the slot's token m)
        for (int c = tid; c < 8 * NG * 4 * 2; c += PT) {
            const int m = c & 7, G = (c >> 3) % NG, o = (c / (8 * NG)) & 3, h = c / (32 * NG);
            uint32_t w[4][2];
#pragma unroll
            for (int tq = 0; tq < 4; ++tq) {
                const u32x4 u = raw[32 * S + (4 * m + o) * S + tq * NG + G];
                w[tq][0] = h ? u[2] : u[0];
                w[tq][1] = h ? u[3] : u[1];
            }
            const int ch = 32 * G + 8 * o + 4 * h;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int wi = j >> 1;
                const uint32_t a0 = (j & 1) ? hi16(w[0][wi]) : lo16(w[0][wi]);
                const uint32_t a1 = (j & 1) ? hi16(w[1][wi]) : lo16(w[1][wi]);
                const uint32_t a2 = (j & 1) ? hi16(w[2][wi]) : lo16(w[2][wi]);
                const uint32_t a3 = (j & 1) ? hi16(w[3][wi]) : lo16(w[3][wi]);
                *reinterpret_cast<uint2*>(&s.vt[ch + j][4 * (m ^ vt_swz(ch + j))]) =
                    make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
            }
        }
    } else {
        constexpr int F = 32 / BITS;            // codes per word
        constexpr uint32_t MASK = (1u << BITS) - 1u;
        constexpr int NP = F / 4;               // 4-token parts of a key word
        const float* kmeta = reinterpret_cast<const float*>(&raw[km_row0(BITS) * S]);
        // keys: item (code row, slot L, part p): channels 8L + 4(row&1) .. +3 of
        // the 4 tokens held by fields 4p .. 4p+3 of word row>>1
        for (int c = tid; c < kc_rows(BITS) * S * NP; c += PT) {
            const int p = c % NP, L = (c / NP) % S, row = c / (NP * S);
            const int w = row >> 1, j0 = 4 * (row & 1);
            const u32x4 u = raw[(kc_row0(BITS) + row) * S + L];
            const float4 sc = *reinterpret_cast<const float4*>(kmeta + ((row & 1) * S + L) * 4);
            const float4 mn = *reinterpret_cast<const float4*>(kmeta + ((2 + (row & 1)) * S + L) * 4);
#pragma unroll
            for (int i = 4 * p; i < 4 * p + 4; ++i) {
                const int t = tok_of(S, L, F * w + i);
                const int sh = BITS * i;
                const float x0 = __builtin_fmaf((float)((u[0] >> sh) & MASK), sc.x, mn.x);
                const float x1 = __builtin_fmaf((float)((u[1] >> sh) & MASK), sc.y, mn.y);
                const float x2 = __builtin_fmaf((float)((u[2] >> sh) & MASK), sc.z, mn.z);
                const float x3 = __builtin_fmaf((float)((u[3] >> sh) & MASK), sc.w, mn.w);
                *reinterpret_cast<uint2*>(&s.k[t][8 * L + j0]) = make_uint2(pack_h2(x0, x1), pack_h2(x2, x3));
            }
        }
        // values: item (token index mm, G, word u, channel quad h): channels
        // 32G + F*u + 4h .. +3 of tokens 4mm .. 4mm+3 (token mm of slots tq*NG + G)
        const float* vmeta = reinterpret_cast<const float*>(&raw[vm_row0(BITS) * S]);
        constexpr int NW = 32 / F;              // words per token and group
        constexpr int NH = F / 4;               // channel quads per word
        for (int c = tid; c < 8 * NG * NW * NH; c += PT) {
            const int mm = c & 7, G = (c >> 3) % NG, u = (c / (8 * NG)) % NW, h = c / (8 * NG * NW);
            const int row = BITS == 4 ? mm : (mm >> 1);
            const int dw = BITS == 4 ? u : 2 * (mm & 1) + u;
            float sv[4], mv[4];
            uint32_t wd[4];
#pragma unroll
            for (int tq = 0; tq < 4; ++tq) {
                const int L = tq * NG + G;
                const float2 sm = *reinterpret_cast<const float2*>(vmeta + ((mm >> 1) * S + L) * 4 + 2 * (mm & 1));
                sv[tq] = sm.x;
                mv[tq] = sm.y;
                const u32x4 q4 = raw[(vc_row0(BITS) + row) * S + L];
                wd[tq] = dw == 0 ? q4[0] : (dw == 1 ? q4[1] : (dw == 2 ? q4[2] : q4[3]));
            }
            const int ch = 32 * G + F * u + 4 * h;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sh = BITS * (4 * h + j);
                float x[4];
#pragma unroll
                for (int tq = 0; tq < 4; ++tq) x[tq] = __builtin_fmaf((float)((wd[tq] >> sh) & MASK), sv[tq], mv[tq]);
                *reinterpret_cast<uint2*>(&s.vt[ch + j][4 * (mm ^ vt_swz(ch + j))]) =
                    make_uint2(pack_h2(x[0], x[1]), pack_h2(x[2], x[3]));
            }
        }
    }
}

}  // namespace

namespace {

// Per-wavefront state: 32 queries (lane = query, both lane halves), the
// unnormalised output O^T [d x 32] in accumulators, running max and sum.
template <int D>
struct PfState {
    f16x8 qf[D / 16];      // lane (lr, lh): channels 16ks + 8lh .. +7 of query qp
    f32x16 o[D / 32];      // register r of tile t: channel 32t + 8(r>>2) + 4lh + (r&3)
    float m, l;
};

// One 32-token block in s.k / s.vt: scores, online softmax, values.  With
// `causal`, token j of the block is new-chunk position base + j, visible to
// query qp when base + j <= qp < P.
template <int D>
__device__ __forceinline__ void pf_block(PfState<D>& w, const PfTile<D>& s, float qscale, bool causal, int base,
                                         int qp, int P) {
    const int lane = threadIdx.x & 63, lr = lane & 31, lh = lane >> 5;
    f32x16 st;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(&s.k[lr][16 * ks + 8 * lh]);
        st = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, w.qf[ks], st, 0, 0, 0);
    }
    // st[r]: token 8(r>>2) + 4lh + (r&3) of the block, query qp
    // raw scores; the scale (> 0) is applied inside the exponent's fma
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float x = st[r];
        if (causal) {
            const int tp = base + 8 * (r >> 2) + 4 * lh + (r & 3);
            if (tp > qp || tp >= P) x = -INFINITY;
        }
        st[r] = x;
        mloc = fmaxf(mloc, x);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32)) * qscale;
    const float mn = fmaxf(w.m, mloc);
    const float alpha = (mn == -INFINITY) ? 1.f : exp2_fast(w.m - mn);
    float ps = 0.f;
    f16x8 pf0, pf1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float pr = (mn == -INFINITY) ? 0.f : exp2_fast(__builtin_fmaf(st[r], qscale, -mn));
        ps += pr;
        if (r < 8) pf0[r] = (_Float16)pr;
        else pf1[r - 8] = (_Float16)pr;
    }
    w.l = __builtin_fmaf(w.l, alpha, ps);
    w.m = mn;
    // the running max rarely rises after the first blocks: rescale only then
    // (alpha is exactly 1 for a lane whose max stayed)
    if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) w.o[t][r] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
        // K step ks2 covers tokens 16ks2 + 8(j>>2) + 4lh + (j&3), j = 0..7: the
        // tokens of accumulator registers 8ks2 .. 8ks2+7 of this lane
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
            // chunks 4ks2 + lh and 4ks2 + 2 + lh of channel 32t + lr (swizzle t)
            const f16x4 v0 = *reinterpret_cast<const f16x4*>(&s.vt[32 * t + lr][4 * ((4 * ks2 + lh) ^ (t & 7))]);
            const f16x4 v1 = *reinterpret_cast<const f16x4*>(&s.vt[32 * t + lr][4 * ((4 * ks2 + 2 + lh) ^ (t & 7))]);
            const f16x8 a = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            w.o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, ks2 ? pf1 : pf0, w.o[t], 0, 0, 0);
        }
    }
}

// Group blocks [lo, hi) of one bitwidth segment.  Raw blocks stream into a
// ring of NR slots by direct global->LDS loads issued NR blocks ahead (one
// block per iteration, re-reading the last block once the segment is
// exhausted, so the number of loads in flight and hence every wait count is
// fixed).  Iteration g dequantizes block g+1 into one fp16 tile while the
// matrix cores consume block g from the other, with one barrier between
// iterations.
template <int D, int BITS>
__device__ __forceinline__ void pf_segment(PfState<D>& w, PfLds<D>& s, const uint8_t* seg_base, int lo, int hi,
                                           float qscale, int qp, int P) {
    constexpr int S = D / 8;
    constexpr int NC = group_rows(BITS) * S;       // 16-byte cells per block
    constexpr int LPW = (NC + PT - 1) / PT;        // 64-cell loads per wavefront and block
    constexpr int SLOT = LPW * PT;                 // cells per ring slot
    constexpr int NR = RING_CELLS / SLOT;          // ring slots
    constexpr int GC = (int)(group_bytes(BITS, D) / 16);
    static_assert(NR >= 3 && (NR - 1) * LPW < 64, "ring depth");
    if (lo >= hi) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const u32x4* seg = reinterpret_cast<const u32x4*>(seg_base);
    auto issue = [&](int g) {
        const int gb = g < hi ? g : hi - 1;
        const u32x4* blk = seg + (size_t)gb * GC;
        u32x4* slot = s.ring + (g % NR) * SLOT;
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int c0 = (j * NWAVE + wave) * 64;    // this wavefront's 64 cells
            const int c = min(c0 + lane, NC - 1);
            __builtin_amdgcn_global_load_lds((glob_void*)(blk + c), (lds_void*)(slot + c0), 16, 0, 0);
        }
    };
#pragma unroll
    for (int i = 0; i < NR; ++i) issue(lo + i);
    __builtin_amdgcn_s_waitcnt(wait_vm((NR - 1) * LPW));      // this wavefront's part of block lo landed
    lds_barrier();
    dequant_block<D, BITS>(s.tile[lo & 1], s.ring + (lo % NR) * SLOT);
    for (int g = lo; g < hi; ++g) {
        __builtin_amdgcn_s_waitcnt(wait_vm((NR - 2) * LPW));  // ... of block g+1 (or its stand-in)
        lds_barrier();           // block g dequantized, block g+1 landed, block g-1 consumed
        issue(g + NR);           // into the slot of block g, dequantized one iteration ago
        if (g + 1 < hi) dequant_block<D, BITS>(s.tile[(g + 1) & 1], s.ring + ((g + 1) % NR) * SLOT);
        pf_block<D>(w, s.tile[g & 1], qscale, false, 0, qp, P);
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(0));                     // the ring is reused by the next segment
    lds_barrier();
}

}  // namespace

// grid: x = query tile (QT queries), y = split, z = sequence * Hq + query head
template <int D>
__global__ __launch_bounds__(PT) void prefill_tile_kernel(PrefillParams p) {
    __shared__ __align__(16) PfLds<D> s;
    constexpr int S = D / 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lh = lane >> 5;
    const int qtile = blockIdx.x, split = blockIdx.y;
    const int bq = blockIdx.z, b = bq / p.Hq, hq = bq % p.Hq;
    const int h = hq / (p.Hq / p.Hkv);
    const int bh = b * p.Hkv + h;
    const int qp = qtile * QT + wave * QPW + (lane & 31);   // this lane's query position
    const bool qvalid = qp < p.P;

    PfState<D> w;
    {
        const uint16_t* qrow = p.q + ((size_t)bq * p.P + (qvalid ? qp : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            w.qf[ks] = __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * lh));
    }
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) w.o[t][r] = 0.f;
    w.m = -INFINITY;
    w.l = 0.f;

    // ---------------- this split's cached group blocks (FP16, INT4, INT2 segments)
    const int gpc = p.C / kGroup;
    int segg[3], total = 0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int cnt = min(max(p.seg_count[b * 3 + k], 0), p.cap[k]);
        segg[k] = cnt * gpc;
        total += segg[k];
    }
    // work list: the cached group blocks, then the new chunk's 32-token blocks;
    // every split takes an equal share of both
    const int nblk = (p.P + 31) / 32;
    const int W = total + nblk;
    const int g0 = (int)((long long)split * W / p.NS), g1 = (int)((long long)(split + 1) * W / p.NS);
    {
        int base = 0;
        pf_segment<D, 16>(w, s, p.pool[0] + (size_t)bh * p.cap[0] * gpc * group_bytes(16, D),
                          max(g0 - base, 0), min(g1 - base, segg[0]), p.qscale, qp, p.P);
        base += segg[0];
        pf_segment<D, 4>(w, s, p.pool[1] + (size_t)bh * p.cap[1] * gpc * group_bytes(4, D),
                         max(g0 - base, 0), min(g1 - base, segg[1]), p.qscale, qp, p.P);
        base += segg[1];
        pf_segment<D, 2>(w, s, p.pool[2] + (size_t)bh * p.cap[2] * gpc * group_bytes(2, D),
                         max(g0 - base, 0), min(g1 - base, segg[2]), p.qscale, qp, p.P);
    }

    // ---------------- this split's blocks of the new chunk's own tokens, causal
    {
        // blocks past this tile's last query see nothing
        const int last = min(nblk, (qtile * QT + QT + 31) / 32);
        const int nb0 = max(g0 - total, 0), nb1 = min(g1 - total, last);
        const uint16_t* kn = p.k_new + (size_t)bh * p.P * D;
        const uint16_t* vn = p.v_new + (size_t)bh * p.P * D;
        for (int nb = nb0; nb < nb1; ++nb) {
            __syncthreads();
            for (int c = tid; c < 32 * S; c += PT) {
                const int t = c / S, L = c % S, tp = 32 * nb + t;
                uint4 ku = make_uint4(0, 0, 0, 0), vu = make_uint4(0, 0, 0, 0);
                if (tp < p.P) {
                    ku = *reinterpret_cast<const uint4*>(kn + (size_t)tp * D + 8 * L);
                    vu = *reinterpret_cast<const uint4*>(vn + (size_t)tp * D + 8 * L);
                }
                *reinterpret_cast<uint4*>(&s.tile[0].k[t][8 * L]) = ku;
                const uint32_t vw[4] = {vu.x, vu.y, vu.z, vu.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c0 = 8 * L + 2 * e, c1 = c0 + 1;
                    s.tile[0].vt[c0][4 * ((t >> 2) ^ vt_swz(c0)) + (t & 3)] =
                        __builtin_bit_cast(_Float16, (uint16_t)(vw[e] & 0xffffu));
                    s.tile[0].vt[c1][4 * ((t >> 2) ^ vt_swz(c1)) + (t & 3)] =
                        __builtin_bit_cast(_Float16, (uint16_t)(vw[e] >> 16));
                }
            }
            __syncthreads();
            pf_block<D>(w, s.tile[0], p.qscale, true, 32 * nb, qp, p.P);
        }
    }

    // ---------------- partial record of this split: o (unnormalised), m, l
    w.l += __shfl_xor(w.l, 32);
    if (qvalid) {
        float* rec = p.part + (((size_t)bq * p.P + qp) * p.NS + split) * (D + 4);
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<float4*>(rec + 32 * t + 8 * g + 4 * lh) =
                    make_float4(w.o[t][4 * g], w.o[t][4 * g + 1], w.o[t][4 * g + 2], w.o[t][4 * g + 3]);
        if (lh == 0) *reinterpret_cast<float2*>(rec + D) = make_float2(w.m, w.l);
    }
}

// One wavefront per (sequence, query head, query): the splits' records merged
// with the log-sum-exp combine; lane l owns channels (D/64)*l .. +D/64-1.
template <int D>
__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillParams p) {
    const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const size_t rows = (size_t)p.B * p.Hq * p.P;
    if (row >= rows) return;
    constexpr int PL = D / 64;                 // channels per lane
    const float* recs = p.part + row * p.NS * (D + 4);
    float M = -INFINITY;
    for (int sp = 0; sp < p.NS; ++sp) M = fmaxf(M, recs[(size_t)sp * (D + 4) + D]);
    float acc[PL] = {}, L = 0.f;
    if (M != -INFINITY) {
        for (int sp = 0; sp < p.NS; ++sp) {
            const float* r = recs + (size_t)sp * (D + 4);
            const float ms = r[D];
            if (ms == -INFINITY) continue;
            const float wgt = exp2_fast(ms - M);
            L = __builtin_fmaf(r[D + 1], wgt, L);
#pragma unroll
            for (int c = 0; c < PL; ++c) acc[c] = __builtin_fmaf(r[PL * lane + c], wgt, acc[c]);
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float* out = p.out + row * D + PL * lane;
#pragma unroll
    for (int c = 0; c < PL; ++c) out[c] = acc[c] * inv;
}

hipError_t launch_prefill(const PrefillParams& pp, int D, hipStream_t st) {
    const dim3 grid((pp.P + QT - 1) / QT, pp.NS, pp.B * pp.Hq);
    const size_t rows = (size_t)pp.B * pp.Hq * pp.P;
    const dim3 cgrid((unsigned)((rows + 3) / 4));
    if (D == 128) {
        prefill_tile_kernel<128><<<grid, PT, 0, st>>>(pp);
        prefill_combine_kernel<128><<<cgrid, 256, 0, st>>>(pp);
    } else if (D == 64) {
        prefill_tile_kernel<64><<<grid, PT, 0, st>>>(pp);
        prefill_combine_kernel<64><<<cgrid, 256, 0, st>>>(pp);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mkv
