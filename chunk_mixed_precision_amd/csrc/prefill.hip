// Chunked-prefill attention over the mixed-bitwidth cache.  A chunk of P new
// tokens is attended before it is quantized (MoQAE "Overall framework":
// ordinary attention over the cache; Cocktail abstract: chunk-level
// computation over bitwidth-contiguous segments): query i of the chunk sees
// every cached token and the chunk's own fp16 tokens 0..i.
//
// Unlike a decode step this is a dense contraction (P queries x T tokens x
// d), so it runs on the matrix cores.  A workgroup holds 256 queries of one
// query head (32 per wavefront) and one split of the cached group blocks;
// with at most 128 queries it holds 128, and its two halves of four
// wavefronts take alternate group blocks, their softmax states merged in LDS
// at the end.  Each 32-token group block is dequantized once into LDS as
// fp16 -- keys token-major, values channel-major -- and shared by the
// wavefronts; each wavefront then computes S^T = K Q^T with
// v_mfma_f32_32x32x16_f16 (lane = query, so the online softmax is
// lane-local), and O^T += V^T P^T with the probabilities made from its own
// score registers.  Splits are merged by a log-sum-exp combine.
#include "mkv_internal.h"
#include "mkv_kernels.h"

namespace mkv {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // a 16-byte cell as a value type

constexpr int NWAVE = 8;                // wavefronts per workgroup (2 per SIMD)
constexpr int PT = 64 * NWAVE;          // threads per workgroup
constexpr int QPW = 32;                 // queries per wavefront
constexpr int QT = QPW * NWAVE;         // queries per workgroup (256)
constexpr int QT_HALF = QT / 2;         // queries per workgroup when P <= 128
constexpr int RING_CELLS = 4096;        // 64 KB ring of raw group-block pairs (16-byte cells)
constexpr int DQ_THREADS = PT / 2;      // threads that dequantize one group block of a pair

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

// Largest rise of the softmax maximum (log2 units) absorbed without moving
// the reference point: probabilities reach at most 2^8 before fp16 rounding.
constexpr float kSlack = 8.f;

// The value of lane l ^ 32.  v_permlane32_swap exchanges the upper half of
// one register with the lower half of another; applied to two copies of x,
// lanes 0-31 of the second copy and lanes 32-63 of the first then hold the
// other half's values.  (Written out: the compiler builtin folded a max of
// its two results to the first one.)  The s_nop covers the VALU write of
// the copies ahead of the permute.
__device__ __forceinline__ float swap_halves(float x) {
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    const bool upper = (threadIdx.x & 32) != 0;
    return __builtin_bit_cast(float, upper ? a : b);
}

// Value tile geometry: channel-major rows of 32 tokens + 4 pad (72 bytes),
// 32 rows per 32-channel group, and 16 more bytes after every group, so that
// group g starts 4g banks further on: the dequant writes of one row of
// lanes (four groups x four 8-channel words) fall on distinct banks.
constexpr int VT_ROW = 36;                        // halves per channel row
constexpr int VT_GROUP = 32 * VT_ROW + 8;         // halves per 32-channel group

template <int D>
struct PfTile {
    _Float16 k[32][D + 8];                 // keys of a block, token-major (rows padded by 16 bytes)
    _Float16 vt[D / 32][VT_GROUP];         // values, channel-major (see VT_ROW / VT_GROUP)
};

// Token chunk c (tokens 4c .. 4c+3) of channel ch in the value tile.
template <int D>
__device__ __forceinline__ _Float16* vt_at(PfTile<D>& s, int ch, int c) {
    return &s.vt[ch >> 5][(ch & 31) * VT_ROW + 4 * c];
}
template <int D>
__device__ __forceinline__ const _Float16* vt_at(const PfTile<D>& s, int ch, int c) {
    return &s.vt[ch >> 5][(ch & 31) * VT_ROW + 4 * c];
}

template <int D>
struct PfLds {
    u32x4 ring[RING_CELLS];                // raw group-block pairs in flight (slots sized per bitwidth)
    PfTile<D> tile[2][2];                  // fp16 block pairs: one being consumed, one being filled
};

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}
__device__ __forceinline__ uint32_t lo16(uint32_t x) { return x & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t x) { return x >> 16; }

// Two fp16 results packed in one word: low = fp16(ya.h * wa + oa), high =
// fp16(yb.h * wb + ob), where .h is the low (HSEL 0) or high (HSEL 1) fp16
// half of ya / yb.  Each product and sum is one fused fp32 operation on the
// fp16 input (v_fma_mix_f32), and one v_cvt_pk_f16_f32 rounds both to fp16:
// on this part that issues faster than writing each half with
// v_fma_mixlo_f16 / v_fma_mixhi_f16 (which round straight to fp16).
// f(integral_constant<int, 0>{}), ..., f(integral_constant<int, N-1>{})
template <int N, int I = 0, class Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
    if constexpr (I < N) {
        fn(std::integral_constant<int, I>{});
        static_for<N, I + 1>(fn);
    }
}

template <int HSEL>
__device__ __forceinline__ uint32_t mix_pair(uint32_t ya, uint32_t yb, float wa, float oa, float wb, float ob) {
    const h2_t ha = __builtin_bit_cast(h2_t, ya), hb = __builtin_bit_cast(h2_t, yb);
    const float fa = __builtin_fmaf((float)ha[HSEL], wa, oa);
    const float fb = __builtin_fmaf((float)hb[HSEL], wb, ob);
    return __builtin_bit_cast(uint32_t, h2_t{(_Float16)fa, (_Float16)fb});
}

// Packed group block (raw, 16-byte cells as laid out in the pool) -> fp16
// keys and values in LDS.  Every thread writes whole 8-byte runs: four
// channels of one token for the keys, four consecutive tokens of one channel
// for the values (gathered from the four lane slots that hold tokens
// 4m .. 4m+3 of a value group).
template <int D, int BITS>
__device__ __forceinline__ void dequant_block(PfTile<D>& s, const u32x4* raw, int tid) {
    constexpr int S = D / 8, NG = D / 32;
    if constexpr (BITS == 16) {
        // keys: row r, lane slot L: channels 8L..8L+7 of token tok(L, r)
        for (int c = tid; c < 32 * S; c += DQ_THREADS) {
            const int r = c / S, L = c % S;
            *reinterpret_cast<u32x4*>(&s.k[tok_of(S, L, r)][8 * L]) = raw[c];
        }
        // values: item (m, G, octet o, half h): channels 32G + 8o + 4h .. +3 of
        // tokens 4m .. 4m+3, i.e. of token m of the slots tq*NG + G, tq = 0..3
        // (row 4m + o holds channels 32G + 8o .. +7 of the slot's token m)
        for (int c = tid; c < 8 * NG * 4 * 2; c += DQ_THREADS) {
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
                *reinterpret_cast<uint2*>(vt_at(s, ch + j, m)) =
                    make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
            }
        }
    } else {
        // A code c placed at bits 4-5 / 4-7 (weight 16) or 6-7 (weight 64) of
        // an fp16 half whose other bits are 0x6400 is the half 1024 + 16c (or
        // 1024 + 64c).  With w = s/16 (s/64) and o = mn - 64s (mn - 16s) one
        // mixed fma gives c*s + mn, rounded once to fp16 straight into the
        // low or high half of the output word.  (o carries one fp32 rounding
        // of at most 2^-24 * 64|s|, far below the fp16 rounding of the tile.)
        constexpr int F = 32 / BITS;            // codes per word
        // magic halves of word x: INT4 y[k] holds fields k (low half) and
        // k + 4 (high half) at bits 4-7; INT2 y[2k] holds fields 2k, 2k + 8 at
        // bits 4-5 and y[2k+1] fields 2k+1, 2k+9 at bits 6-7
        // (the magic constant sits in a register so that mask-and-insert is
        // one v_and_or_b32: a VOP3 takes no literal operand on this target)
        uint32_t vmagic;
        asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(vmagic));
        auto magic = [vmagic](uint32_t x, uint32_t* y) {
            const uint32_t src[4] = {x << 4, x, x >> 4, x >> 8};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (BITS == 4) {
                    y[k] = (src[k] & 0x00F000F0u) | vmagic;
                } else {
                    y[2 * k] = (src[k] & 0x00300030u) | vmagic;
                    y[2 * k + 1] = (src[k] & 0x00C000C0u) | vmagic;
                }
            }
        };
        // field f of a word: its magic register and half, and whether its
        // weight is the 64 one
        // (reg_of, half_of and wide_of are compile-time for every field below)
        auto reg_of = [](int f) { return BITS == 4 ? (f & 3) : (f & 7); };
        auto wide_of = [](int f) { return BITS == 2 && (f & 1); };
        // one output word from channel/token words a and b (fields f)
        auto pair_out = [&](auto f_tag, const uint32_t* ya, const uint32_t* yb, float wna, float ona, float wwa,
                            float owa, float wnb, float onb, float wwb, float owb) {
            constexpr int f = decltype(f_tag)::value;
            constexpr int HS = BITS == 4 ? (f >> 2) : (f >> 3);
            return wide_of(f) ? mix_pair<HS>(ya[reg_of(f)], yb[reg_of(f)], wwa, owa, wwb, owb)
                              : mix_pair<HS>(ya[reg_of(f)], yb[reg_of(f)], wna, ona, wnb, onb);
        };

        constexpr int KH = BITS == 4 ? 1 : 2;   // key items per code cell (fields split in halves)
        constexpr int NK = kc_rows(BITS) * S * KH;
        constexpr int NW = 32 / F;              // value words per token and group
        constexpr int VH = BITS == 4 ? 1 : 2;   // value items per word (channels split in halves)
        constexpr int NV = 8 * NG * NW * VH;
        constexpr int FPI = F / KH;             // fields per item (8)
        static_assert(NK % 64 == 0 && NV % 64 == 0 && NK + NV <= DQ_THREADS,
                      "one item per thread, wave-uniform kinds");
        static_assert(F / KH == 8 && F / VH == 8, "eight fields per item");
        if (tid < NK) {
            // keys: cell (code row, slot L) = channels 8L + 4(row&1) .. +3; its
            // word row>>1 holds field positions F*(row>>1) .. of each channel;
            // this item takes fields FPI*kh .. +FPI-1
            const int L = tid % S, row = (tid / S) % kc_rows(BITS), kh = tid / (S * kc_rows(BITS));
            const int w = row >> 1, j0 = 4 * (row & 1);
            const u32x4 u = raw[(kc_row0(BITS) + row) * S + L];
            const float* kmeta = reinterpret_cast<const float*>(&raw[km_row0(BITS) * S]);
            const float4 sc = *reinterpret_cast<const float4*>(kmeta + ((row & 1) * S + L) * 4);
            const float4 mn = *reinterpret_cast<const float4*>(kmeta + ((2 + (row & 1)) * S + L) * 4);
            const float scs[4] = {sc.x, sc.y, sc.z, sc.w}, mns[4] = {mn.x, mn.y, mn.z, mn.w};
            float wn[4], on[4], ww[4], ow[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                wn[c] = scs[c] * 0.0625f;
                on[c] = __builtin_fmaf(-64.f, scs[c], mns[c]);
                ww[c] = scs[c] * 0.015625f;
                ow[c] = __builtin_fmaf(-16.f, scs[c], mns[c]);
            }
            uint32_t y[4][8];
#pragma unroll
            for (int c = 0; c < 4; ++c) magic(u[c], y[c]);
            // token of field position F*w + f: the xor of f into that of F*w
            // (f < 16 touches only the bits that tok_of permutes)
            const int t0 = tok_of(S, L, F * w);
            _Float16* krow = &s.k[0][8 * L + j0];
            auto fields = [&](auto kh_tag) {
                constexpr int KHV = decltype(kh_tag)::value;
                static_for<FPI>([&](auto i_tag) {
                    constexpr int f = FPI * KHV + decltype(i_tag)::value;
                    static_assert(f < 16, "field inside its 16-token half");
                    const int t = t0 ^ f;
                    const uint32_t o0 = pair_out(std::integral_constant<int, f>{}, y[0], y[1], wn[0], on[0], ww[0],
                                                 ow[0], wn[1], on[1], ww[1], ow[1]);
                    const uint32_t o1 = pair_out(std::integral_constant<int, f>{}, y[2], y[3], wn[2], on[2], ww[2],
                                                 ow[2], wn[3], on[3], ww[3], ow[3]);
                    *reinterpret_cast<uint2*>(krow + t * (D + 8)) = make_uint2(o0, o1);
                });
            };
            if (KH == 1 || kh == 0) fields(std::integral_constant<int, 0>{});
            else fields(std::integral_constant<int, KH - 1>{});
        } else if (tid < NK + NV) {
            // values: item (token index mm, G, word u, channel half vh): the
            // channels 32G + F*u + 8vh .. +7 of tokens 4mm .. 4mm+3 (token mm of
            // the slots tq*NG + G)
            const int c = tid - NK;
            // lanes next to each other take other groups and words of the same
            // token quad: their raw words and their tile rows both spread
            // over the banks
            const int G = c % NG, u = (c / NG) % NW, vh = (c / (NG * NW)) % VH, mm = c / (NG * NW * VH);
            const int row = BITS == 4 ? mm : (mm >> 1);
            const int dw = BITS == 4 ? u : 2 * (mm & 1) + u;
            const float* vmeta = reinterpret_cast<const float*>(&raw[vm_row0(BITS) * S]);
            float wn[4], on[4], ww[4], ow[4];
            uint32_t y[4][8];
#pragma unroll
            for (int tq = 0; tq < 4; ++tq) {
                const int L = vslot_of(tq, G, NG);
                const float2 sm = *reinterpret_cast<const float2*>(vmeta + ((mm >> 1) * S + L) * 4 + 2 * (mm & 1));
                wn[tq] = sm.x * 0.0625f;
                on[tq] = __builtin_fmaf(-64.f, sm.x, sm.y);
                ww[tq] = sm.x * 0.015625f;
                ow[tq] = __builtin_fmaf(-16.f, sm.x, sm.y);
                magic(reinterpret_cast<const uint32_t*>(&raw[(vc_row0(BITS) + row) * S + L])[dw], y[tq]);
            }
            const int ch0 = 32 * G + F * u + 8 * vh;
            auto channels = [&](auto vh_tag) {
                constexpr int VHV = decltype(vh_tag)::value;
                static_for<8>([&](auto i_tag) {
                    constexpr int i = decltype(i_tag)::value;
                    constexpr int f = 8 * VHV + i;
                    const uint32_t o0 = pair_out(std::integral_constant<int, f>{}, y[0], y[1], wn[0], on[0], ww[0],
                                                 ow[0], wn[1], on[1], ww[1], ow[1]);
                    const uint32_t o1 = pair_out(std::integral_constant<int, f>{}, y[2], y[3], wn[2], on[2], ww[2],
                                                 ow[2], wn[3], on[3], ww[3], ow[3]);
                    *reinterpret_cast<uint2*>(vt_at(s, ch0 + i, mm)) = make_uint2(o0, o1);
                });
            };
            if (VH == 1 || vh == 0) channels(std::integral_constant<int, 0>{});
            else channels(std::integral_constant<int, VH - 1>{});
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
    // every fragment read of the block goes out first: the key fragments,
    // then the value fragments (K step ks2 of tile t covers tokens 16ks2 +
    // 8(j>>2) + 4lh + (j&3), j = 0..7 -- the tokens of accumulator registers
    // 8ks2 .. 8ks2+7 of this lane -- i.e. chunks 4ks2 + lh and 4ks2 + 2 + lh
    // of channel 32t + lr), whose latency the scores and the softmax hide
    f16x8 kf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) kf[ks] = *reinterpret_cast<const f16x8*>(&s.k[lr][16 * ks + 8 * lh]);
    __builtin_amdgcn_sched_barrier(0);
    f16x8 vf[D / 32][2];
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
            const f16x4 v0 = *reinterpret_cast<const f16x4*>(vt_at(s, 32 * t + lr, 4 * ks2 + lh));
            const f16x4 v1 = *reinterpret_cast<const f16x4*>(vt_at(s, 32 * t + lr, 4 * ks2 + 2 + lh));
            vf[t][ks2] = f16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        }
    f32x16 st;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) st = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ks], w.qf[ks], st, 0, 0, 0);
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
    mloc = fmaxf(mloc, swap_halves(mloc)) * qscale;     // with the query's other tokens
    // The reference point m moves only when the block's maximum exceeds it by
    // more than kSlack (log2 units): probabilities then stay below 2^kSlack,
    // far inside fp16 and fp32 range, and o and l carry the same factor, so
    // o / l is unchanged while the rescale of o becomes rare.  The first
    // visible token always moves m off -inf (alpha = exp2(-inf) = 0).
    const bool raise = mloc > w.m + kSlack;
    const float mn = raise ? mloc : w.m;
    const float alpha = raise ? exp2_fast(w.m - mn) : 1.f;
    // a lane with no visible token yet (mn = -inf) has only -inf scores,
    // which the reference 0 sends to exp2(-inf) = 0
    const float mref = (mn == -INFINITY) ? 0.f : mn;
    f16x8 pf0, pf1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float pr = exp2_fast(__builtin_fmaf(st[r], qscale, -mref));
        if (r < 8) pf0[r] = (_Float16)pr;
        else pf1[r - 8] = (_Float16)pr;
    }
    // the denominator sums the fp16 probabilities that weight the values,
    // two per v_dot2_f32_f16 (products by 1 are exact, the sum is fp32)
    float ps = 0.f, ps1 = 0.f;
    const h2_t one = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ps = __builtin_amdgcn_fdot2(h2_t{pf0[2 * i], pf0[2 * i + 1]}, one, ps, false);
        ps1 = __builtin_amdgcn_fdot2(h2_t{pf1[2 * i], pf1[2 * i + 1]}, one, ps1, false);
    }
    ps += ps1;
    w.l = __builtin_fmaf(w.l, alpha, ps);
    w.m = mn;
    if (__ballot(raise)) {
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) w.o[t][r] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2)
            w.o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[t][ks2], ks2 ? pf1 : pf0, w.o[t], 0, 0, 0);
}

// Group blocks [lo, hi) of one bitwidth segment, two at a time.  Raw
// block pairs (adjacent in the pool) stream into a ring of NR slots by
// direct global->LDS loads issued NR pairs ahead (one pair per iteration,
// re-reading the last pair once the segment is exhausted, so the number of
// loads in flight and hence every wait count is fixed).  Iteration j
// dequantizes pair j+1 into one pair of fp16 tiles -- threads 0 .. PT/2-1
// the first block, the others the second -- while the matrix cores consume
// pair j from the other, with one barrier between iterations: the barrier,
// the ring traffic and the dequant latency are paid once per 64 tokens.
// A pair whose second block lies past hi (an odd count) has only its first
// block dequantized and attended.  With HALF, wavefronts 0-3 attend the first
// block of each pair and wavefronts 4-7 the second.
template <int D, int BITS, bool HALF>
__device__ __forceinline__ void pf_segment(PfState<D>& w, PfLds<D>& s, const uint8_t* seg_base, int lo, int hi,
                                           float qscale, int qp, int P) {
    constexpr int S = D / 8;
    constexpr int NC = group_rows(BITS) * S;       // 16-byte cells per block
    constexpr int LPW = (2 * NC + PT - 1) / PT;    // 64-cell loads per wavefront and pair
    constexpr int SLOT = LPW * PT;                 // cells per ring slot
    constexpr int NR = RING_CELLS / SLOT;          // ring slots
    constexpr int GC = (int)(group_bytes(BITS, D) / 16);
    static_assert(GC == NC && NR >= 2 && (NR - 1) * LPW < 64, "ring depth");
    if (lo >= hi) return;
    const int np = (hi - lo + 1) / 2;              // pairs
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = (int)threadIdx.x / DQ_THREADS, htid = (int)threadIdx.x % DQ_THREADS;
    const int grp = __builtin_amdgcn_readfirstlane(wave) >> 2;     // wavefronts 0-3 or 4-7
    const u32x4* seg = reinterpret_cast<const u32x4*>(seg_base);
    auto issue = [&](int j) {
        const int jj = j < np ? j : np - 1;
        const int first = lo + 2 * jj;
        const int ncells = min(2, hi - first) * NC;   // the pair's cells inside the segment
        const u32x4* blk = seg + (size_t)first * GC;
        u32x4* slot = s.ring + (j % NR) * SLOT;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int c0 = (i * NWAVE + wave) * 64;    // this wavefront's 64 cells
            const int c = min(c0 + lane, ncells - 1);
            __builtin_amdgcn_global_load_lds((glob_void*)(blk + c), (lds_void*)(slot + c0), 16, 0, 0);
        }
    };
    auto dequant_pair = [&](int j) {
        if (half == 0 || lo + 2 * j + 1 < hi)
            dequant_block<D, BITS>(s.tile[j & 1][half], s.ring + (j % NR) * SLOT + half * NC, htid);
    };
#pragma unroll
    for (int i = 0; i < NR; ++i) issue(i);
    __builtin_amdgcn_s_waitcnt(wait_vm((NR - 1) * LPW));      // this wavefront's part of pair 0 landed
    lds_barrier();
    dequant_pair(0);
    for (int j = 0; j < np; ++j) {
        __builtin_amdgcn_s_waitcnt(wait_vm((NR - 2) * LPW));  // ... of pair j+1 (or its stand-in)
        lds_barrier();           // pair j dequantized, pair j+1 landed, pair j-1 consumed
        issue(j + NR);           // into the slot of pair j, dequantized one iteration ago
        // Wavefronts 0-3 dequantize before they compute, 4-7 after: the two
        // wavefronts of each SIMD then run opposite phases (one on the vector
        // unit while the other feeds the matrix core).
        const bool dq_first = grp == 0;
        if (dq_first && j + 1 < np) dequant_pair(j + 1);
        if constexpr (HALF) {
            if (grp == 0 || lo + 2 * j + 1 < hi) pf_block<D>(w, s.tile[j & 1][grp], qscale, false, 0, qp, P);
        } else {
            pf_block<D>(w, s.tile[j & 1][0], qscale, false, 0, qp, P);
            if (lo + 2 * j + 1 < hi) pf_block<D>(w, s.tile[j & 1][1], qscale, false, 0, qp, P);
        }
        if (!dq_first && j + 1 < np) dequant_pair(j + 1);
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(0));                     // the ring is reused by the next segment
    lds_barrier();
}

}  // namespace

// grid: x = query tile (QT, or QT_HALF with HALF, queries), y = split,
// z = sequence * Hq + query head
template <int D, bool HALF>
__global__ __launch_bounds__(PT) void prefill_tile_kernel(PrefillParams p) {
    __shared__ __align__(16) PfLds<D> s;
    constexpr int S = D / 8;
    constexpr int QW = HALF ? NWAVE / 2 : NWAVE;     // wavefronts per set of queries
    constexpr int QTK = QPW * QW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int lh = lane >> 5;
    const int qtile = blockIdx.x, split = blockIdx.y;
    const int bq = blockIdx.z, b = bq / p.Hq, hq = bq % p.Hq;
    const int h = hq / (p.Hq / p.Hkv);
    const int bh = b * p.Hkv + h;
    const int qp = qtile * QTK + (wave % QW) * QPW + (lane & 31);   // this lane's query position
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
        pf_segment<D, 16, HALF>(w, s, p.pool[0] + (size_t)bh * p.cap[0] * gpc * group_bytes(16, D),
                                max(g0 - base, 0), min(g1 - base, segg[0]), p.qscale, qp, p.P);
        base += segg[0];
        pf_segment<D, 4, HALF>(w, s, p.pool[1] + (size_t)bh * p.cap[1] * gpc * group_bytes(4, D),
                               max(g0 - base, 0), min(g1 - base, segg[1]), p.qscale, qp, p.P);
        base += segg[1];
        pf_segment<D, 2, HALF>(w, s, p.pool[2] + (size_t)bh * p.cap[2] * gpc * group_bytes(2, D),
                               max(g0 - base, 0), min(g1 - base, segg[2]), p.qscale, qp, p.P);
    }

    // ---------------- this split's blocks of the new chunk's own tokens, causal
    // (two at a time with HALF: one per half of the workgroup)
    {
        // blocks past this tile's last query see nothing
        const int last = min(nblk, (qtile * QTK + QTK + 31) / 32);
        const int nb0 = max(g0 - total, 0), nb1 = min(g1 - total, last);
        const uint16_t* kn = p.k_new + (size_t)bh * p.P * D;
        const uint16_t* vn = p.v_new + (size_t)bh * p.P * D;
        constexpr int NBI = HALF ? 2 : 1;           // blocks per iteration
        for (int nb = nb0; nb < nb1; nb += NBI) {
            const int nload = min(NBI, nb1 - nb);
            __syncthreads();
            for (int c = tid; c < nload * 32 * S; c += PT) {
                const int bi = c / (32 * S), t = (c / S) % 32, L = c % S, tp = 32 * (nb + bi) + t;
                PfTile<D>& tl = s.tile[0][bi];
                uint4 ku = make_uint4(0, 0, 0, 0), vu = make_uint4(0, 0, 0, 0);
                if (tp < p.P) {
                    ku = *reinterpret_cast<const uint4*>(kn + (size_t)tp * D + 8 * L);
                    vu = *reinterpret_cast<const uint4*>(vn + (size_t)tp * D + 8 * L);
                }
                *reinterpret_cast<uint4*>(&tl.k[t][8 * L]) = ku;
                const uint32_t vw[4] = {vu.x, vu.y, vu.z, vu.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c0 = 8 * L + 2 * e, c1 = c0 + 1;
                    vt_at(tl, c0, t >> 2)[t & 3] = __builtin_bit_cast(_Float16, (uint16_t)(vw[e] & 0xffffu));
                    vt_at(tl, c1, t >> 2)[t & 3] = __builtin_bit_cast(_Float16, (uint16_t)(vw[e] >> 16));
                }
            }
            __syncthreads();
            const int bi = HALF ? (wave_u >> 2) : 0;
            if (bi < nload) pf_block<D>(w, s.tile[0][bi], p.qscale, true, 32 * (nb + bi), qp, p.P);
        }
    }

    // ---------------- HALF: the second half's state merged into the first's
    // (the same log-sum-exp merge as the combine), through LDS laid out
    // [value][wavefront][lane]; the second half then has nothing left to do
    if constexpr (HALF) {
        constexpr int NO = D / 2;                   // accumulator values per lane
        static_assert((NO + 2) * 4 * 64 * sizeof(float) <= sizeof(PfLds<D>), "merge area");
        float* xs = reinterpret_cast<float*>(&s);
        const int wq = wave_u & 3;
        auto at = [&](int k) { return xs + ((size_t)k * 4 + wq) * 64 + lane; };
        __syncthreads();                            // every wavefront is done with the tiles
        if (wave_u >= 4) {
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) *at(16 * t + r) = w.o[t][r];
            *at(NO) = w.m;
            *at(NO + 1) = w.l;
        }
        __syncthreads();
        if (wave_u >= 4) return;
        const float m2 = *at(NO), l2 = *at(NO + 1);
        const float mx = fmaxf(w.m, m2);
        const float a1 = (w.m == -INFINITY) ? 0.f : exp2_fast(w.m - mx);
        const float a2 = (m2 == -INFINITY) ? 0.f : exp2_fast(m2 - mx);
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) w.o[t][r] = __builtin_fmaf(*at(16 * t + r), a2, w.o[t][r] * a1);
        w.l = __builtin_fmaf(l2, a2, w.l * a1);
        w.m = mx;
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
// Lane sp first loads split sp's (m, l) (at most 32 splits), so the maximum,
// the weights and the denominator come from one round of loads and wave
// reductions; the splits' channel values are then loaded in batches of
// eight, independent of each other.
template <int D>
__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillParams p) {
    const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const size_t rows = (size_t)p.B * p.Hq * p.P;
    if (row >= rows) return;
    constexpr int PL = D / 64;                 // channels per lane
    constexpr int BATCH = 8;
    const float* recs = p.part + row * p.NS * (D + 4);
    float ms = -INFINITY, ls = 0.f;
    if (lane < p.NS) {
        const float2 ml = *reinterpret_cast<const float2*>(recs + (size_t)lane * (D + 4) + D);
        ms = ml.x;
        ls = ml.y;
    }
    float M = ms;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    // weight of split `lane` (0 for a split that saw no token, and for all
    // of them when no split did)
    const float wl = (ms == -INFINITY) ? 0.f : exp2_fast(ms - M);
    float L = ls * wl;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    float acc[PL] = {};
    for (int s0 = 0; s0 < p.NS; s0 += BATCH) {
        float v[BATCH][PL];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int sp = min(s0 + j, p.NS - 1);
            const float* r = recs + (size_t)sp * (D + 4) + PL * lane;
#pragma unroll
            for (int c = 0; c < PL; ++c) v[j][c] = r[c];
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            if (s0 + j >= p.NS) break;
            const float wgt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s0 + j));
            if (wgt == 0.f) continue;
#pragma unroll
            for (int c = 0; c < PL; ++c) acc[c] = __builtin_fmaf(v[j][c], wgt, acc[c]);
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float* out = p.out + row * D + PL * lane;
#pragma unroll
    for (int c = 0; c < PL; ++c) out[c] = acc[c] * inv;
}

int prefill_query_tile(int P) { return P <= QT_HALF ? QT_HALF : QT; }

hipError_t launch_prefill(const PrefillParams& pp, int D, hipStream_t st) {
    const int qt = prefill_query_tile(pp.P);
    const bool half = qt == QT_HALF;
    const dim3 grid((pp.P + qt - 1) / qt, pp.NS, pp.B * pp.Hq);
    const size_t rows = (size_t)pp.B * pp.Hq * pp.P;
    const dim3 cgrid((unsigned)((rows + 3) / 4));
    if (D == 128) {
        if (half) prefill_tile_kernel<128, true><<<grid, PT, 0, st>>>(pp);
        else prefill_tile_kernel<128, false><<<grid, PT, 0, st>>>(pp);
        prefill_combine_kernel<128><<<cgrid, 256, 0, st>>>(pp);
    } else if (D == 64) {
        if (half) prefill_tile_kernel<64, true><<<grid, PT, 0, st>>>(pp);
        else prefill_tile_kernel<64, false><<<grid, PT, 0, st>>>(pp);
        prefill_combine_kernel<64><<<cgrid, 256, 0, st>>>(pp);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mkv
