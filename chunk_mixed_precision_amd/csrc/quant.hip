// Quantize + pack one layer's K/V of routed chunks into the per-bitwidth
// segment pools (MoQAE "Overall framework": the cache is quantized at the
// voted bitwidth; "Related work", KIVI: keys per channel; Cocktail abstract:
// chunks land in their bitwidth's contiguous segment).
//
// One 64-lane wavefront handles one group block: 32 tokens of one
// (sequence, KV head).  Arithmetic is float32 with one rounding per
// operation (this file is built with -ffp-contract=off):
//   mn = min + 0, mx = max + 0 (a -0 extreme becomes +0), s = (mx - mn) / L,
//   r = 1 / s,
//   code = min(rint((x - mn) * r), L),   s == 0 -> all codes 0.
// For INT-b chunks every lane owns whole quantization groups, so minima,
// maxima, divisions and packing need no other lane: keys pass once through
// LDS (16-byte row stores, then each lane reads its D/64 channels of all 32
// tokens, in the order in which the reader's fields hold them); values are
// read directly as whole 32-channel groups of one token.  Inputs are
// expected to be finite.
#include "mkv_internal.h"
#include "mkv_kernels.h"

namespace mkv {

// Pool writes are streaming: every byte is written once and read back only by
// later calls, so they go out as nontemporal stores (the `nt` bit), which
// measured a few percent faster than plain stores here.
template <class T>
__device__ __forceinline__ void store_nt(uint8_t* p, T v) {
    static_assert(sizeof(T) % 4 == 0, "whole dwords");
    typedef uint32_t dwords __attribute__((ext_vector_type(sizeof(T) / 4)));
    __builtin_nontemporal_store(__builtin_bit_cast(dwords, v), reinterpret_cast<dwords*>(p));
}


namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// fl(x - mn) for the fp16 value in the low (HI = 0) or high half of w, in one
// v_fma_mix_f32 (x * 1 + (-mn), a single rounding): the same value as
// converting x exactly to float32 and subtracting.
template <int HI>
__device__ __forceinline__ float sub_mix(uint32_t w, float neg_mn) {
    float r;
    if constexpr (HI == 0)
        asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(neg_mn));
    else
        asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(neg_mn));
    return r;
}

// The code of one value as a float: rint(fl(fl(x - mn) * r)).  The clamp to
// L of the definition is never active: x <= mx gives
// fl(x - mn) * r <= fl(mx - mn) * fl(1 / fl((mx - mn) / L)) = L (1 + d),
// |d| <= 3 * 2^-24, which rounds to L; s == 0 gives r = 0 and code 0.
template <int HI>
__device__ __forceinline__ float code_f(uint32_t w, float neg_mn, float r) {
    return __builtin_rintf(sub_mix<HI>(w, neg_mn) * r);
}

// Scale, reciprocal and minimum of one group from its fp16 extremes.
template <int BITS>
__device__ __forceinline__ void group_params(_Float16 mnh, _Float16 mxh, float& s, float& r, float& mn) {
    constexpr float Lf = (float)((1 << BITS) - 1);
    mn = (float)mnh + 0.0f;
    const float mx = (float)mxh + 0.0f;
    s = (mx - mn) / Lf;
    r = s == 0.0f ? 0.0f : 1.0f / s;
}

// Pack 8 (INT4) or 16 (INT2) codes, given as floats, LSB first into a word.
template <int BITS>
__device__ __forceinline__ uint32_t pack_word(const float* c) {
    uint32_t w = 0;
    if constexpr (BITS == 4) {
#pragma unroll
        for (int b = 0; b < 4; ++b) w = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(c[2 * b + 1], 16.f, c[2 * b]), b, w);
    } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float v = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(c[4 * b + 3], 4.f, c[4 * b + 2]), 4.f, c[4 * b + 1]), 4.f, c[4 * b]);
            w = __builtin_amdgcn_cvt_pk_u8_f32(v, b, w);
        }
    }
    return w;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(64) void quant_pack_kernel(QuantParams p) {
    constexpr int S = D / 8;          // lane slots (16-byte cells) per token row
    constexpr int TPI = 64 / S;       // tokens covered by one wave-wide load
    constexpr int NL = 32 / TPI;      // loads per lane per tensor
    constexpr int NG = D / 32;        // value groups per token

    __shared__ __align__(16) _Float16 k_lds[32][D];  // key tile [token][channel]

    const int lane = threadIdx.x;
    const int ls = lane % S, tr = lane / S;
    const int gi = blockIdx.x;
    const int bh = blockIdx.y;
    const int b = bh / p.Hkv;
    const int gpc = p.C / kGroup;
    const int chunk = p.chunk_offset + gi / gpc;
    const int gg = gi % gpc;

    const int bits = p.chunk_bits[(size_t)b * p.n_max + chunk];
    const int k = expert_of_bits(bits);
    const int rank = p.chunk_rank[(size_t)b * p.n_max + chunk];
    if (k < 0 || rank < 0 || rank >= p.cap[k]) {
        if (lane == 0 && p.overflow) p.overflow[0] = 1;
        return;
    }
    const size_t GB = group_bytes(bits, D);
    uint8_t* dst = p.pool[k] + (((size_t)bh * p.cap[k] + rank) * gpc + gg) * GB;

    const size_t src_off = ((size_t)bh * p.T + (size_t)gi * kGroup) * D + 8 * ls;
    const uint4* ksrc = reinterpret_cast<const uint4*>(p.k + src_off);
    const uint4* vsrc = reinterpret_cast<const uint4*>(p.v + src_off);

    if (bits == 16) {
        // Bit-for-bit copies, rows permuted per the layout.
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4* ks4 = reinterpret_cast<const u32x4*>(ksrc);
        const u32x4* vs4 = reinterpret_cast<const u32x4*>(vsrc);
        u32x4 kcell[NL], vcell[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int t = tr + TPI * i;
            kcell[i] = ks4[(size_t)t * (D / 8)];
            vcell[i] = vs4[(size_t)t * (D / 8)];
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int t = tr + TPI * i;
            const int kr = tok_of(S, ls, t);
            store_nt(dst + ((size_t)kr * S + ls) * 16, kcell[i]);
            const int vr = ((t >> 2) << 2) | (ls & 3);
            const int vl = vslot_of(t & 3, ls >> 2, NG);
            store_nt(dst + ((size_t)(vc_row0(16) + vr) * S + vl) * 16, vcell[i]);
        }
        return;
    }

    auto body = [&](auto bits_tag) {
        constexpr int BITS = decltype(bits_tag)::value;
        constexpr int F = 32 / BITS;             // codes per word
        constexpr int CPL = D / 64;              // key channels per lane
        constexpr int UPL = D / 64;              // value groups (token x 32 channels) per lane

        // ---------------- keys: the block's 32 x D fp16 tile through LDS
        uint4 kcell[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) kcell[i] = ksrc[(size_t)(tr + TPI * i) * (D / 8)];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int t = tr + TPI * i;
            *reinterpret_cast<uint4*>(&k_lds[t][8 * ls]) = kcell[i];
        }
        // values of this lane's groups: 64 contiguous bytes each
        uint4 vg[UPL][4];
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
            const int u = lane + 64 * j, t = u / NG, G = u % NG;
            const uint4* src = reinterpret_cast<const uint4*>(p.v + ((size_t)bh * p.T + (size_t)gi * kGroup + t) * D + 32 * G);
#pragma unroll
            for (int c = 0; c < 4; ++c) vg[j][c] = src[c];
        }
        __syncthreads();

        // key channels j0 .. j0+CPL-1 of all 32 tokens, field position r
        // holding token tok(L, r) of the reader's lane slot L
        const int j0 = CPL * lane, L = j0 >> 3, sub = (j0 >> 2) & 1, e0 = j0 & 3;
        uint32_t kw[32];
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            const int t = tok_of(D / 8, L, r);
            if constexpr (CPL == 2) kw[r] = *reinterpret_cast<const uint32_t*>(&k_lds[t][j0]);
            else kw[r] = (uint32_t)__builtin_bit_cast(uint16_t, k_lds[t][j0]);
        }
        float ks[CPL], kr[CPL], kmn[CPL], kneg[CPL];
        {
            half2_t mn = __builtin_bit_cast(half2_t, kw[0]), mx = mn;
#pragma unroll
            for (int r = 1; r < 32; ++r) {
                const half2_t x = __builtin_bit_cast(half2_t, kw[r]);
                mn = __builtin_elementwise_min(mn, x);
                mx = __builtin_elementwise_max(mx, x);
            }
            group_params<BITS>(mn.x, mx.x, ks[0], kr[0], kmn[0]);
            if constexpr (CPL == 2) group_params<BITS>(mn.y, mx.y, ks[1], kr[1], kmn[1]);
#pragma unroll
            for (int c = 0; c < CPL; ++c) kneg[c] = -kmn[c];
        }
        uint8_t* kcd = dst + (size_t)kc_row0(BITS) * S * 16;
#pragma unroll
        for (int w = 0; w < 32 / F; ++w) {
            uint32_t word[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                float cf[F];
#pragma unroll
                for (int i = 0; i < F; ++i)
                    cf[i] = c == 0 ? code_f<0>(kw[F * w + i], kneg[0], kr[0]) : code_f<1>(kw[F * w + i], kneg[c], kr[c]);
                word[c] = pack_word<BITS>(cf);
            }
            uint8_t* at = kcd + ((size_t)(2 * w + sub) * S + L) * 16 + e0 * 4;
            if constexpr (CPL == 2) store_nt(at, make_uint2(word[0], word[1]));
            else store_nt(at, word[0]);
        }
        {   // key meta: rows 0/1 scales, rows 2/3 minima of channels 8L + 4 sub + e
            uint8_t* km = dst + (size_t)km_row0(BITS) * S * 16;
            uint8_t* as = km + ((size_t)sub * S + L) * 16 + e0 * 4;
            uint8_t* am = km + ((size_t)(2 + sub) * S + L) * 16 + e0 * 4;
            if constexpr (CPL == 2) {
                store_nt(as, make_float2(ks[0], ks[1]));
                store_nt(am, make_float2(kmn[0], kmn[1]));
            } else {
                store_nt(as, ks[0]);
                store_nt(am, kmn[0]);
            }
        }

        // ---------------- values: groups of 32 channels of one token
        uint8_t* vcd = dst + (size_t)vc_row0(BITS) * S * 16;
        uint8_t* vmd = dst + (size_t)vm_row0(BITS) * S * 16;
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
            const int u = lane + 64 * j, t = u / NG, G = u % NG;
            const uint32_t vw[16] = {vg[j][0].x, vg[j][0].y, vg[j][0].z, vg[j][0].w, vg[j][1].x, vg[j][1].y,
                                     vg[j][1].z, vg[j][1].w, vg[j][2].x, vg[j][2].y, vg[j][2].z, vg[j][2].w,
                                     vg[j][3].x, vg[j][3].y, vg[j][3].z, vg[j][3].w};
            half2_t mn = __builtin_bit_cast(half2_t, vw[0]), mx = mn;
#pragma unroll
            for (int i = 1; i < 16; ++i) {
                const half2_t x = __builtin_bit_cast(half2_t, vw[i]);
                mn = __builtin_elementwise_min(mn, x);
                mx = __builtin_elementwise_max(mx, x);
            }
            const _Float16 mnh = mn.x < mn.y ? mn.x : mn.y;
            const _Float16 mxh = mx.x > mx.y ? mx.x : mx.y;
            float vs, vr, vmn;
            group_params<BITS>(mnh, mxh, vs, vr, vmn);
            const float vneg = -vmn;
            // word u' of the token holds channels F*u' .. F*u' + F-1 of the group
            uint32_t words[32 / F];
#pragma unroll
            for (int w = 0; w < 32 / F; ++w) {
                float cf[F];
#pragma unroll
                for (int i = 0; i < F; i += 2) {
                    cf[i] = code_f<0>(vw[(F * w + i) >> 1], vneg, vr);
                    cf[i + 1] = code_f<1>(vw[(F * w + i) >> 1], vneg, vr);
                }
                words[w] = pack_word<BITS>(cf);
            }
            const int m = t >> 2, Ls = vslot_of(t & 3, G, NG);
            if constexpr (BITS == 4) {
                store_nt(vcd + ((size_t)m * S + Ls) * 16, make_uint4(words[0], words[1], words[2], words[3]));
            } else {
                store_nt(vcd + ((size_t)(m >> 1) * S + Ls) * 16 + (m & 1) * 8, make_uint2(words[0], words[1]));
            }
            store_nt(vmd + ((size_t)(m >> 1) * S + Ls) * 16 + (m & 1) * 8, make_float2(vs, vmn));
        }
    };
    if (bits == 4) body(std::integral_constant<int, 4>{});
    else body(std::integral_constant<int, 2>{});
}

// Each one-wavefront workgroup holds 16 loads (16 KB) in flight.  With only
// the key tile's LDS (8 KB at d = 128) the registers allow 16 of them per
// CU; reserving kQuantLdsPerGroup bytes of LDS per workgroup caps that at 10,
// which streams faster on this part (fewer requests in flight per CU): 4-9 %
// on the 32k, 128k, 13B and GQA layers.
constexpr unsigned kQuantLdsPerGroup = 16384;

hipError_t launch_quant(const QuantParams& qp, int D, int ngroups, hipStream_t st) {
    const dim3 grid(ngroups, qp.B * qp.Hkv);
    if (D == 128) {
        constexpr unsigned used = sizeof(_Float16) * 32 * 128;
        quant_pack_kernel<128><<<grid, 64, kQuantLdsPerGroup - used, st>>>(qp);
    } else {
        constexpr unsigned used = sizeof(_Float16) * 32 * 64;
        quant_pack_kernel<64><<<grid, 64, kQuantLdsPerGroup - used, st>>>(qp);
    }
    return hipGetLastError();
}

}  // namespace mkv
