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
#include "mkv_internal.h"
#include "mkv_kernels.h"

namespace mkv {

namespace {

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// fp16 values of one 16-byte cell (8 channels).
__device__ __forceinline__ void cell_to_float(const uint4& c, float* f) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = h2f(w[i] & 0xFFFFu);
        f[2 * i + 1] = h2f(w[i] >> 16);
    }
}

template <int BITS>
__device__ __forceinline__ uint32_t code_of(float x, float mn, float r, bool zero) {
    constexpr float Lf = (float)((1 << BITS) - 1);
    if (zero) return 0u;
    float t = x - mn;
    t = t * r;
    t = __builtin_rintf(t);          // v_rndne_f32: round half to even
    t = fminf(t, Lf);
    return (uint32_t)t;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(64) void quant_pack_kernel(QuantParams p) {
    constexpr int S = D / 8;          // lane slots (16-byte cells) per token row
    constexpr int TPI = 64 / S;       // tokens covered by one wave-wide load
    constexpr int NL = 32 / TPI;      // loads per lane per tensor
    constexpr int NG = D / 32;        // value groups per token

    __shared__ uint8_t kc_lds[D][32];  // key codes [channel][token]

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

    uint4 kcell[NL], vcell[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int t = tr + TPI * i;
        kcell[i] = ksrc[(size_t)t * (D / 8)];
        vcell[i] = vsrc[(size_t)t * (D / 8)];
    }

    if (bits == 16) {
        // Bit-for-bit copies, rows permuted per the layout.
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int t = tr + TPI * i;
            const int kr = tok_of(S, ls, t);
            *reinterpret_cast<uint4*>(dst + ((size_t)kr * S + ls) * 16) = kcell[i];
            const int vr = ((t >> 2) << 2) | (ls & 3);
            const int vl = vslot_of(t & 3, ls >> 2, NG);
            *reinterpret_cast<uint4*>(dst + ((size_t)(vc_row0(16) + vr) * S + vl) * 16) = vcell[i];
        }
        return;
    }

    auto body = [&](auto bits_tag) {
        constexpr int BITS = decltype(bits_tag)::value;
        constexpr float Lf = (float)((1 << BITS) - 1);
        constexpr int F = 32 / BITS;

        // ---------------- keys: groups of 32 tokens per channel
        float kf[NL][8];
#pragma unroll
        for (int i = 0; i < NL; ++i) cell_to_float(kcell[i], kf[i]);
        float kmn[8], kmx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float a = kf[0][e], c = kf[0][e];
#pragma unroll
            for (int i = 1; i < NL; ++i) { a = fminf(a, kf[i][e]); c = fmaxf(c, kf[i][e]); }
#pragma unroll
            for (int off = S; off < 64; off <<= 1) {
                a = fminf(a, __shfl_xor(a, off));
                c = fmaxf(c, __shfl_xor(c, off));
            }
            kmn[e] = a + 0.0f;
            kmx[e] = c + 0.0f;
        }
        float ks[8], kr[8];
        bool kz[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float range = kmx[e] - kmn[e];
            ks[e] = range / Lf;
            kz[e] = ks[e] == 0.0f;
            kr[e] = kz[e] ? 0.0f : 1.0f / ks[e];
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int t = tr + TPI * i;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                kc_lds[8 * ls + e][t] = (uint8_t)code_of<BITS>(kf[i][e], kmn[e], kr[e], kz[e]);
        }
        if (tr == 0) {
            float4* km = reinterpret_cast<float4*>(dst + (size_t)km_row0(BITS) * S * 16);  // key meta rows
            km[0 * S + ls] = make_float4(ks[0], ks[1], ks[2], ks[3]);
            km[1 * S + ls] = make_float4(ks[4], ks[5], ks[6], ks[7]);
            km[2 * S + ls] = make_float4(kmn[0], kmn[1], kmn[2], kmn[3]);
            km[3 * S + ls] = make_float4(kmn[4], kmn[5], kmn[6], kmn[7]);
        }

        // ---------------- values: groups of 32 channels per token
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int t = tr + TPI * i;
            float vf[8];
            cell_to_float(vcell[i], vf);
            float a = vf[0], c = vf[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) { a = fminf(a, vf[e]); c = fmaxf(c, vf[e]); }
            // the 4 lanes ls = 4G..4G+3 of this token hold the group's 32 channels
            a = fminf(a, __shfl_xor(a, 1)); c = fmaxf(c, __shfl_xor(c, 1));
            a = fminf(a, __shfl_xor(a, 2)); c = fmaxf(c, __shfl_xor(c, 2));
            const float mn = a + 0.0f;
            const float mx = c + 0.0f;
            const float s = (mx - mn) / Lf;
            const bool z = s == 0.0f;
            const float r = z ? 0.0f : 1.0f / s;
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) word |= code_of<BITS>(vf[e], mn, r, z) << (BITS * e);
            const int G = ls >> 2;
            const int m = t >> 2;
            const int vl = vslot_of(t & 3, G, NG);
            uint8_t* vc = dst + (size_t)vc_row0(BITS) * S * 16;
            if constexpr (BITS == 4) {
                // word u = ls of the token (channels 8ls..8ls+7) is dword ls&3 of the cell
                *reinterpret_cast<uint32_t*>(vc + ((size_t)m * S + vl) * 16 + (ls & 3) * 4) = word;
            } else {
                // 16 bits per lane; lanes 2u', 2u'+1 form word u' = ls>>1 (low half from the even lane)
                const uint32_t other = __shfl_xor(word, 1);
                if ((ls & 1) == 0) {
                    const uint32_t full = word | (other << 16);
                    const int upos = (ls >> 1) & 1;
                    *reinterpret_cast<uint32_t*>(vc + ((size_t)(m >> 1) * S + vl) * 16 + ((m & 1) * 2 + upos) * 4) = full;
                }
            }
            if ((ls & 3) == 0) {
                uint8_t* vm = dst + (size_t)vm_row0(BITS) * S * 16;
                *reinterpret_cast<float2*>(vm + ((size_t)(m >> 1) * S + vl) * 16 + (m & 1) * 8) = make_float2(s, mn);
            }
        }

        __syncthreads();
        // ---------------- key code cells: gather from LDS in the reader's order
        constexpr int KCR = kc_rows(BITS);
        uint8_t* kcd = dst + (size_t)kc_row0(BITS) * S * 16;
        for (int c = lane; c < KCR * S; c += 64) {
            const int row = c / S, L = c % S;
            const int w = row >> 1;
            uint32_t words[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 8 * L + 4 * (row & 1) + e;
                uint32_t acc = 0;
#pragma unroll
                for (int i = 0; i < F; ++i) acc |= (uint32_t)kc_lds[j][tok_of(S, L, F * w + i)] << (BITS * i);
                words[e] = acc;
            }
            *reinterpret_cast<uint4*>(kcd + ((size_t)row * S + L) * 16) = make_uint4(words[0], words[1], words[2], words[3]);
        }
    };
    if (bits == 4) body(std::integral_constant<int, 4>{});
    else body(std::integral_constant<int, 2>{});
}

hipError_t launch_quant(const QuantParams& qp, int D, int ngroups, hipStream_t st) {
    const dim3 grid(ngroups, qp.B * qp.Hkv);
    if (D == 128) quant_pack_kernel<128><<<grid, 64, 0, st>>>(qp);
    else quant_pack_kernel<64><<<grid, 64, 0, st>>>(qp);
    return hipGetLastError();
}

}  // namespace mkv
