// Split-K decode attention over the mixed-bitwidth packed cache
// (MoQAE "Overall framework": ordinary attention after quantization;
// Cocktail abstract: chunk-level computation over bitwidth-contiguous
// segments, so every tile below has a single bitwidth and no wavefront ever
// branches on bitwidth inside its inner loop).
//
// Work unit: one 64-lane wavefront = one tile = a run of group blocks
// (32 tokens each) of one (sequence, KV head, bitwidth segment).  A wave is
// split into R = 64/S rows of S = d/8 lanes; each row handles one group
// block per iteration (GQA: the rows of one iteration take the same group
// for different query heads).  Inside a row, lane slot L owns channels
// 8L..8L+7 of the keys and value group L % (d/32) of tokens L / (d/32) + 4m.
//
// Scores: s_t = sum_j q_j * (code_tj * s_j + mn_j) is evaluated as
// sum_j (q_j s_j) code_tj + sum_j q_j mn_j, so key dequantization costs one
// FMA per code.  Codes are unpacked with v_cvt_f32_ubyteN on masked words,
// and scale factors of 16 / 4^m are folded into the per-channel weights.
// Per-row partial sums are combined with a select-free DPP reduce-scatter
// (the layout's per-lane token xor makes every butterfly step keep the low
// registers).  Values: o_j = sum_t (p_t s_t) code_tj + sum_t p_t mn_t.
// Everything accumulates in fp32; softmax is online, in the log2 domain.
#include "mkv_internal.h"
#include "mkv_kernels.h"

namespace mkv {

namespace {

constexpr int kDppRowMirror = 0x140;      // lane i <-> 15 - i within 16
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i within 8
constexpr int kDppXor1 = 0xB1;            // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;            // quad_perm [2,3,0,1]

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int B>
__device__ __forceinline__ float cvt_ub(uint32_t x) {
    float r;
    if constexpr (B == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x));
    else if constexpr (B == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x));
    else if constexpr (B == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t as_h2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }
__device__ __forceinline__ float lo_h(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float hi_h(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row-wide max over the S lanes of a row (butterfly; every lane gets it).
template <int S>
__device__ __forceinline__ float row_max(float v) {
    if constexpr (S == 16) v = fmaxf(v, dpp<kDppRowMirror>(v));
    v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppXor1>(v));
    return v;
}

// Reduce-scatter of 32 per-token partial sums over the S lanes of a row.
// On return acc[0 .. 32/S-1] hold the full sums of tokens tok_xor(S,L) ^ i.
template <int S>
__device__ __forceinline__ void row_reduce_scatter(float* acc) {
    if constexpr (S == 16) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += dpp<kDppRowMirror>(acc[r + 16]);
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] += dpp<kDppRowHalfMirror>(acc[r + 8]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += dpp<kDppXor2>(acc[r + 4]);
#pragma unroll
        for (int r = 0; r < 2; ++r) acc[r] += dpp<kDppXor1>(acc[r + 2]);
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += dpp<kDppRowHalfMirror>(acc[r + 16]);
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] += dpp<kDppXor2>(acc[r + 8]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += dpp<kDppXor1>(acc[r + 4]);
    }
}

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ float4 ldf4(const uint8_t* p) { return *reinterpret_cast<const float4*>(p); }

template <int BITS, int D, int HB>
__device__ __forceinline__ void tile_body(const AttnParams& p, int k, int bh, int x, int g0, int g1) {
    constexpr int S = D / 8;
    constexpr int R = 64 / S;          // rows per wave
    constexpr int NG = D / 32;         // value groups per token
    constexpr int GPI = R / HB;        // group blocks per iteration
    constexpr int NT = 32 / S;         // tokens per lane after the reduce-scatter
    constexpr int KCR = kc_rows(BITS);
    constexpr int VCR = vc_rows(BITS);
    constexpr size_t GB = group_bytes(BITS, D);
    constexpr size_t ROWB = (size_t)S * 16;

    __shared__ float plds[R][32];

    const int lane = threadIdx.x;
    const int row = lane / S, L = lane % S;
    const int hb = row % HB, gslot = row / HB;
    const int G = L % NG, tq = L / NG;
    const int fx = tok_xor(S, L);
    const int C = p.C;
    const int b = bh / p.Hkv, h = bh % p.Hkv;
    const int hq = h * HB + hb;

    const uint8_t* seg = p.pool[k] + (size_t)bh * p.cap[k] * (C / kGroup) * GB;

    // query channels 8L..8L+7 of head hq
    const uint4 qc = *reinterpret_cast<const uint4*>(p.q + ((size_t)b * p.Hq + hq) * D + 8 * L);
    const uint32_t qw[4] = {qc.x, qc.y, qc.z, qc.w};
    float qs[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        qs[2 * e] = lo_h(qw[e]) * p.qscale;
        qs[2 * e + 1] = hi_h(qw[e]) * p.qscale;
    }

    float M = -INFINITY;   // running max of this row (log2 domain), row-uniform
    float lsum = 0.f;      // this lane's share of the softmax denominator
    float o[32];           // channels 32G .. 32G+31
    float pm = 0.f;        // sum_t p_t * mn_t over this lane's value tokens
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] = 0.f;

    for (int gbase = g0; gbase < g1; gbase += GPI) {
        const int gi = gbase + gslot;
        const bool valid = gi < g1;
        const uint8_t* gp = seg + (size_t)(valid ? gi : g1 - 1) * GB;

        // ---------------- scores
        float acc[32];
        if constexpr (BITS == 16) {
            const half2_t q0 = as_h2(qw[0]), q1 = as_h2(qw[1]), q2 = as_h2(qw[2]), q3 = as_h2(qw[3]);
#pragma unroll
            for (int r = 0; r < 32; ++r) {
                const uint4 c = ld16(gp + r * ROWB + L * 16);
                float a = __builtin_amdgcn_fdot2(as_h2(c.x), q0, 0.f, false);
                a = __builtin_amdgcn_fdot2(as_h2(c.y), q1, a, false);
                a = __builtin_amdgcn_fdot2(as_h2(c.z), q2, a, false);
                a = __builtin_amdgcn_fdot2(as_h2(c.w), q3, a, false);
                acc[r] = a;
            }
        } else {
            uint4 kc[KCR];
#pragma unroll
            for (int i = 0; i < KCR; ++i) kc[i] = ld16(gp + i * ROWB + L * 16);
            const uint8_t* kmp = gp + (size_t)km_row0(BITS) * ROWB + L * 16;
            const float4 s0 = ldf4(kmp), s1 = ldf4(kmp + ROWB), m0 = ldf4(kmp + 2 * ROWB), m1 = ldf4(kmp + 3 * ROWB);
            const float ks[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
            const float kmn[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
            float bias = 0.f;
            float qp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bias = __builtin_fmaf(qs[e], kmn[e], bias);
                qp[e] = qs[e] * ks[e];
            }
#pragma unroll
            for (int r = 0; r < 32; ++r) acc[r] = bias;
            if constexpr (BITS == 4) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int w = i >> 1;
                    const uint32_t ws[4] = {kc[i].x, kc[i].y, kc[i].z, kc[i].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float qa = qp[4 * (i & 1) + e];
                        const float qb = qa * 0.0625f;
                        const uint32_t lo = ws[e] & 0x0F0F0F0Fu, hi = ws[e] & 0xF0F0F0F0u;
                        acc[8 * w + 0] = __builtin_fmaf(qa, cvt_ub<0>(lo), acc[8 * w + 0]);
                        acc[8 * w + 1] = __builtin_fmaf(qb, cvt_ub<0>(hi), acc[8 * w + 1]);
                        acc[8 * w + 2] = __builtin_fmaf(qa, cvt_ub<1>(lo), acc[8 * w + 2]);
                        acc[8 * w + 3] = __builtin_fmaf(qb, cvt_ub<1>(hi), acc[8 * w + 3]);
                        acc[8 * w + 4] = __builtin_fmaf(qa, cvt_ub<2>(lo), acc[8 * w + 4]);
                        acc[8 * w + 5] = __builtin_fmaf(qb, cvt_ub<2>(hi), acc[8 * w + 5]);
                        acc[8 * w + 6] = __builtin_fmaf(qa, cvt_ub<3>(lo), acc[8 * w + 6]);
                        acc[8 * w + 7] = __builtin_fmaf(qb, cvt_ub<3>(hi), acc[8 * w + 7]);
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int w = i >> 1;
                    const uint32_t ws[4] = {kc[i].x, kc[i].y, kc[i].z, kc[i].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float q0 = qp[4 * (i & 1) + e];
                        const float qm[4] = {q0, q0 * 0.25f, q0 * 0.0625f, q0 * 0.015625f};
#pragma unroll
                        for (int mm = 0; mm < 4; ++mm) {
                            const uint32_t part = ws[e] & (0x03030303u << (2 * mm));
                            acc[16 * w + 0 + mm] = __builtin_fmaf(qm[mm], cvt_ub<0>(part), acc[16 * w + 0 + mm]);
                            acc[16 * w + 4 + mm] = __builtin_fmaf(qm[mm], cvt_ub<1>(part), acc[16 * w + 4 + mm]);
                            acc[16 * w + 8 + mm] = __builtin_fmaf(qm[mm], cvt_ub<2>(part), acc[16 * w + 8 + mm]);
                            acc[16 * w + 12 + mm] = __builtin_fmaf(qm[mm], cvt_ub<3>(part), acc[16 * w + 12 + mm]);
                        }
                    }
                }
            }
        }
        row_reduce_scatter<S>(acc);
        float sc[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            float v = acc[i];
            if constexpr (BITS == 16) v *= p.qscale;
            sc[i] = valid ? v : -INFINITY;
        }

        // ---------------- online softmax (row-uniform running max)
        float mloc = sc[0];
#pragma unroll
        for (int i = 1; i < NT; ++i) mloc = fmaxf(mloc, sc[i]);
        mloc = row_max<S>(mloc);
        const float Mn = fmaxf(M, mloc);
        const float alpha = (Mn == -INFINITY) ? 1.f : fast_exp2(M - Mn);
        M = Mn;
        float pt[NT];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            pt[i] = valid ? fast_exp2(sc[i] - Mn) : 0.f;
            psum += pt[i];
        }
        lsum = __builtin_fmaf(lsum, alpha, psum);
        pm *= alpha;
#pragma unroll
        for (int c = 0; c < 32; ++c) o[c] *= alpha;

        // hand the probabilities to the value layout: slot (t & 3) * 8 + (t >> 2)
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const int t = fx ^ i;
            plds[row][(t & 3) * 8 + (t >> 2)] = pt[i];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const float4 pa = *reinterpret_cast<const float4*>(&plds[row][tq * 8]);
        const float4 pb = *reinterpret_cast<const float4*>(&plds[row][tq * 8 + 4]);
        const float pv8[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};

        // ---------------- values
        const uint8_t* vcp = gp + (size_t)vc_row0(BITS) * ROWB + L * 16;
        if constexpr (BITS == 16) {
#pragma unroll
            for (int r = 0; r < 32; ++r) {
                const uint4 c = ld16(vcp + r * ROWB);
                const float pr = pv8[r >> 2];
                const int cb = 8 * (r & 3);
                const uint32_t ws[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[cb + 2 * e] = __builtin_fmaf(pr, lo_h(ws[e]), o[cb + 2 * e]);
                    o[cb + 2 * e + 1] = __builtin_fmaf(pr, hi_h(ws[e]), o[cb + 2 * e + 1]);
                }
            }
        } else {
            uint4 vc[VCR];
#pragma unroll
            for (int i = 0; i < VCR; ++i) vc[i] = ld16(vcp + i * ROWB);
            const uint8_t* vmp = gp + (size_t)vm_row0(BITS) * ROWB + L * 16;
            float4 vm[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) vm[i] = ldf4(vmp + i * ROWB);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const float s = (m & 1) ? vm[m >> 1].z : vm[m >> 1].x;
                const float mn = (m & 1) ? vm[m >> 1].w : vm[m >> 1].y;
                const float pr = pv8[m];
                const float pv = pr * s;
                pm = __builtin_fmaf(pr, mn, pm);
                if constexpr (BITS == 4) {
                    const uint32_t ws[4] = {vc[m].x, vc[m].y, vc[m].z, vc[m].w};
                    const float pb16 = pv * 0.0625f;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint32_t lo = ws[u] & 0x0F0F0F0Fu, hi = ws[u] & 0xF0F0F0F0u;
                        o[8 * u + 0] = __builtin_fmaf(pv, cvt_ub<0>(lo), o[8 * u + 0]);
                        o[8 * u + 1] = __builtin_fmaf(pb16, cvt_ub<0>(hi), o[8 * u + 1]);
                        o[8 * u + 2] = __builtin_fmaf(pv, cvt_ub<1>(lo), o[8 * u + 2]);
                        o[8 * u + 3] = __builtin_fmaf(pb16, cvt_ub<1>(hi), o[8 * u + 3]);
                        o[8 * u + 4] = __builtin_fmaf(pv, cvt_ub<2>(lo), o[8 * u + 4]);
                        o[8 * u + 5] = __builtin_fmaf(pb16, cvt_ub<2>(hi), o[8 * u + 5]);
                        o[8 * u + 6] = __builtin_fmaf(pv, cvt_ub<3>(lo), o[8 * u + 6]);
                        o[8 * u + 7] = __builtin_fmaf(pb16, cvt_ub<3>(hi), o[8 * u + 7]);
                    }
                } else {
                    const uint32_t w0 = (m & 1) ? vc[m >> 1].z : vc[m >> 1].x;
                    const uint32_t w1 = (m & 1) ? vc[m >> 1].w : vc[m >> 1].y;
                    const uint32_t ws[2] = {w0, w1};
                    const float pvm[4] = {pv, pv * 0.25f, pv * 0.0625f, pv * 0.015625f};
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
#pragma unroll
                        for (int mm = 0; mm < 4; ++mm) {
                            const uint32_t part = ws[u] & (0x03030303u << (2 * mm));
                            o[16 * u + 0 + mm] = __builtin_fmaf(pvm[mm], cvt_ub<0>(part), o[16 * u + 0 + mm]);
                            o[16 * u + 4 + mm] = __builtin_fmaf(pvm[mm], cvt_ub<1>(part), o[16 * u + 4 + mm]);
                            o[16 * u + 8 + mm] = __builtin_fmaf(pvm[mm], cvt_ub<2>(part), o[16 * u + 8 + mm]);
                            o[16 * u + 12 + mm] = __builtin_fmaf(pvm[mm], cvt_ub<3>(part), o[16 * u + 12 + mm]);
                        }
                    }
                }
            }
        }
    }

    // ---------------- merge rows of the same head, then lanes of the same value group
    if constexpr (BITS != 16) {
#pragma unroll
        for (int c = 0; c < 32; ++c) o[c] += pm;
    }
    float Mx = M;
#pragma unroll
    for (int off = S * HB; off < 64; off <<= 1) Mx = fmaxf(Mx, __shfl_xor(Mx, off));
    const float sc = (M == -INFINITY) ? 0.f : fast_exp2(M - Mx);
    lsum *= sc;
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] *= sc;
#pragma unroll
    for (int off = 1; off < S; off <<= 1) lsum += __shfl_xor(lsum, off);
#pragma unroll
    for (int off = S * HB; off < 64; off <<= 1) lsum += __shfl_xor(lsum, off);
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        float v = o[c];
#pragma unroll
        for (int off = NG; off < S; off <<= 1) v += __shfl_xor(v, off);
#pragma unroll
        for (int off = S * HB; off < 64; off <<= 1) v += __shfl_xor(v, off);
        o[c] = v;
    }
    if (row == hb && tq == 0) {
        float* rec = p.part + (((size_t)bh * p.nt_total + x) * HB + hb) * (D + 4);
        float4* o4 = reinterpret_cast<float4*>(rec + 32 * G);
#pragma unroll
        for (int c = 0; c < 8; ++c) o4[c] = make_float4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
        if (G == 0) *reinterpret_cast<float4*>(rec + D) = make_float4(Mx, lsum, 0.f, 0.f);
    }
}

__device__ __forceinline__ void tile_of(const int* nt, int x, int& k, int& j) {
    if (x < nt[0]) { k = 0; j = x; }
    else if (x < nt[0] + nt[1]) { k = 1; j = x - nt[0]; }
    else { k = 2; j = x - nt[0] - nt[1]; }
}

}  // namespace

template <int D, int HB>
__global__ __launch_bounds__(64) void attn_tile_kernel(AttnParams p) {
    const int x = blockIdx.x, bh = blockIdx.y;
    int k, j;
    tile_of(p.nt, x, k, j);
    const int b = bh / p.Hkv;
    // chunks beyond the pool's capacity were never written: never read them
    const int seg_groups = min(p.seg_count[b * 3 + k], p.cap[k]) * (p.C / kGroup);
    const int g0 = j * p.tg[k];
    if (g0 >= seg_groups) return;
    const int g1 = min(g0 + p.tg[k], seg_groups);
    if (k == 0) tile_body<16, D, HB>(p, k, bh, x, g0, g1);
    else if (k == 1) tile_body<4, D, HB>(p, k, bh, x, g0, g1);
    else tile_body<2, D, HB>(p, k, bh, x, g0, g1);
}

// One block of D threads per (sequence, query head): thread j owns channel j.
template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(CombineParams p) {
    __shared__ float ts[4096];
    __shared__ float qsh[D];
    const int bq = blockIdx.x;
    const int b = bq / p.Hq, hq = bq % p.Hq;
    const int g = p.Hq / p.Hkv;
    const int h = hq / g, hb = hq % g;
    const int bh = b * p.Hkv + h;
    const int j = threadIdx.x;
    const int gpc = p.C / kGroup;
    int seg_groups[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) seg_groups[k] = min(p.seg_count[b * 3 + k], p.cap[k]) * gpc;

    float M = -INFINITY;
    for (int x = 0; x < p.nt_total; ++x) {
        int k, jt;
        tile_of(p.nt, x, k, jt);
        if (jt * p.tg[k] >= seg_groups[k]) continue;
        const float* rec = p.part + (((size_t)bh * p.nt_total + x) * g + hb) * (D + 4);
        M = fmaxf(M, rec[D]);
    }
    const int tl = p.tail_len;
    if (tl > 0) {
        qsh[j] = (float)__builtin_bit_cast(_Float16, p.q[((size_t)b * p.Hq + hq) * D + j]);
        __syncthreads();
        const uint16_t* tk = p.tail_k + (size_t)bh * tl * D;
        for (int t = j; t < tl; t += D) {
            float a = 0.f;
            for (int c = 0; c < D; ++c) a = __builtin_fmaf(qsh[c], (float)__builtin_bit_cast(_Float16, tk[(size_t)t * D + c]), a);
            ts[t] = a * p.qscale;
        }
        __syncthreads();
        for (int t = 0; t < tl; ++t) M = fmaxf(M, ts[t]);
    }
    float l = 0.f, o = 0.f;
    for (int x = 0; x < p.nt_total; ++x) {
        int k, jt;
        tile_of(p.nt, x, k, jt);
        if (jt * p.tg[k] >= seg_groups[k]) continue;
        const float* rec = p.part + (((size_t)bh * p.nt_total + x) * g + hb) * (D + 4);
        const float w = fast_exp2(rec[D] - M);
        l = __builtin_fmaf(w, rec[D + 1], l);
        o = __builtin_fmaf(w, rec[j], o);
    }
    if (tl > 0) {
        const uint16_t* tv = p.tail_v + (size_t)bh * tl * D;
        for (int t = 0; t < tl; ++t) {
            const float w = fast_exp2(ts[t] - M);
            l += w;
            o = __builtin_fmaf(w, (float)__builtin_bit_cast(_Float16, tv[(size_t)t * D + j]), o);
        }
    }
    p.out[((size_t)b * p.Hq + hq) * D + j] = l > 0.f ? o / l : 0.f;
}

hipError_t launch_attention(const AttnParams& ap, const CombineParams& cp, int D, int HB, hipStream_t st) {
    const dim3 grid_t(ap.nt_total, ap.B * ap.Hkv);
    if (ap.nt_total > 0) {
#define MKV_ATTN_CASE(DD, HH)                                                        \
        if (D == DD && HB == HH) attn_tile_kernel<DD, HH><<<grid_t, 64, 0, st>>>(ap); \
        else
        MKV_ATTN_CASE(128, 1) MKV_ATTN_CASE(128, 2) MKV_ATTN_CASE(128, 4)
        MKV_ATTN_CASE(64, 1) MKV_ATTN_CASE(64, 2) MKV_ATTN_CASE(64, 4)
        return hipErrorInvalidValue;
#undef MKV_ATTN_CASE
    }
    const dim3 grid_c(cp.B * cp.Hq);
    if (D == 128) attn_combine_kernel<128><<<grid_c, 128, 0, st>>>(cp);
    else attn_combine_kernel<64><<<grid_c, 64, 0, st>>>(cp);
    return hipGetLastError();
}

}  // namespace mkv
