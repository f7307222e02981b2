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

__device__ __forceinline__ float4 as_f4(const uint4& u) { return __builtin_bit_cast(float4, u); }

// Rows of one load phase.  INT-b: phase 0 = key codes + key meta, phase 1 =
// value codes + value meta.  FP16: eight phases of 8 rows (key rows 0-7,
// 8-15, 16-23, 24-31, then the value rows likewise).
template <int BITS> __host__ __device__ constexpr int ph_rows() { return BITS == 16 ? 8 : 2 * BITS + 4; }
template <int BITS> __host__ __device__ constexpr int n_phases() { return BITS == 16 ? 8 : 2; }

template <int BITS, int D>
__device__ __forceinline__ void load_phase(uint4* buf, const uint8_t* gp, int phase, int L) {
    constexpr int NR = ph_rows<BITS>();
    constexpr size_t ROWB = (size_t)(D / 8) * 16;
    const uint8_t* src = gp + (size_t)phase * NR * ROWB + L * 16;
#pragma unroll
    for (int i = 0; i < NR; ++i) buf[i] = ld16(src + i * ROWB);
}

// Combine the partials of two softmax runs: (m, l, o) <- (m, l, o) + (m2, l2, o2).
template <int N>
__device__ __forceinline__ void merge_run(float& m, float& l, float* o, float m2, float l2, const float* o2) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    const float a = fast_exp2(m - mn), b = fast_exp2(m2 - mn);
    l = l * a + l2 * b;
#pragma unroll
    for (int c = 0; c < N; ++c) o[c] = o[c] * a + o2[c] * b;
    m = mn;
}

template <int BITS, int D, int HB>
__device__ __forceinline__ void tile_body(const AttnParams& p, int k, int bh, int x, int g0, int g1) {
    constexpr int S = D / 8;
    constexpr int R = 64 / S;          // rows per wave
    constexpr int NG = D / 32;         // value groups per token
    constexpr int GPI = R / HB;        // group blocks per iteration
    constexpr int NT = 32 / S;         // tokens per lane after the reduce-scatter
    constexpr int KCR = kc_rows(BITS);
    constexpr int VCR = vc_rows(BITS);
    constexpr int NR = ph_rows<BITS>();
    constexpr size_t GB = group_bytes(BITS, D);

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

    auto group_ptr = [&](int gbase) {
        const int gi = gbase + gslot;
        return seg + (size_t)(gi < g1 ? gi : g1 - 1) * GB;
    };

    // ---- scores of the keys in `acc` -> probabilities in LDS, online-softmax update
    float pv8[8];
    auto softmax_step = [&](float* acc, bool valid) {
        row_reduce_scatter<S>(acc);
        float sc[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            float v = acc[i];
            if constexpr (BITS == 16) v *= p.qscale;
            sc[i] = valid ? v : -INFINITY;
        }
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
        pv8[0] = pa.x; pv8[1] = pa.y; pv8[2] = pa.z; pv8[3] = pa.w;
        pv8[4] = pb.x; pv8[5] = pb.y; pv8[6] = pb.z; pv8[7] = pb.w;
    };

    // ---- INT-b key phase: buf rows 0..KCR-1 codes, KCR..KCR+3 (scale, min)
    auto keys_int = [&](const uint4* buf, float* acc) {
        const float4 s0 = as_f4(buf[KCR]), s1 = as_f4(buf[KCR + 1]);
        const float4 m0 = as_f4(buf[KCR + 2]), m1 = as_f4(buf[KCR + 3]);
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
            for (int i = 0; i < KCR; ++i) {
                const int w = i >> 1;
                const uint32_t ws[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
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
            for (int i = 0; i < KCR; ++i) {
                const int w = i >> 1;
                const uint32_t ws[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
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
    };

    // ---- INT-b value phase: buf rows 0..VCR-1 codes, VCR..VCR+3 (scale, min) pairs
    auto values_int = [&](const uint4* buf) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float4 sm = as_f4(buf[VCR + (m >> 1)]);
            const float s = (m & 1) ? sm.z : sm.x;
            const float mn = (m & 1) ? sm.w : sm.y;
            const float pr = pv8[m];
            const float pv = pr * s;
            pm = __builtin_fmaf(pr, mn, pm);
            if constexpr (BITS == 4) {
                const uint32_t ws[4] = {buf[m].x, buf[m].y, buf[m].z, buf[m].w};
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
                const uint4 c = buf[m >> 1];
                const uint32_t ws[2] = {(m & 1) ? c.z : c.x, (m & 1) ? c.w : c.y};
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
    };

    // ---- FP16 phases: 8 key rows (q . k with v_dot2) or 8 value rows
    const half2_t qh0 = as_h2(qw[0]), qh1 = as_h2(qw[1]), qh2 = as_h2(qw[2]), qh3 = as_h2(qw[3]);
    auto keys_fp16 = [&](const uint4* buf, float* acc) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            float a = __builtin_amdgcn_fdot2(as_h2(buf[r].x), qh0, 0.f, false);
            a = __builtin_amdgcn_fdot2(as_h2(buf[r].y), qh1, a, false);
            a = __builtin_amdgcn_fdot2(as_h2(buf[r].z), qh2, a, false);
            a = __builtin_amdgcn_fdot2(as_h2(buf[r].w), qh3, a, false);
            acc[r] = a;
        }
    };
    auto values_fp16 = [&](const uint4* buf, int mbase) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float pr = pv8[mbase + (r >> 2)];
            const int cb = 8 * (r & 3);
            const uint32_t ws[4] = {buf[r].x, buf[r].y, buf[r].z, buf[r].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[cb + 2 * e] = __builtin_fmaf(pr, lo_h(ws[e]), o[cb + 2 * e]);
                o[cb + 2 * e + 1] = __builtin_fmaf(pr, hi_h(ws[e]), o[cb + 2 * e + 1]);
            }
        }
    };

    // ---- main loop: every phase's loads are issued one phase ahead of use,
    // into the other of two register buffers (across groups too)
    constexpr int NPH = n_phases<BITS>();
    uint4 bufA[NR], bufB[NR];
    const uint8_t* gp = group_ptr(g0);
    load_phase<BITS, D>(bufA, gp, 0, L);
    for (int gbase = g0; gbase < g1; gbase += GPI) {
        const bool valid = gbase + gslot < g1;
        const bool has_next = gbase + GPI < g1;
        const uint8_t* gn = has_next ? group_ptr(gbase + GPI) : gp;
        float acc[32];
#pragma unroll
        for (int ph = 0; ph < NPH; ++ph) {
            uint4* cur = (ph & 1) ? bufB : bufA;
            uint4* nxt = (ph & 1) ? bufA : bufB;
            // (on the last iteration gn == gp: the prefetch re-reads this
            // group, a cache hit, and keeps the code free of a branch whose
            // merge point would force the compiler to wait for every load)
            load_phase<BITS, D>(nxt, ph + 1 < NPH ? gp : gn, ph + 1 < NPH ? ph + 1 : 0, L);
            // keep the prefetch above this phase's arithmetic: the scheduler
            // would otherwise sink it below the wait for `cur`
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (BITS == 16) {
                if (ph < 4) keys_fp16(cur, acc + 8 * ph);
                else values_fp16(cur, 2 * (ph - 4));
                if (ph == 3) softmax_step(acc, valid);
            } else {
                if (ph == 0) {
                    keys_int(cur, acc);
                    softmax_step(acc, valid);
                } else {
                    values_int(cur);
                }
            }
        }
        gp = gn;
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

// Equal-byte split of one (sequence, KV head).  Its three segments, taken
// in the order FP16, INT4, INT2, form one byte range of `total` bytes that
// is cut into nw = ceil(total / per_wave) near-equal parts; part w covers
// bytes [w*total/nw, (w+1)*total/nw).  A group block belongs to the part
// that contains its first byte.  Every wavefront (and the combine) derives
// the same split from seg_count, so no schedule is stored.
struct Split {
    int segg[3];        // group blocks in each segment
    long long pre[3];   // first byte of each segment
    long long total;
    int nw;
};

template <int D>
__device__ __forceinline__ Split split_of(const AttnParams& p, int b) {
    Split sp;
    const int gpc = p.C / kGroup;
    sp.total = 0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        // chunks beyond a pool's capacity were never written: never read them
        sp.segg[k] = min(p.seg_count[b * 3 + k], p.cap[k]) * gpc;
        sp.pre[k] = sp.total;
        sp.total += (long long)sp.segg[k] * (long long)group_bytes(bits_of_expert(k), D);
    }
    sp.nw = (int)((sp.total + p.per_wave - 1) / p.per_wave);
    return sp;
}

// Group range [g0, g1) of segment k owned by part w.
template <int D>
__device__ __forceinline__ void part_groups(const Split& sp, int w, int k, int& g0, int& g1) {
    const long long gb = (long long)group_bytes(bits_of_expert(k), D);
    const long long o0 = (long long)w * sp.total / sp.nw - sp.pre[k];
    const long long o1 = (long long)(w + 1) * sp.total / sp.nw - sp.pre[k];
    long long a = o0 <= 0 ? 0 : (o0 + gb - 1) / gb;
    long long c = o1 <= 0 ? 0 : (o1 + gb - 1) / gb;
    g0 = (int)(a < sp.segg[k] ? a : sp.segg[k]);
    g1 = (int)(c < sp.segg[k] ? c : sp.segg[k]);
}

}  // namespace

// grid (nw_max, B*Hkv): wavefront (w, bh) streams part w of (b, h), one
// single-bitwidth piece per segment it overlaps, and writes one partial per
// piece at slot (w, k).
template <int D, int HB>
__global__ __launch_bounds__(64, 2) void attn_tile_kernel(AttnParams p) {
    const int w = blockIdx.x, bh = blockIdx.y;
    const int b = bh / p.Hkv;
    const Split sp = split_of<D>(p, b);
    if (w >= sp.nw) return;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        int g0, g1;
        part_groups<D>(sp, w, k, g0, g1);
        if (g0 >= g1) continue;
        const int slot = w * 3 + k;
        if (k == 0) tile_body<16, D, HB>(p, k, bh, slot, g0, g1);
        else if (k == 1) tile_body<4, D, HB>(p, k, bh, slot, g0, g1);
        else tile_body<2, D, HB>(p, k, bh, slot, g0, g1);
    }
}

// Merge the tile partials (and the fp16 tail) of one (sequence, KV head)
// into the outputs of its HB query heads.  256 threads: thread (tgi, qd)
// owns channel quad qd and walks tiles tgi, tgi + TGR, ...; every partial
// load is independent of the others.
template <int D, int HB>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p) {
    constexpr int QPR = D / 4;            // float4 quads per record
    constexpr int TGR = 256 / QPR;        // tile groups
    __shared__ float ts[4096];            // tail scores (log2 domain)
    __shared__ float red[256 * 4];
    __shared__ float lred[256];
    __shared__ float mred[8];
    const int bh = blockIdx.x;
    const int b = bh / p.Hkv, h = bh % p.Hkv;
    const int tid = threadIdx.x, qd = tid % QPR, tgi = tid / QPR;
    const Split sp = split_of<D>(p, b);
    // the pieces of this (b, h), in order: part w, segment k
    const int npiece = sp.nw * 3;
    auto piece_valid = [&](int v) {
        int g0, g1;
        part_groups<D>(sp, v / 3, v % 3, g0, g1);
        return g0 < g1;
    };
    auto rec_of = [&](int v, int hb) {
        return p.part + (((size_t)bh * p.nt_total + v) * HB + hb) * (D + 4);
    };
    for (int hb = 0; hb < HB; ++hb) {
        const int hq = h * HB + hb;
        // tail scores
        if (p.tail_len > 0) {
            const uint16_t* qp = p.q + ((size_t)b * p.Hq + hq) * D;
            const uint16_t* tk = p.tail_k + (size_t)bh * p.tail_len * D;
            for (int t = tid; t < p.tail_len; t += 256) {
                float s = 0.f;
                for (int c = 0; c < D; ++c)
                    s = __builtin_fmaf((float)__builtin_bit_cast(_Float16, qp[c]),
                                       (float)__builtin_bit_cast(_Float16, tk[(size_t)t * D + c]), s);
                ts[t] = s * p.qscale;
            }
        }
        // global max over tile maxima and tail scores
        float m = -INFINITY;
        for (int v = tid; v < npiece; v += 256)
            if (piece_valid(v)) m = fmaxf(m, rec_of(v, hb)[D]);
        for (int t = tid; t < p.tail_len; t += 256) m = fmaxf(m, ts[t]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        if ((tid & 63) == 0) mred[tid >> 6] = m;
        __syncthreads();
        const float M = fmaxf(fmaxf(mred[0], mred[1]), fmaxf(mred[2], mred[3]));
        // weighted sums
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        float lacc = 0.f;
        if (M != -INFINITY) {
            for (int v = tgi; v < npiece; v += TGR) {
                if (!piece_valid(v)) continue;
                const float* rec = rec_of(v, hb);
                const float2 ml = *reinterpret_cast<const float2*>(rec + D);
                const float4 o4 = *reinterpret_cast<const float4*>(rec + 4 * qd);
                const float w = fast_exp2(ml.x - M);
                acc.x = __builtin_fmaf(w, o4.x, acc.x);
                acc.y = __builtin_fmaf(w, o4.y, acc.y);
                acc.z = __builtin_fmaf(w, o4.z, acc.z);
                acc.w = __builtin_fmaf(w, o4.w, acc.w);
                lacc = __builtin_fmaf(w, ml.y, lacc);
            }
            const uint16_t* tv = p.tail_v + (size_t)bh * p.tail_len * D + 4 * qd;
            for (int t = tgi; t < p.tail_len; t += TGR) {
                const float w = fast_exp2(ts[t] - M);
                acc.x = __builtin_fmaf(w, (float)__builtin_bit_cast(_Float16, tv[(size_t)t * D + 0]), acc.x);
                acc.y = __builtin_fmaf(w, (float)__builtin_bit_cast(_Float16, tv[(size_t)t * D + 1]), acc.y);
                acc.z = __builtin_fmaf(w, (float)__builtin_bit_cast(_Float16, tv[(size_t)t * D + 2]), acc.z);
                acc.w = __builtin_fmaf(w, (float)__builtin_bit_cast(_Float16, tv[(size_t)t * D + 3]), acc.w);
                lacc += w;
            }
        }
        red[tid * 4 + 0] = acc.x;
        red[tid * 4 + 1] = acc.y;
        red[tid * 4 + 2] = acc.z;
        red[tid * 4 + 3] = acc.w;
        lred[tid] = lacc;
        __syncthreads();
        if (tid < QPR) {
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
            float l = 0.f;
            for (int gi = 0; gi < TGR; ++gi) {
                const int src = gi * QPR + tid;
                o.x += red[src * 4 + 0];
                o.y += red[src * 4 + 1];
                o.z += red[src * 4 + 2];
                o.w += red[src * 4 + 3];
                l += lred[gi * QPR];
            }
            const float inv = l > 0.f ? 1.f / l : 0.f;
            *reinterpret_cast<float4*>(p.out + ((size_t)b * p.Hq + hq) * D + 4 * tid) =
                make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
        }
        __syncthreads();
    }
}

hipError_t launch_attention(const AttnParams& ap, int D, int HB, hipStream_t st) {
    const dim3 grid(ap.nt_total / 3, ap.B * ap.Hkv);
    const dim3 cgrid(ap.B * ap.Hkv);
#define MKV_ATTN_CASE(DD, HH)                                                          \
    if (D == DD && HB == HH) {                                                         \
        if (ap.nt_total > 0) attn_tile_kernel<DD, HH><<<grid, 64, 0, st>>>(ap);        \
        attn_combine_kernel<DD, HH><<<cgrid, 256, 0, st>>>(ap);                        \
    } else
    MKV_ATTN_CASE(128, 1) MKV_ATTN_CASE(128, 2) MKV_ATTN_CASE(128, 4)
    MKV_ATTN_CASE(64, 1) MKV_ATTN_CASE(64, 2) MKV_ATTN_CASE(64, 4)
    return hipErrorInvalidValue;
#undef MKV_ATTN_CASE
    return hipGetLastError();
}

}  // namespace mkv
