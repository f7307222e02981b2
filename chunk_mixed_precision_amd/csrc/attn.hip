// Split-K decode attention over the mixed-bitwidth packed cache
// (MoQAE "Overall framework": ordinary attention after quantization;
// Cocktail abstract: chunk-level computation over bitwidth-contiguous
// segments, so every tile below has a single bitwidth and no wavefront ever
// branches on bitwidth inside its inner loop).
//
// Work: the packed bytes of each (sequence, KV head) (its FP16, INT4 and INT2
// segments in that order) are cut into equal-byte parts, one 64-lane
// wavefront per part; a part crossing a segment boundary is processed as one
// single-bitwidth piece per segment, each leaving one partial.  A wave is
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

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ float4 ldf4(const uint8_t* p) { return *reinterpret_cast<const float4*>(p); }

__device__ __forceinline__ float4 as_f4(const uint4& u) { return __builtin_bit_cast(float4, u); }

// Every load phase brings in 8 rows of a group block (8 x 16 B per lane).
// INT4: 3 phases: rows 0-7 = key meta + key codes of tokens 0-15, rows 8-15 =
//       key codes of tokens 16-31 + value meta, rows 16-23 = value codes.
// INT2: 2 phases: key meta + key codes, value meta + value codes.
// FP16: 8 phases: key rows 0-31, then value rows 0-31.
template <int BITS> __host__ __device__ constexpr int n_phases() { return BITS == 16 ? 8 : (BITS == 4 ? 3 : 2); }

template <int D>
__device__ __forceinline__ void load_rows8(uint4* buf, const uint8_t* gp, int phase, int L) {
    constexpr size_t ROWB = (size_t)(D / 8) * 16;
    const uint8_t* src = gp + (size_t)phase * 8 * ROWB + L * 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) buf[i] = ld16(src + i * ROWB);
}

// Reduce-scatter of one half (16 per-token partial sums) over the S lanes of
// a row.  On return acc[0 .. 16/S-1] hold the full sums of tokens
// (tok_xor(S, L) ^ i) of that half.
template <int S>
__device__ __forceinline__ void reduce_half(float* acc) {
    if constexpr (S == 16) {
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] += dpp<kDppRowMirror>(acc[r + 8]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += dpp<kDppRowHalfMirror>(acc[r + 4]);
#pragma unroll
        for (int r = 0; r < 2; ++r) acc[r] += dpp<kDppXor2>(acc[r + 2]);
        acc[0] += dpp<kDppXor1>(acc[1]);
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] += dpp<kDppRowHalfMirror>(acc[r + 8]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += dpp<kDppXor2>(acc[r + 4]);
#pragma unroll
        for (int r = 0; r < 2; ++r) acc[r] += dpp<kDppXor1>(acc[r + 2]);
    }
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
__device__ __forceinline__ void tile_body(const AttnParams& p, int k, int bh, int slot, int g0, int g1) {
    constexpr int S = D / 8;
    constexpr int R = 64 / S;          // rows per wave
    constexpr int NG = D / 32;         // value groups per token
    constexpr int GPI = R / HB;        // group blocks per iteration
    constexpr int NTH = 16 / S;        // tokens per lane and key half after the reduce-scatter
    constexpr int NPH = n_phases<BITS>();
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
    const half2_t qh0 = as_h2(qw[0]), qh1 = as_h2(qw[1]), qh2 = as_h2(qw[2]), qh3 = as_h2(qw[3]);

    float M = -INFINITY;   // running max of this row (log2 domain), row-uniform
    float lsum = 0.f;      // this lane's share of the softmax denominator
    float o[32];           // channels 32G .. 32G+31
    float pm = 0.f;        // sum_t p_t * mn_t over this lane's value tokens
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] = 0.f;

    float sc[2 * NTH];     // this lane's key scores: half 0, then half 1
    float pw[8];           // value weights of tokens tq + 4m (p * scale for INT-b)
    float qp[8];           // q_j * s_j (INT-b), this group
    float bias = 0.f;      // sum_j q_j * mn_j over this lane's channels (INT-b)
    float acc[16];

    auto group_ptr = [&](int gbase) {
        const int gi = gbase + gslot;
        return seg + (size_t)(gi < g1 ? gi : g1 - 1) * GB;
    };

    // ---- online-softmax update from sc[], probabilities to the value layout
    auto softmax_step = [&](bool valid) {
        float mloc = -INFINITY;
#pragma unroll
        for (int i = 0; i < 2 * NTH; ++i) {
            if (!valid) sc[i] = -INFINITY;
            mloc = fmaxf(mloc, sc[i]);
        }
        mloc = row_max<S>(mloc);
        const float Mn = fmaxf(M, mloc);
        const float alpha = (Mn == -INFINITY) ? 1.f : fast_exp2(M - Mn);
        M = Mn;
        float pt[2 * NTH];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 2 * NTH; ++i) {
            pt[i] = valid ? fast_exp2(sc[i] - Mn) : 0.f;
            psum += pt[i];
        }
        lsum = __builtin_fmaf(lsum, alpha, psum);
        pm *= alpha;
#pragma unroll
        for (int c = 0; c < 32; ++c) o[c] *= alpha;
        // slot of token t in the value layout: (t & 3) * 8 + (t >> 2)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < NTH; ++i) {
                const int t = 16 * hh + (fx ^ i);
                plds[row][(t & 3) * 8 + (t >> 2)] = pt[hh * NTH + i];
            }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const float4 pa = *reinterpret_cast<const float4*>(&plds[row][tq * 8]);
        const float4 pb = *reinterpret_cast<const float4*>(&plds[row][tq * 8 + 4]);
        pw[0] = pa.x; pw[1] = pa.y; pw[2] = pa.z; pw[3] = pa.w;
        pw[4] = pb.x; pw[5] = pb.y; pw[6] = pb.z; pw[7] = pb.w;
    };

    // ---- INT-b pieces
    auto key_meta = [&](const uint4* m4) {           // rows: scale lo, scale hi, min lo, min hi
        const float4 s0 = as_f4(m4[0]), s1 = as_f4(m4[1]), n0 = as_f4(m4[2]), n1 = as_f4(m4[3]);
        const float ks[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const float kmn[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
        bias = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bias = __builtin_fmaf(qs[e], kmn[e], bias);
            qp[e] = qs[e] * ks[e];
        }
    };
    auto key_half_int4 = [&](const uint4* rows) {    // 4 key-code rows of one half
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = bias;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int w = i >> 1;
            const uint32_t ws[4] = {rows[i].x, rows[i].y, rows[i].z, rows[i].w};
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
    };
    auto key_half_int2 = [&](const uint4* rows) {    // 2 key-code rows of one half
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = bias;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t ws[4] = {rows[i].x, rows[i].y, rows[i].z, rows[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float q0 = qp[4 * i + e];
                const float qm[4] = {q0, q0 * 0.25f, q0 * 0.0625f, q0 * 0.015625f};
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    const uint32_t part = ws[e] & (0x03030303u << (2 * mm));
                    acc[0 + mm] = __builtin_fmaf(qm[mm], cvt_ub<0>(part), acc[0 + mm]);
                    acc[4 + mm] = __builtin_fmaf(qm[mm], cvt_ub<1>(part), acc[4 + mm]);
                    acc[8 + mm] = __builtin_fmaf(qm[mm], cvt_ub<2>(part), acc[8 + mm]);
                    acc[12 + mm] = __builtin_fmaf(qm[mm], cvt_ub<3>(part), acc[12 + mm]);
                }
            }
        }
    };
    auto take_half = [&](int hh) {
        reduce_half<S>(acc);
#pragma unroll
        for (int i = 0; i < NTH; ++i) sc[hh * NTH + i] = acc[i];
    };
    auto value_meta = [&](const uint4* m4) {         // (scale, min) of tokens t_{2r}, t_{2r+1}
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float4 sm = as_f4(m4[m >> 1]);
            const float s = (m & 1) ? sm.z : sm.x;
            const float mn = (m & 1) ? sm.w : sm.y;
            pm = __builtin_fmaf(pw[m], mn, pm);
            pw[m] *= s;
        }
    };
    auto values_int4 = [&](const uint4* rows) {      // row m: token tq + 4m
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint32_t ws[4] = {rows[m].x, rows[m].y, rows[m].z, rows[m].w};
            const float pv = pw[m], pb16 = pv * 0.0625f;
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
        }
    };
    auto values_int2 = [&](const uint4* rows) {      // row r: tokens t_{2r} (dwords 0,1), t_{2r+1} (2,3)
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint4 c = rows[m >> 1];
            const uint32_t ws[2] = {(m & 1) ? c.z : c.x, (m & 1) ? c.w : c.y};
            const float pv = pw[m];
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
    };

    // ---- FP16 pieces: 8 key rows (q . k with v_dot2) or 8 value rows
    auto keys_fp16 = [&](const uint4* rows, int r0) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            float a = __builtin_amdgcn_fdot2(as_h2(rows[r].x), qh0, 0.f, false);
            a = __builtin_amdgcn_fdot2(as_h2(rows[r].y), qh1, a, false);
            a = __builtin_amdgcn_fdot2(as_h2(rows[r].z), qh2, a, false);
            a = __builtin_amdgcn_fdot2(as_h2(rows[r].w), qh3, a, false);
            acc[r0 + r] = a;
        }
    };
    auto values_fp16 = [&](const uint4* rows, int mbase) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float pr = pw[mbase + (r >> 2)];
            const int cb = 8 * (r & 3);
            const uint32_t ws[4] = {rows[r].x, rows[r].y, rows[r].z, rows[r].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[cb + 2 * e] = __builtin_fmaf(pr, lo_h(ws[e]), o[cb + 2 * e]);
                o[cb + 2 * e + 1] = __builtin_fmaf(pr, hi_h(ws[e]), o[cb + 2 * e + 1]);
            }
        }
    };

    // one phase's arithmetic on the rows in `cur`
    auto compute_phase = [&](int ph, const uint4* cur, bool valid) {
        if constexpr (BITS == 4) {
            if (ph == 0) {
                key_meta(cur);
                key_half_int4(cur + 4);
                take_half(0);
            } else if (ph == 1) {
                key_half_int4(cur);
                take_half(1);
                softmax_step(valid);
                value_meta(cur + 4);
            } else {
                values_int4(cur);
            }
        } else if constexpr (BITS == 2) {
            if (ph == 0) {
                key_meta(cur);
                key_half_int2(cur + 4);
                take_half(0);
                key_half_int2(cur + 6);
                take_half(1);
                softmax_step(valid);
            } else {
                value_meta(cur);
                values_int2(cur + 4);
            }
        } else {
            if (ph < 4) {
                keys_fp16(cur, 8 * (ph & 1));
                if (ph & 1) {
                    take_half(ph >> 1);
                    if (ph == 3) {
#pragma unroll
                        for (int i = 0; i < 2 * NTH; ++i) sc[i] *= p.qscale;
                        softmax_step(valid);
                    }
                }
            } else {
                values_fp16(cur, 2 * (ph - 4));
            }
        }
    };

    // ---- main loop.  Every phase's loads are issued one phase ahead, into
    // the other of two 8-row register buffers; the last phase of a group
    // prefetches the next group's first phase (or, at the end, re-reads this
    // group: a cache hit that keeps the loop free of a branch whose merge
    // point would make the compiler wait for every outstanding load).
    uint4 bufA[8], bufB[8];
    auto run_group = [&](auto par_tag, int gbase, const uint8_t* gp, const uint8_t* gn) {
        constexpr int PAR = decltype(par_tag)::value;
        const bool valid = gbase + gslot < g1;
#pragma unroll
        for (int ph = 0; ph < NPH; ++ph) {
            uint4* cur = ((ph + PAR) & 1) ? bufB : bufA;
            uint4* nxt = ((ph + PAR) & 1) ? bufA : bufB;
            load_rows8<D>(nxt, ph + 1 < NPH ? gp : gn, ph + 1 < NPH ? ph + 1 : 0, L);
            __builtin_amdgcn_sched_barrier(0);
            compute_phase(ph, cur, valid);
        }
    };
    const uint8_t* gp = group_ptr(g0);
    load_rows8<D>(bufA, gp, 0, L);
    if constexpr (NPH % 2 == 0) {
        for (int gbase = g0; gbase < g1; gbase += GPI) {
            const uint8_t* gn = gbase + GPI < g1 ? group_ptr(gbase + GPI) : gp;
            run_group(std::integral_constant<int, 0>{}, gbase, gp, gn);
            gp = gn;
        }
    } else {
        // odd phase count: buffer parity flips every group, so groups go in pairs
        for (int gbase = g0; gbase < g1; gbase += 2 * GPI) {
            const uint8_t* gn = gbase + GPI < g1 ? group_ptr(gbase + GPI) : gp;
            run_group(std::integral_constant<int, 0>{}, gbase, gp, gn);
            if (gbase + GPI < g1) {
                const uint8_t* gn2 = gbase + 2 * GPI < g1 ? group_ptr(gbase + 2 * GPI) : gn;
                run_group(std::integral_constant<int, 1>{}, gbase + GPI, gn, gn2);
                gp = gn2;
            } else {
                gp = gn;
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
    const float rs = (M == -INFINITY) ? 0.f : fast_exp2(M - Mx);
    lsum *= rs;
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] *= rs;
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
        float* rec = p.part + (((size_t)bh * p.nt_total + slot) * HB + hb) * (D + 4);
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
__global__ __launch_bounds__(64, 3) void attn_tile_kernel(AttnParams p) {
    const int w = blockIdx.x, bh = blockIdx.y;
    const int b = bh / p.Hkv;
    const Split sp = split_of<D>(p, b);
    if (w >= sp.nw) return;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        int g0, g1;
        part_groups<D>(sp, w, k, g0, g1);
        const int slot = w * 3 + k;
        if (g0 >= g1) {
            // empty piece: mark it so the combine skips it
            if (threadIdx.x < HB) {
                float* rec = p.part + (((size_t)bh * p.nt_total + slot) * HB + threadIdx.x) * (D + 4);
                *reinterpret_cast<float4*>(rec + D) = make_float4(-INFINITY, 0.f, 0.f, 0.f);
            }
            continue;
        }
        if (k == 0) tile_body<16, D, HB>(p, k, bh, slot, g0, g1);
        else if (k == 1) tile_body<4, D, HB>(p, k, bh, slot, g0, g1);
        else tile_body<2, D, HB>(p, k, bh, slot, g0, g1);
    }
}

// Merge the piece partials (and the fp16 tail) of one (sequence, KV head)
// into the outputs of its HB query heads.  512 threads: thread (tgi, qd)
// owns channel quad qd and merges pieces tgi, tgi + TGR, ... online, with
// its loads batched so that they are in flight together; a piece without
// group blocks carries m = -inf and is skipped.
template <int D, int HB>
__global__ __launch_bounds__(512) void attn_combine_kernel(AttnParams p) {
    constexpr int NT = 512;
    constexpr int QPR = D / 4;            // float4 quads per record
    constexpr int TGR = NT / QPR;         // piece groups
    constexpr int BATCH = 4;
    __shared__ float ts[4096];            // tail scores (log2 domain)
    __shared__ float4 red_o[NT];
    __shared__ float2 red_ml[NT];
    const int bh = blockIdx.x;
    const int b = bh / p.Hkv, h = bh % p.Hkv;
    const int tid = threadIdx.x, qd = tid % QPR, tgi = tid / QPR;
    const int npiece = split_of<D>(p, b).nw * 3;
    auto rec_of = [&](int v, int hb) {
        return p.part + (((size_t)bh * p.nt_total + v) * HB + hb) * (D + 4);
    };
    for (int hb = 0; hb < HB; ++hb) {
        const int hq = h * HB + hb;
        if (p.tail_len > 0) {
            const uint16_t* qp = p.q + ((size_t)b * p.Hq + hq) * D;
            const uint16_t* tk = p.tail_k + (size_t)bh * p.tail_len * D;
            for (int t = tid; t < p.tail_len; t += NT) {
                float s = 0.f;
                for (int c = 0; c < D; ++c)
                    s = __builtin_fmaf((float)__builtin_bit_cast(_Float16, qp[c]),
                                       (float)__builtin_bit_cast(_Float16, tk[(size_t)t * D + c]), s);
                ts[t] = s * p.qscale;
            }
            __syncthreads();
        }
        float m = -INFINITY, l = 0.f;
        float o[4] = {0.f, 0.f, 0.f, 0.f};
        for (int v0 = tgi; v0 < npiece; v0 += TGR * BATCH) {
            float2 ml[BATCH];
            float4 ov[BATCH];
#pragma unroll
            for (int j = 0; j < BATCH; ++j) {
                const int v = v0 + j * TGR;
                const float* rec = rec_of(v < npiece ? v : v0, hb);
                ml[j] = *reinterpret_cast<const float2*>(rec + D);
                ov[j] = *reinterpret_cast<const float4*>(rec + 4 * qd);
                if (v >= npiece) ml[j].x = -INFINITY;
            }
#pragma unroll
            for (int j = 0; j < BATCH; ++j) {
                if (ml[j].x == -INFINITY) continue;
                const float o2[4] = {ov[j].x, ov[j].y, ov[j].z, ov[j].w};
                merge_run<4>(m, l, o, ml[j].x, ml[j].y, o2);
            }
        }
        if (p.tail_len > 0) {
            const uint16_t* tv = p.tail_v + (size_t)bh * p.tail_len * D + 4 * qd;
            for (int t = tgi; t < p.tail_len; t += TGR) {
                float vf[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) vf[c] = (float)__builtin_bit_cast(_Float16, tv[(size_t)t * D + c]);
                merge_run<4>(m, l, o, ts[t], 1.f, vf);
            }
        }
        red_o[tid] = make_float4(o[0], o[1], o[2], o[3]);
        red_ml[tid] = make_float2(m, l);
        __syncthreads();
        if (tid < QPR) {
            float mm = -INFINITY, ll = 0.f;
            float oo[4] = {0.f, 0.f, 0.f, 0.f};
            for (int gi = 0; gi < TGR; ++gi) {
                const float4 x = red_o[gi * QPR + tid];
                const float2 y = red_ml[gi * QPR + tid];
                const float o2[4] = {x.x, x.y, x.z, x.w};
                merge_run<4>(mm, ll, oo, y.x, y.y, o2);
            }
            const float inv = ll > 0.f ? 1.f / ll : 0.f;
            *reinterpret_cast<float4*>(p.out + ((size_t)b * p.Hq + hq) * D + 4 * tid) =
                make_float4(oo[0] * inv, oo[1] * inv, oo[2] * inv, oo[3] * inv);
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
        attn_combine_kernel<DD, HH><<<cgrid, 512, 0, st>>>(ap);                        \
    } else
    MKV_ATTN_CASE(128, 1) MKV_ATTN_CASE(128, 2) MKV_ATTN_CASE(128, 4)
    MKV_ATTN_CASE(64, 1) MKV_ATTN_CASE(64, 2) MKV_ATTN_CASE(64, 4)
    return hipErrorInvalidValue;
#undef MKV_ATTN_CASE
    return hipGetLastError();
}

}  // namespace mkv
