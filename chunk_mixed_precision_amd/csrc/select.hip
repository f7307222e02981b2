// Similarity-based chunk selection (Cocktail abstract: chunk-level
// quantization search picks each chunk's bitwidth from the similarity
// between the chunk and the query).  A chunk is summarised by the sum of its
// tokens' embeddings -- the direction of their mean -- and scored by its
// cosine with the query embedding; two thresholds map the score to FP16,
// INT4 or INT2.  The work is one streaming read of the embeddings (HBM
// bound).  The thresholds are applied by the reorder kernel's first step,
// which then reorders the chunks exactly as after routing.
#include "mkv_internal.h"
#include "mkv_kernels.h"

namespace mkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

// bf16 -> float32 is exact: the bf16 bits are the high half of the float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace

// One workgroup of 4 wavefronts per (512-dim slice, new chunk, sequence).
// Lane l holds dims 8l..8l+7 of the slice; wavefront w sums tokens w, w+4,
// ... of the chunk with two 16-byte loads in flight per lane (four or more
// made the whole read slower on this part).  The four wavefronts' sums meet
// in LDS (added in wavefront order), and wavefront 0 reduces q.S, |S|^2 and
// |q|^2 over the slice.
__global__ __launch_bounds__(256) void sim_partial_kernel(SimParams p) {
    __shared__ float4 red[4][2][64];
    const int slice = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d0 = slice * kSimSlice + lane * 8;
    const bool act = d0 < p.D;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (act) {
        const uint16_t* xr = p.x + ((size_t)b * p.T + (size_t)c * p.C) * p.D + d0;
        for (int t = wave; t < p.C; t += 8) {
            uint4 u[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int tt = t + 4 * j;
                u[j] = make_uint4(0, 0, 0, 0);
                if (tt < p.C) {   // read once: nontemporal
                    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + (size_t)tt * p.D));
                    u[j] = make_uint4(x.x, x.y, x.z, x.w);
                }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t w4[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] += bf16_lo(w4[e]);
                    acc[2 * e + 1] += bf16_hi(w4[e]);
                }
            }
        }
    }
    red[wave][0][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    red[wave][1][lane] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    __syncthreads();
    if (wave != 0) return;
    float dot = 0.f, ss = 0.f, qq = 0.f;
    if (act) {
        const uint4 qu = *reinterpret_cast<const uint4*>(p.qe + (size_t)b * p.D + d0);
        const uint32_t qw[4] = {qu.x, qu.y, qu.z, qu.w};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float4 r0 = red[0][h][lane], r1 = red[1][h][lane], r2 = red[2][h][lane], r3 = red[3][h][lane];
            const float sv[4] = {((r0.x + r1.x) + r2.x) + r3.x, ((r0.y + r1.y) + r2.y) + r3.y,
                                 ((r0.z + r1.z) + r2.z) + r3.z, ((r0.w + r1.w) + r2.w) + r3.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = 4 * h + e;
                const float q = (k & 1) ? bf16_hi(qw[k >> 1]) : bf16_lo(qw[k >> 1]);
                dot = __builtin_fmaf(sv[e], q, dot);
                ss = __builtin_fmaf(sv[e], sv[e], ss);
                qq = __builtin_fmaf(q, q, qq);
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        dot += __shfl_xor(dot, off);
        ss += __shfl_xor(ss, off);
        qq += __shfl_xor(qq, off);
    }
    if (lane == 0) {
        const int n_new = p.T / p.C;
        p.part[((size_t)b * n_new + c) * p.ds + slice] = make_float4(dot, ss, qq, 0.f);
    }
}

hipError_t launch_similarity(const SimParams& sp, hipStream_t st) {
    const int n_new = sp.T / sp.C;
    sim_partial_kernel<<<dim3(sp.ds, n_new, sp.B), 256, 0, st>>>(sp);
    return hipGetLastError();
}

}  // namespace mkv
