// Router, chunk vote, routing freezing and reorder (MoQAE "Key designs":
// Quantization-Aware Experts, routing freezing, routing sharing; Cocktail
// abstract: chunks reordered by bitwidth before quantization).
//
// Router: z = SiLU((x W1^T) .* (x W2^T)) W3^T + b3.  The two projections are
// one bf16 GEMM on the MFMA units ([M x D] . [D x 2I], fp32 accumulation).
// A workgroup owns 128 tokens x 64 inner indices: it computes both h1 and h2
// for those indices (W1 rows and the matching W2 rows share the tile), so the
// gate and the W3 projection run in the epilogue and only 3 partial logits
// per (token, 64-wide inner slice) reach memory.  The vote kernel sums the
// slices in a fixed order, adds b3 and takes the argmax: results are
// deterministic run to run.
#include "mkv_internal.h"
#include "mkv_kernels.h"

namespace mkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = kRouterBM;          // 128 tokens
constexpr int BI = kRouterBI;          // 64 inner indices -> 128 W12 rows
constexpr int BN = 2 * BI;
constexpr int BK = kRouterBK;          // 32
constexpr int LDK = BK + 8;            // padded LDS row (bf16 elements)

}  // namespace

// 256 threads = 4 waves as 2 (tokens) x 2 (inner).  Wave (wm, wn) computes
// tokens wm*64 .. +63 against W1 rows and W2 rows of inner indices
// wn*32 .. +31 with 2 x 2 MFMA 32x32x16 blocks.
__global__ __launch_bounds__(256) void router_gemm_kernel(RouterParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (BM + BN) * LDK];
    constexpr int STAGE = (BM + BN) * LDK;   // one stage: A tile then B tile

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int m0 = blockIdx.x * BM;
    const int i0 = blockIdx.y * BI;
    const int D = p.D;

    // global -> LDS staging: each thread moves 2 x 16 B of A and 2 x 16 B of B per stage
    int a_row[2], a_col[2], b_row[2];
    const uint16_t* a_src[2];
    const uint16_t* b_src[2];
    bool a_ok[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = tid + 256 * q;
        a_row[q] = idx >> 2;
        a_col[q] = (idx & 3) * 8;
        a_ok[q] = (m0 + a_row[q]) < p.M;
        a_src[q] = p.x + (size_t)(a_ok[q] ? m0 + a_row[q] : 0) * D + a_col[q];
        b_row[q] = idx >> 2;
        const int wrow = b_row[q] < BI ? i0 + b_row[q] : p.I + i0 + (b_row[q] - BI);
        b_src[q] = p.w12 + (size_t)wrow * D + a_col[q];
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;

    uint4 ra[2], rb[2];
    auto gload = [&](int k0) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            ra[q] = a_ok[q] ? *reinterpret_cast<const uint4*>(a_src[q] + k0) : make_uint4(0, 0, 0, 0);
            rb[q] = *reinterpret_cast<const uint4*>(b_src[q] + k0);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            *reinterpret_cast<uint4*>(lds + buf * STAGE + a_row[q] * LDK + a_col[q]) = ra[q];
            *reinterpret_cast<uint4*>(lds + buf * STAGE + BM * LDK + b_row[q] * LDK + a_col[q]) = rb[q];
        }
    };

    const int nk = D / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int lr = lane & 31, lk = (lane >> 5) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const uint16_t* As = lds + cur * STAGE;
        const uint16_t* Bs = As + BM * LDK;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                af[mb] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + mb * 32 + lr) * LDK + ks * 16 + lk);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                bfr[nb] = *reinterpret_cast<const bf16x8*>(Bs + (nb * BI + wn * 32 + lr) * LDK + ks * 16 + lk);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            sstore(cur ^ 1);
        }
        __syncthreads();
    }

    // ---------------- epilogue: gate, then this slice's share of W3
    float* a_lds = reinterpret_cast<float*>(lds);     // [BM][BI + 1]
    constexpr int LDA = BI + 1;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tok = wm * 64 + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int ii = wn * 32 + lr;
            const float u = acc[mb][0][r] * acc[mb][1][r];
            const float a = u / (1.0f + expf(-u));
            a_lds[tok * LDA + ii] = a;
        }
    __syncthreads();
    {
        const int tok = tid >> 1, half = tid & 1;
        const float* arow = a_lds + tok * LDA + half * 32;
        const float* w3 = p.w3 + i0 + half * 32;
        float z0 = 0.f, z1 = 0.f, z2 = 0.f;
        for (int i = 0; i < 32; ++i) {
            const float a = arow[i];
            z0 = __builtin_fmaf(a, w3[i], z0);
            z1 = __builtin_fmaf(a, w3[p.I + i], z1);
            z2 = __builtin_fmaf(a, w3[2 * p.I + i], z2);
        }
        // fixed order: lower half + upper half on both lanes of the pair
        const float y0 = __shfl_xor(z0, 1), y1 = __shfl_xor(z1, 1), y2 = __shfl_xor(z2, 1);
        if (half == 0 && m0 + tok < p.M) {
            float* zp = p.zpart + ((size_t)blockIdx.y * p.M + m0 + tok) * 3;
            zp[0] = z0 + y0;
            zp[1] = z1 + y1;
            zp[2] = z2 + y2;
        }
    }
}

// One block of 256 threads per (new chunk, sequence).
__global__ __launch_bounds__(256) void vote_kernel(VoteParams p) {
    __shared__ int cnt[3];
    const int c = blockIdx.x, b = blockIdx.y;
    if (threadIdx.x < 3) cnt[threadIdx.x] = 0;
    __syncthreads();
    const int M = p.B * p.T;
    for (int t = threadIdx.x; t < p.C; t += blockDim.x) {
        const size_t row = (size_t)b * p.T + (size_t)c * p.C + t;
        float z[3];
        if (p.zpart) {
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                float s = 0.f;
                for (int tile = 0; tile < p.ntile; ++tile) s += p.zpart[((size_t)tile * M + row) * 3 + k];
                z[k] = s + p.b3[k];
            }
            if (p.logits_out) {
#pragma unroll
                for (int k = 0; k < 3; ++k) p.logits_out[row * 3 + k] = z[k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < 3; ++k) z[k] = p.logits_in[row * 3 + k];
        }
        int e = 0;
        float best = z[0];
        if (z[1] > best) { e = 1; best = z[1]; }
        if (z[2] > best) { e = 2; }
        if (p.token_expert) p.token_expert[row] = (uint8_t)e;
        atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int v = 0;
        if (cnt[1] > cnt[v]) v = 1;
        if (cnt[2] > cnt[v]) v = 2;
        const int chunk = p.chunk_offset + c;
        if (p.freeze_first && chunk == 0) v = 0;
        p.chunk_bits[(size_t)b * p.n_max + chunk] = (uint8_t)bits_of_expert(v);
    }
}

// One block of 256 threads per sequence: stable partition of chunks
// [0, n_total) into the FP16, INT4, INT2 segments.
__global__ __launch_bounds__(256) void reorder_kernel(ReorderParams p) {
    __shared__ int pre[3][257];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int n = p.n_total;
    const int per = (n + 255) / 256;
    const int c0 = min(tid * per, n), c1 = min(c0 + per, n);
    const uint8_t* bits = p.chunk_bits + (size_t)b * p.n_max;
    int local[3] = {0, 0, 0};
    for (int c = c0; c < c1; ++c) {
        int k = expert_of_bits(bits[c]);
        if (k < 0) {
            if (p.bad) p.bad[0] = 1;
            k = 2;
        }
        ++local[k];
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) pre[k][tid + 1] = local[k];
    if (tid == 0) {
        pre[0][0] = pre[1][0] = pre[2][0] = 0;
    }
    __syncthreads();
    if (tid < 3) {
        for (int i = 1; i <= 256; ++i) pre[tid][i] += pre[tid][i - 1];
    }
    __syncthreads();
    const int tot0 = pre[0][256], tot1 = pre[1][256], tot2 = pre[2][256];
    if (tid == 0) {
        p.seg_count[b * 3 + 0] = tot0;
        p.seg_count[b * 3 + 1] = tot1;
        p.seg_count[b * 3 + 2] = tot2;
    }
    const int start[3] = {0, tot0, tot0 + tot1};
    int run[3] = {pre[0][tid], pre[1][tid], pre[2][tid]};
    for (int c = c0; c < c1; ++c) {
        int k = expert_of_bits(bits[c]);
        if (k < 0) k = 2;
        const int r = run[k]++;
        p.chunk_rank[(size_t)b * p.n_max + c] = r;
        p.perm[(size_t)b * p.n_max + start[k] + r] = c;
    }
}

hipError_t launch_router(const RouterParams& rp, hipStream_t st) {
    const dim3 grid((rp.M + BM - 1) / BM, rp.I / BI);
    router_gemm_kernel<<<grid, 256, 0, st>>>(rp);
    return hipGetLastError();
}

hipError_t launch_vote(const VoteParams& vp, int n_new, hipStream_t st) {
    vote_kernel<<<dim3(n_new, vp.B), 256, 0, st>>>(vp);
    return hipGetLastError();
}

hipError_t launch_reorder(const ReorderParams& rp, int B, hipStream_t st) {
    reorder_kernel<<<dim3(B), 256, 0, st>>>(rp);
    return hipGetLastError();
}

}  // namespace mkv
