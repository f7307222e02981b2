// Router, chunk vote, routing freezing and reorder (MoQAE "Key designs":
// Quantization-Aware Experts, routing freezing, routing sharing; Cocktail
// abstract: chunks reordered by bitwidth before quantization).
//
// Router: z = SiLU((x W1^T) .* (x W2^T)) W3^T + b3.  The two projections are
// one bf16 GEMM on the MFMA units ([M x D] . [D x 2I], fp32 accumulation).
// A workgroup owns 256 tokens x 128 inner indices: it computes both h1 and h2
// for those indices (W1 rows and the matching W2 rows share the tile), so the
// gate and the W3 projection run in the epilogue and only 3 partial logits
// per (token, 128-wide inner slice) reach memory.  The vote kernel sums the
// slices in a fixed order, adds b3 and takes the argmax: results are
// deterministic run to run.
#include "mkv_internal.h"
#include "mkv_kernels.h"

namespace mkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glob_void;

constexpr int BM = kRouterBM;          // 256 tokens
constexpr int BI = kRouterBI;          // 128 inner indices -> 256 W12 rows
constexpr int BN = 2 * BI;
constexpr int BK = kRouterBK;          // 32 bf16 = 64 B per row and stage
constexpr int ROWB = BK * 2;           // bytes per tile row in LDS
constexpr int STAGE = (BM + BN) * ROWB;   // A tile then B tile
constexpr int LDA = BM / 2 + 1;        // epilogue: a[inner][128 tokens], padded row
constexpr int LDS_BYTES = (2 * STAGE > BI * LDA * 4) ? 2 * STAGE : BI * LDA * 4;

// 16-byte chunk c of tile row r sits at chunk c ^ ((r >> 1) & 3) of its
// 64-byte LDS row: the eight rows read by one MFMA operand load then fall on
// distinct bank groups.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 3); }

}  // namespace

// Router GEMM with the gate and the W3 projection fused in the epilogue.
// Workgroup tile: 256 tokens x 128 inner indices (W1 and W2 rows of those
// indices), K staged 32 at a time through two LDS buffers filled by
// direct global->LDS loads.  256 threads = 4 waves as 2 (tokens) x 2 (inner);
// wave (wm, wn) owns tokens wm*128..+127 and inner wn*64..+63: 4 x 4 MFMA
// 32x32x16 bf16 blocks (two W1 and two W2 column blocks).  Tiles are ordered
// so that the eight inner tiles of a token tile run on one XCD and share its
// L2.
__global__ __launch_bounds__(256, 1) void router_gemm_kernel(RouterParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int NT = p.I / BI;
    const int MT = (p.M + BM - 1) / BM;
    // XCD-aware order: workgroup id -> (token tile, inner tile)
    const int id = blockIdx.x;
    const int xcd = id & 7, local = id >> 3;
    const int mt = (local / NT) * 8 + xcd, nt = local % NT;
    if (mt >= MT) return;
    const int m0 = mt * BM, i0 = nt * BI;
    const int D = p.D;

    // this lane's source rows for its 4 + 4 direct loads per stage: load j of
    // wave w fills LDS bytes [(4w + j) KB, +1 KB) of the A (or B) region
    const uint16_t* a_src[4];
    const uint16_t* b_src[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = (wave * 4 + j) * 16 + (lane >> 2);     // tile row
        const int c = swz(r, lane & 3);                      // logical chunk held by this slot
        const int xr = min(m0 + r, p.M - 1);                 // rows past M read a valid row
        a_src[j] = p.x + (size_t)xr * D + c * 8;
        const int wr = r < BI ? i0 + r : p.I + i0 + (r - BI);
        b_src[j] = p.w12 + (size_t)wr * D + c * 8;
    }
    auto stage_load = [&](int buf, int k0) {
        uint8_t* base = lds + buf * STAGE;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            __builtin_amdgcn_global_load_lds((glob_void*)(a_src[j] + k0),
                                             (lds_void*)(base + (wave * 4 + j) * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((glob_void*)(b_src[j] + k0),
                                             (lds_void*)(base + BM * ROWB + (wave * 4 + j) * 1024), 16, 0, 0);
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;

    const int lr = lane & 31, lh = lane >> 5;
    const int nk = D / BK;
    stage_load(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) stage_load(cur ^ 1, (kt + 1) * BK);
        const uint8_t* As = lds + cur * STAGE;
        const uint8_t* Bs = As + BM * ROWB;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int c = 2 * ks + lh;
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int r = wm * 128 + mb * 32 + lr;
                af[mb] = *reinterpret_cast<const bf16x8*>(As + r * ROWB + swz(r, c) * 16);
            }
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int r = (nb < 2 ? 0 : BI) + wn * 64 + (nb & 1) * 32 + lr;
                bfr[nb] = *reinterpret_cast<const bf16x8*>(Bs + r * ROWB + swz(r, c) * 16);
            }
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---------------- epilogue: a = SiLU(h1 * h2), then this tile's share of
    // z = a W3^T, in two rounds of 128 tokens through LDS as a[inner][token]
    float* a_lds = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int round = 0; round < 2; ++round) {
        if (wm == round) {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int tok = mb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                        const int ii = wn * 64 + nb * 32 + lr;
                        const float u = acc[mb][nb][r] * acc[mb][nb + 2][r];
                        a_lds[ii * LDA + tok] = u / (1.0f + expf(-u));
                    }
        }
        __syncthreads();
        {
            const int tok = tid >> 1, half = tid & 1;
            const float* w3 = p.w3 + i0 + half * 64;
            float z0 = 0.f, z1 = 0.f, z2 = 0.f;
            for (int i = 0; i < 64; ++i) {
                const float a = a_lds[(half * 64 + i) * LDA + tok];
                z0 = __builtin_fmaf(a, w3[i], z0);
                z1 = __builtin_fmaf(a, w3[p.I + i], z1);
                z2 = __builtin_fmaf(a, w3[2 * p.I + i], z2);
            }
            // fixed order: lower half + upper half
            const float y0 = __shfl_xor(z0, 1), y1 = __shfl_xor(z1, 1), y2 = __shfl_xor(z2, 1);
            const int row = m0 + round * 128 + tok;
            if (half == 0 && row < p.M) {
                float* zp = p.zpart + ((size_t)nt * p.M + row) * 3;
                zp[0] = z0 + y0;
                zp[1] = z1 + y1;
                zp[2] = z2 + y2;
            }
        }
        __syncthreads();
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
    const int MT = (rp.M + BM - 1) / BM;
    const int MT8 = (MT + 7) / 8 * 8;
    router_gemm_kernel<<<dim3(MT8 * (rp.I / BI)), 256, 0, st>>>(rp);
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
