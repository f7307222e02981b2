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
constexpr int BK = kRouterBK;          // K elements per LDS stage
constexpr int NW = kRouterWaves;       // wavefronts per workgroup (2 per SIMD)
constexpr int NT = 64 * NW;            // threads
constexpr int ROWB = BK * 2;           // bytes per tile row and stage
constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
constexpr int STAGE = (BM + BN) * ROWB;   // A tile then B tile
constexpr int LPS = BM * ROWB / (NT * 16);  // direct loads per thread and stage, for A (and for B)
constexpr int LDA = BM + 1;            // epilogue: a[inner][token], padded row of floats
constexpr int NSTAGE = kRouterStages;  // LDS ring depth
constexpr int LDS_BYTES = (NSTAGE * STAGE > BI * LDA * 4) ? NSTAGE * STAGE : BI * LDA * 4;
static_assert((CPR == 8 || CPR == 4) && BM == BN && BM * ROWB % (NT * 16) == 0, "router tile shape");
static_assert(NSTAGE == 2, "the main loop alternates two LDS stages");

// 16-byte chunk c of tile row r sits at chunk c ^ ((r / (256 / ROWB)) % CPR)
// of its LDS row: the 16 rows that one 256-byte LDS cycle of a fragment
// load serves then fall on 16 distinct bank groups.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r / (256 / ROWB)) & (CPR - 1)); }

// s_waitcnt immediate: lgkmcnt(0), the other counters left at their maximum
// (gfx9 encoding).
constexpr int kWaitLgkm0 = 0xC07F;

}  // namespace

// Router GEMM with the gate and the W3 projection fused in the epilogue.
// Workgroup tile: 256 tokens x 128 inner indices (the W1 and the W2 rows of
// those indices), K staged 64 at a time through two LDS buffers filled by
// direct buffer->LDS loads.  512 threads = 8 waves, two per SIMD so that
// one wave's LDS fragment reads overlap the other's MFMAs: wave (wm, wn)
// owns tokens wm*128..+127 and inner wn*32..+31, i.e. 4 x 2 MFMA 32x32x16
// bf16 blocks (h1 and h2 of the same inner indices).  Each wave keeps two
// register sets of fragments: the LDS reads of the next 16-wide K step go
// out before the MFMAs of the current one, and the wait for them comes
// only at the start of the next step.  Tiles are ordered so that the eight
// inner tiles of a token tile run on one XCD and share its L2.
__global__ __launch_bounds__(NT, 2) void router_gemm_kernel(RouterParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int NTI = p.I / BI;
    const int MT = (p.M + BM - 1) / BM;
    // XCD-aware order: workgroup id -> (token tile, inner tile)
    const int id = blockIdx.x;
    const int xcd = id & 7, local = id >> 3;
    const int mt = (local / NTI) * 8 + xcd, nt = local % NTI;
    if (mt >= MT) return;
    const int m0 = mt * BM, i0 = nt * BI;
    const int D = p.D;

    // Direct loads: load j of this thread fills LDS bytes [(j*NT + tid)*16,
    // +16) of the A (and of the B) region of a stage.  Addresses are a
    // wave-uniform base (the workgroup's first row, advanced by K) plus a
    // 32-bit per-lane byte offset, so the loads take the scalar-base form.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint8_t* xbase = reinterpret_cast<const uint8_t*>(p.x + (size_t)m0 * D);
    const uint8_t* wbase = reinterpret_cast<const uint8_t*>(p.w12 + (size_t)i0 * D);
    uint32_t a_off[LPS], b_off[LPS];
#pragma unroll
    for (int j = 0; j < LPS; ++j) {
        const int r = (j * NT + tid) / CPR;                  // tile row
        const int c = swz(r, tid % CPR);                     // logical chunk held by this slot
        const int xr = min(r, p.M - 1 - m0);                 // rows past M read a valid row
        a_off[j] = (uint32_t)(xr * D + c * 8) * 2u;
        const int wr = r < BI ? r : p.I + (r - BI);
        b_off[j] = (uint32_t)(wr * D + c * 8) * 2u;
    }
    // buffer resources over the workgroup's rows (no range limit: every
    // offset is in bounds by construction)
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)xbase, (short)0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc((void*)wbase, (short)0, -1, 0x00020000);
    auto stage_load = [&](int buf, int k0) {
        uint8_t* base = lds + buf * STAGE + wave_u * 64 * 16;
        const unsigned koff = (unsigned)k0 * 2u;
#pragma unroll
        for (int j = 0; j < LPS; ++j) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_void*)(base + j * NT * 16), 16, a_off[j], koff, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void*)(base + BM * ROWB + j * NT * 16), 16, b_off[j],
                                                     koff, 0, 0);
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;

    const int lr = lane & 31, lh = lane >> 5;
    const int nk = D / BK;
    // fragments of K step ks of the stage in buffer buf
    auto load_frags = [&](bf16x8* af, bf16x8* bfr, int buf, int ks) {
        const uint8_t* As = lds + buf * STAGE;
        const uint8_t* Bs = As + BM * ROWB;
        const int c = 2 * ks + lh;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int r = wm * 128 + mb * 32 + lr;
            af[mb] = *reinterpret_cast<const bf16x8*>(As + r * ROWB + swz(r, c) * 16);
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int r = nb * BI + wn * 32 + lr;
            bfr[nb] = *reinterpret_cast<const bf16x8*>(Bs + r * ROWB + swz(r, c) * 16);
        }
    };
    // Two LDS stages.  Stage kt+1 is issued (after the barrier of step
    // kt-1's last K step) into the buffer that stage kt-1 left, and awaited
    // before the last K step of stage kt.  Fragments are double-buffered in
    // registers: the reads of the next K step (the first of the next stage,
    // after the barrier) go out before the MFMAs of the current one.
    bf16x8 af[2][4], bfr[2][2];
    stage_load(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (nk > 1) stage_load(1, BK);
    load_frags(af[0], bfr[0], 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int f = ks & 1;
            // this step's fragments (read during the previous step's MFMAs)
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 1 < BK / 16) {
                load_frags(af[f ^ 1], bfr[f ^ 1], cur, ks + 1);
            } else if (kt + 1 < nk) {
                // every lane's part of stage kt+1 has landed and every wave
                // has finished reading stage kt: its buffer takes stage kt+2
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (kt + 2 < nk) stage_load(cur, (kt + 2) * BK);
                load_frags(af[f ^ 1], bfr[f ^ 1], cur ^ 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[f][mb], bfr[f][nb], acc[mb][nb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();

    // ---------------- epilogue: a = SiLU(h1 * h2) = u * sigmoid(u) into LDS as
    // a[inner][token], then this tile's share of z = a W3^T: thread (half,
    // token) sums 64 inner indices; the two halves are added in a fixed order.
    float* a_lds = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tok = wm * 128 + mb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            const int ii = wn * 32 + lr;
            const float u = acc[mb][0][r] * acc[mb][1][r];
            const float e = __builtin_amdgcn_exp2f(-u * 1.4426950408889634f);
            a_lds[ii * LDA + tok] = u * __builtin_amdgcn_rcpf(1.0f + e);
        }
    __syncthreads();
    {
        const int tok = tid % BM;
        const int half = __builtin_amdgcn_readfirstlane(tid / BM);      // wave-uniform
        const float* w3 = p.w3 + i0 + half * (BI / 2);
        float z0 = 0.f, z1 = 0.f, z2 = 0.f;
#pragma unroll 8
        for (int i = 0; i < BI / 2; ++i) {
            const float a = a_lds[(half * (BI / 2) + i) * LDA + tok];
            z0 = __builtin_fmaf(a, w3[i], z0);
            z1 = __builtin_fmaf(a, w3[p.I + i], z1);
            z2 = __builtin_fmaf(a, w3[2 * p.I + i], z2);
        }
        __syncthreads();
        float* zz = a_lds;                    // [BM][3] partials of the upper half
        if (half == 1) {
            zz[tok * 3 + 0] = z0;
            zz[tok * 3 + 1] = z1;
            zz[tok * 3 + 2] = z2;
        }
        __syncthreads();
        const int row = m0 + tok;
        if (half == 0 && row < p.M) {
            float* zp = p.zpart + ((size_t)nt * p.M + row) * 3;
            zp[0] = z0 + zz[tok * 3 + 0];
            zp[1] = z1 + zz[tok * 3 + 1];
            zp[2] = z2 + zz[tok * 3 + 2];
        }
    }
}

// One block of 256 threads per (new chunk, sequence).  Each wavefront counts
// its tokens' experts with ballots and popcounts, the four wavefronts' counts
// meet in LDS, and the chunk takes the expert with the most tokens (the
// smallest index on a tie).
__global__ __launch_bounds__(256) void vote_kernel(VoteParams p) {
    __shared__ int wcnt[4][3];            // per-wavefront expert counts
    const int c = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int M = p.B * p.T;
    // counts of this wavefront's tokens, wave-uniform (ballot + popcount;
    // a lane past the chunk end takes no part in the ballots)
    int n_all = 0, n1 = 0, n2 = 0;
    for (int t = threadIdx.x; t < p.C; t += blockDim.x) {
        const size_t row = (size_t)b * p.T + (size_t)c * p.C + t;
        float z[3];
        if (p.zpart) {
            // the slices in tile order (the loads of eight tiles go out together)
            float s0 = 0.f, s1 = 0.f, s2 = 0.f;
#pragma unroll 8
            for (int tile = 0; tile < p.ntile; ++tile) {
                const float* zp = p.zpart + ((size_t)tile * M + row) * 3;
                s0 += zp[0];
                s1 += zp[1];
                s2 += zp[2];
            }
            z[0] = s0 + p.b3[0];
            z[1] = s1 + p.b3[1];
            z[2] = s2 + p.b3[2];
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
        n_all += __popcll(__ballot(1));
        n1 += __popcll(__ballot(e == 1));
        n2 += __popcll(__ballot(e == 2));
    }
    if (lane == 0) {
        wcnt[wave][0] = n_all - n1 - n2;
        wcnt[wave][1] = n1;
        wcnt[wave][2] = n2;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int cnt[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) cnt[k] = (wcnt[0][k] + wcnt[1][k]) + (wcnt[2][k] + wcnt[3][k]);
        int v = 0;
        if (cnt[1] > cnt[v]) v = 1;
        if (cnt[2] > cnt[v]) v = 2;
        const int chunk = p.chunk_offset + c;
        if (p.freeze_first && chunk == 0) v = 0;
        p.chunk_bits[(size_t)b * p.n_max + chunk] = (uint8_t)bits_of_expert(v);
    }
}

// One block of 256 threads per sequence: stable partition of chunks
// [0, n_total) into the FP16, INT4, INT2 segments.  Thread t owns a
// contiguous share of the chunks; its slot in each segment is the count of
// that segment's chunks in the shares before it (a wavefront DPP scan plus
// the four wavefronts' totals).
__global__ __launch_bounds__(256) void reorder_kernel(ReorderParams p) {
    __shared__ int wtot[4][3];            // per-wavefront segment counts
    const int b = blockIdx.x, tid = threadIdx.x;
    const int n = p.n_total;
    const int per = (n + 255) / 256;
    const int c0 = min(tid * per, n), c1 = min(c0 + per, n);
    const uint8_t* bits = p.chunk_bits + (size_t)b * p.n_max;
    if (p.sel.sel_part) {
        // Similarity selection of the new chunks in this thread's share (the
        // thread reads back only bitwidths it wrote itself): the slices'
        // sums in slice order, the cosine in fp32 (0 when either vector is
        // zero), FP16 at or above tau_hi, INT4 at or above tau_lo, INT2
        // below; routing freezing pins chunk 0 to FP16.
        const SelectStep& q = p.sel;
        for (int c = max(c0, q.first); c < min(c1, q.first + q.n_new); ++c) {
            const int cn = c - q.first;
            float dot = 0.f, ss = 0.f, qq = 0.f;
            const float4* pp = q.sel_part + ((size_t)b * q.n_new + cn) * q.ds;
#pragma unroll 8
            for (int s = 0; s < q.ds; ++s) {   // in slice order; eight loads go out together
                const float4 v = pp[s];
                dot += v.x;
                ss += v.y;
                qq += v.z;
            }
            const float den = sqrtf(ss) * sqrtf(qq);
            const float sim = den > 0.f ? dot / den : 0.f;
            int e = sim >= q.tau_hi ? 0 : (sim >= q.tau_lo ? 1 : 2);
            if (q.freeze_first && c == 0) e = 0;
            q.chunk_bits[(size_t)b * p.n_max + c] = (uint8_t)bits_of_expert(e);
            if (q.sim) q.sim[(size_t)b * q.n_new + cn] = sim;
        }
    }
    int local[3] = {0, 0, 0};
    for (int c = c0; c < c1; ++c) {
        int k = expert_of_bits(bits[c]);
        if (k < 0) {
            if (p.bad) p.bad[0] = 1;
            k = 2;
        }
        ++local[k];
    }
    // exclusive prefix of the counts in thread order: a DPP scan inside each
    // wavefront, then the four wavefronts' totals through LDS
    const int lane = tid & 63, wave = tid >> 6;
    int incl[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) incl[k] = wave_incl_sum(local[k]);
    if (lane == 63) {
#pragma unroll
        for (int k = 0; k < 3; ++k) wtot[wave][k] = incl[k];
    }
    __syncthreads();
    int excl[3], tot[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        int before = 0, all = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int x = wtot[w][k];
            before += w < wave ? x : 0;
            all += x;
        }
        excl[k] = before + incl[k] - local[k];
        tot[k] = all;
    }
    const int tot0 = tot[0], tot1 = tot[1], tot2 = tot[2];
    if (tid == 0) {
        p.seg_count[b * 3 + 0] = tot0;
        p.seg_count[b * 3 + 1] = tot1;
        p.seg_count[b * 3 + 2] = tot2;
    }
    const int start[3] = {0, tot0, tot0 + tot1};
    int run[3] = {excl[0], excl[1], excl[2]};
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
    router_gemm_kernel<<<dim3(MT8 * (rp.I / BI)), NT, 0, st>>>(rp);
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
