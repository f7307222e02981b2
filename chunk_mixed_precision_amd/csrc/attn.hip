// Split-K decode attention over the mixed-bitwidth packed cache
// (MoQAE "Overall framework": ordinary attention after quantization;
// Cocktail abstract: chunk-level computation over bitwidth-contiguous
// segments, so every work unit below has a single bitwidth and no wavefront
// ever branches on bitwidth inside its inner loop).
//
// Work.  The packed bytes of each (sequence, KV head) -- its FP16, INT4 and
// INT2 segments in that order -- are cut into units of one wavefront
// iteration (GPI group blocks of one segment).  All (sequence, head) streams
// are laid end to end and split into ranges of equal cost, one per workgroup
// of kAttnWaves wavefronts (one CU's worth); a unit's cost is its bytes times
// a per-bitwidth weight, because an INT2 byte holds more codes to dequantize
// than an INT4 byte and an FP16 byte fewer.  A range may span several
// (sequence, head) streams, each giving one "piece".  Inside a piece the
// wavefronts take units from a workgroup-local ticket counter in LDS, so a
// wavefront that the CU's scheduler favours simply takes more units and all
// of them finish together.  Each wavefront keeps one online-softmax state
// across the units (and bitwidths) it takes; at the end of a piece the
// workgroup merges its wavefronts' states in LDS and writes one partial.  A
// second launch merges the partials of each (sequence, head).
//
// A wavefront is split into R = 64/S rows of S = d/8 lanes; each row handles
// one group block per iteration for one query head, or for two with two query
// heads per KV head.  With four heads per KV head two rows share a group block
// and split its data (keys by token, values by channel), each serving all
// four heads (run_piece_g4).  Inside a row, lane slot L owns channels
// 8L..8L+7 of the keys and value group L % (d/32) of tokens L / (d/32) + 4m.
//
// Scores: s_t = sum_j q_j * (code_tj * s_j + mn_j) is evaluated as
// sum_j (q_j s_j) code_tj + sum_j q_j mn_j, so key dequantization costs one
// FMA per code and head: a masked code field ORed into an fp16 exponent
// pattern is converted and multiplied in one v_fma_mix_f32, and the
// pattern's constant is taken off the accumulator once per group.  Per-row
// partial sums are combined with a select-free DPP reduce-scatter (the
// layout's per-lane token xor makes every butterfly step keep the low
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

// Packed codes are read once per call: nontemporal loads (the `nt` bit) keep
// them from displacing reusable lines and stream measurably faster than
// plain loads on this part.
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
    const u32x4_nt x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ float4 ldf4(const uint8_t* p) { return *reinterpret_cast<const float4*>(p); }

__device__ __forceinline__ float4 as_f4(const uint4& u) { return __builtin_bit_cast(float4, u); }

// Every load phase brings in 8 rows of a group block (8 x 16 B per lane).
// INT4: 3 phases: rows 0-7 = key meta + key codes of tokens 0-15, rows 8-15 =
//       key codes of tokens 16-31 + value meta, rows 16-23 = value codes.
// INT2: 2 phases: key meta + key codes, value meta + value codes.
// FP16: 8 phases: key rows 0-31, then value rows 0-31.
template <int BITS> __host__ __device__ constexpr int n_phases() { return BITS == 16 ? 8 : (BITS == 4 ? 3 : 2); }

// Rows 8*phase .. 8*phase+7 of the group block at base + voff (base is
// wave-uniform, voff = this lane's byte offset: its row's block and its
// 16-byte cell).
template <int D>
__device__ __forceinline__ void load_rows8(uint4* buf, const uint8_t* base, uint32_t voff, int phase) {
    constexpr size_t ROWB = (size_t)(D / 8) * 16;
    const uint8_t* src = base + (size_t)phase * 8 * ROWB;
#pragma unroll
    for (int i = 0; i < 8; ++i) buf[i] = ld16(src + voff + i * ROWB);
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


// ---------------------------------------------------------------- work map
// A wave-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ long long uniform64(long long x) {
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(unsigned long long)x);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)x >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}

// Units of one (sequence, head) stream.  Every head of a sequence has the
// same segment sizes, so the geometry depends on the sequence only.
template <int D, int HB>
struct SeqUnits {
    static constexpr int GPI = (512 / D) * attn_heads_per_row(HB) / HB;   // group blocks per unit
    int segg[3];        // group blocks written in each segment
    int nu[3];          // units in each segment
    int ubase[3];       // index of each segment's first unit
    int soff[3];        // cost offset of each segment's first unit in the stream
    int cost;           // cost of the whole stream (units x unit cost)
    int units;

    // Cost of one unit of segment k, in granules of kAttnGranule bytes.
    static constexpr int unit_cost(int k) {
        return GPI * group_bytes(bits_of_expert(k), D) * attn_cost16(HB, k) / (16 * kAttnGranule);
    }
    static_assert(GPI * group_bytes(16, D) * attn_cost16(HB, 0) % (16 * kAttnGranule) == 0 &&
                  GPI * group_bytes(4, D) * attn_cost16(HB, 1) % (16 * kAttnGranule) == 0 &&
                  GPI * group_bytes(2, D) * attn_cost16(HB, 2) % (16 * kAttnGranule) == 0,
                  "unit costs are whole granules");

    __device__ __forceinline__ void init(const AttnParams& p, int b) {
        init_counts(p, p.seg_count[b * 3 + 0], p.seg_count[b * 3 + 1], p.seg_count[b * 3 + 2]);
    }
    // from the sequence's chunk counts (FP16, INT4, INT2)
    __device__ __forceinline__ void init_counts(const AttnParams& p, int c0, int c1, int c2) {
        const int gpc = p.C / kGroup;
        const int cnt3[3] = {c0, c1, c2};
        int off = 0;
        int u = 0;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            // chunks beyond a pool's capacity were never written: never read them
            const int cnt = min(max(cnt3[k], 0), p.cap[k]);
            segg[k] = cnt * gpc;
            nu[k] = (segg[k] + GPI - 1) / GPI;
            ubase[k] = u;
            soff[k] = off;
            u += nu[k];
            off += nu[k] * unit_cost(k);
        }
        units = u;
        cost = off;
    }

    // Index of the first unit whose start is at or after stream offset x
    // (units when there is none).
    __device__ __forceinline__ int first_at_or_after(int x) const {
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            if (nu[k] == 0) continue;
            const int rel = x - soff[k];
            const int u = rel <= 0 ? 0 : (int)(((unsigned)rel + unit_cost(k) - 1) / (unsigned)unit_cost(k));
            if (u < nu[k]) return ubase[k] + u;
        }
        return units;
    }

    __device__ __forceinline__ int unit_start(int U) const {
        if (U < ubase[1]) return soff[0] + (U - ubase[0]) * unit_cost(0);
        if (U < ubase[2]) return soff[1] + (U - ubase[1]) * unit_cost(1);
        return soff[2] + (U - ubase[2]) * unit_cost(2);
    }
};

// Cost of the whole cache (every (sequence, head) stream), computed by one
// wavefront with one sequence per lane; every lane gets the result.
template <int D, int HB>
__device__ __forceinline__ int total_cost(const AttnParams& p) {
    const int lane = threadIdx.x & 63;
    int t = 0;
    for (int b0 = 0; b0 < p.B; b0 += 64) {
        const int b = b0 + lane;
        int x = 0;
        if (b < p.B) {
            SeqUnits<D, HB> su;
            su.init(p, b);
            x = su.cost;
        }
        t += wave_sum(x);
    }
    return t * p.Hkv;
}

// Workgroups actually used: at most G, and few enough that every range is at
// least kAttnMinWgCost long (longer than any unit, so each workgroup
// between the first and the last owner of a stream owns a unit of it).
__device__ __forceinline__ int used_workgroups(const AttnParams& p, int total) {
    const int g = total / (int)(kAttnMinWgCost / kAttnGranule);
    return max(1, min(p.G, g));
}

// Start of workgroup w's range, floor(w*T/G).  In fp64: the product is
// exact (below 2^40) and the correctly rounded quotient of two such numbers
// never crosses an integer (a non-integer quotient below 2^31 lies at least
// 1/G from one), so the floor is exact -- and much cheaper than a 64-bit
// integer division.
__device__ __forceinline__ int split_point(int w, int total, int G) {
    return (int)(((double)w * (double)total) / (double)G);
}

// The workgroup whose cost range contains global offset x:
// range w = [floor(w*T/G), floor((w+1)*T/G)), i.e. floor(((x+1)*G - 1) / T)
// (exact in fp64 as above).
__device__ __forceinline__ int owner_of(int x, int total, int G) {
    return (int)(((double)(x + 1) * (double)G - 1.0) / (double)total);
}

// Global offset of sequence b's first stream (head 0): Hkv * sum of the
// stream costs of sequences 0 .. b-1.  One wavefront, every lane gets it.
template <int D, int HB>
__device__ __forceinline__ int seq_offset(const AttnParams& p, int b) {
    const int lane = threadIdx.x & 63;
    int t = 0;
    for (int b0 = 0; b0 < b; b0 += 64) {
        const int bb = b0 + lane;
        int x = 0;
        if (bb < b) {
            SeqUnits<D, HB> su;
            su.init(p, bb);
            x = su.cost;
        }
        t += wave_sum(x);
    }
    return t * p.Hkv;
}

// The sequence whose streams contain global offset x (x < total), and the
// global offset of its first stream.  One wavefront, uniform result.
template <int D, int HB>
__device__ __forceinline__ int seq_containing(const AttnParams& p, int x, int& seq_off) {
    const int lane = threadIdx.x & 63;
    int carry = 0;
    for (int b0 = 0; b0 < p.B; b0 += 64) {
        const int b = b0 + lane;
        int v = 0;
        if (b < p.B) {
            SeqUnits<D, HB> su;
            su.init(p, b);
            v = su.cost * p.Hkv;
        }
        const int incl = wave_incl_sum(v);
        const unsigned long long hit = __ballot(b < p.B && carry + incl > x);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            seq_off = carry + __builtin_amdgcn_readlane(incl - v, l);
            return b0 + l;
        }
        carry += __builtin_amdgcn_readlane(incl, 63);
    }
    seq_off = carry;
    return p.B;
}

// ---------------------------------------------------------------- one piece
// Units [U0, U1) of the stream of (b, h), processed by the kAttnWaves
// wavefronts of the workgroup, which take units from the ticket counter
// *ctr: ticket t is unit U0 + (t - tbase).  The counter is never reset: a
// piece consumes exactly (U1 - U0) + kAttnWaves tickets (one per unit and
// one failing grab per wavefront), all before the workgroup barrier that
// ends the piece, so the caller knows the next piece's base.  Leaves one
// partial per query head of the group at record `slot`.
//
// One or two query heads per KV head: a row serves all HB of them, so every
// code word is unpacked once and feeds the heads' FMAs.  (Four heads per KV
// head take run_piece_g4.)
template <int D, int HB>
__device__ __forceinline__ void run_piece(const AttnParams& p, const SeqUnits<D, HB>& su, int b, int h, int U0,
                                          int U1, int tbase, int slot, int* ctr, float* plds, float* rec) {
    constexpr int S = D / 8;
    constexpr int R = 64 / S;          // rows per wave
    constexpr int NG = D / 32;         // value groups per token
    constexpr int HPR = attn_heads_per_row(HB);
    constexpr int GPI = R;             // group blocks per unit: one per row
    static_assert(HPR == HB, "a row serves every head of its KV head");
    constexpr int NTH = 16 / S;        // tokens per lane and key half after the reduce-scatter
    constexpr int RECF = D + 4;        // floats per merged record
    static_assert(GPI == SeqUnits<D, HB>::GPI, "unit geometry");

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = lane / S, L = lane % S;
    const int gslot = row;
    const int G = L % NG, tq = L / NG;
    const int fx = tok_xor(S, L);
    const int bh = b * p.Hkv + h;
    const int hq0 = h * p.hpk + p.hoff;  // this row's first query head

    // segment base pointers of this (b, h)
    const size_t gpc = (size_t)(p.C / kGroup);
    const uint8_t* seg16 = p.pool[0] + (size_t)bh * p.cap[0] * gpc * group_bytes(16, D);
    const uint8_t* seg4 = p.pool[1] + (size_t)bh * p.cap[1] * gpc * group_bytes(4, D);
    const uint8_t* seg2 = p.pool[2] + (size_t)bh * p.cap[2] * gpc * group_bytes(2, D);

    // the first unit's loads go out before the query's
    uint4 bufA[8], bufB[8];
    auto grab = [&]() -> int {
        int t = 0;
        if (lane == 0) t = atomicAdd(ctr, 1);
        return U0 + (__builtin_amdgcn_readfirstlane(t) - tbase);
    };
    // Unit U (any segment): the wave-uniform address of its first group
    // block and this lane's offset from there (its row's block, rows past the
    // end of the segment re-read the first block, and its 16-byte cell).
    auto unit_addr = [&](int U, uint32_t& voff) -> const uint8_t* {
        int k = 0, u = U;
        const uint8_t* base = seg16;
        uint32_t gb = (uint32_t)group_bytes(16, D);
        if (U >= su.ubase[2]) {
            k = 2; u = U - su.ubase[2]; base = seg2; gb = (uint32_t)group_bytes(2, D);
        } else if (U >= su.ubase[1]) {
            k = 1; u = U - su.ubase[1]; base = seg4; gb = (uint32_t)group_bytes(4, D);
        }
        const int segg = k == 0 ? su.segg[0] : (k == 1 ? su.segg[1] : su.segg[2]);
        const bool live = u * GPI + gslot < segg;
        voff = (live ? (uint32_t)gslot * gb : 0u) + (uint32_t)L * 16u;
        return base + (size_t)u * GPI * gb;
    };
    int U = grab();
    uint32_t vo = 0;
    const uint8_t* ub = seg16;
    if (U < U1) {
        ub = unit_addr(U, vo);
        load_rows8<D>(bufA, ub, vo, 0);
    }

    // query channels 8L..8L+7 of this row's heads
    uint32_t qw[HPR][4];
#pragma unroll
    for (int j = 0; j < HPR; ++j) {
        const uint4 qc = *reinterpret_cast<const uint4*>(p.q + ((size_t)b * p.Hq + hq0 + j) * D + 8 * L);
        qw[j][0] = qc.x; qw[j][1] = qc.y; qw[j][2] = qc.z; qw[j][3] = qc.w;
    }
    float qs[HPR][8];      // q * log2(e)/sqrt(d) in fp32 (INT-b keys), set after the FP16 segment

    float M[HPR];          // running max of this row and head (log2 domain), row-uniform
    float lsum[HPR];       // this lane's share of the softmax denominator
    float o[HPR][32];      // channels 32G .. 32G+31
    float pm[HPR];         // sum_t p_t * mn_t over this lane's value tokens
#pragma unroll
    for (int j = 0; j < HPR; ++j) {
        M[j] = -INFINITY;
        lsum[j] = 0.f;
        pm[j] = 0.f;
#pragma unroll
        for (int c = 0; c < 32; ++c) o[j][c] = 0.f;
    }

    float sc[HPR][2 * NTH];   // this lane's key scores: half 0, then half 1
    float pw[HPR][8];         // value weights of tokens tq + 4m: p (FP16), p * scale / 16 (INT-b)
    float kw[HPR][8];         // key weights q_j * s_j / 16 of this lane's channels (INT-b), this group
    float koff[HPR];          // initial key accumulator of codes at bits 4-7: sum_j q_j mn_j - 1024 * sum_j kw_j
    float koff64[HPR];        // the same for INT2 codes at bits 6-7 (weights kw/4): sum_j q_j mn_j - 256 * sum_j kw_j
    float alpha_v[HPR];       // softmax rescale still owed to o[] (INT-b: applied with the value offset)
    float acc[HPR][16];

    // INT-b codes are converted and multiplied in one v_fma_mix_f32: a code c
    // at bits 4-5 / 4-7 (or 6-7) of an fp16 half whose other bits are 0x6400
    // is the fp16 number 1024 + 16c (or 1024 + 64c).  With the weight w/16
    // (w/64) the product is 64w + cw (16w + cw); the constant parts of one
    // group are taken off the accumulator beforehand.  Keeping every code in
    // the upper half of the 10-bit mantissa bounds the offset at 64 times
    // the weight, so the fp32 accumulators lose at most a few bits.
    uint32_t vmagic;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(vmagic));
    // With two query heads per row the INT4 codes are instead unpacked into
    // bytes and converted to fp32 (v_cvt_f32_ubyte), once for both heads,
    // and multiplied with plain fp32 FMAs, which issue faster than the mixed
    // fp16/fp32 ones; the weights then carry no 1/16 and the accumulators no
    // pattern offset.
    constexpr bool CVT4 = HPR == 2;
    auto lo16 = [](uint32_t y) { return (float)__builtin_bit_cast(half2_t, y).x; };
    auto hi16 = [](uint32_t y) { return (float)__builtin_bit_cast(half2_t, y).y; };

    // ---- online-softmax update from sc[], probabilities to the value layout.
    // FP16 units rescale o[] here; INT-b units leave the factor in alpha_v
    // for the value phase, which folds it into the offset subtraction.
    auto softmax_step = [&](auto bits_tag, bool valid) {
        constexpr int BITS = decltype(bits_tag)::value;
#pragma unroll
        for (int j = 0; j < HPR; ++j) {
            float mloc = -INFINITY;
#pragma unroll
            for (int i = 0; i < 2 * NTH; ++i) {
                if (!valid) sc[j][i] = -INFINITY;
                mloc = fmaxf(mloc, sc[j][i]);
            }
            mloc = row_max<S>(mloc);
            const float Mn = fmaxf(M[j], mloc);
            const float alpha = (Mn == -INFINITY) ? 1.f : fast_exp2(M[j] - Mn);
            M[j] = Mn;
            float pt[2 * NTH];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 2 * NTH; ++i) {
                pt[i] = valid ? fast_exp2(sc[j][i] - Mn) : 0.f;
                psum += pt[i];
            }
            lsum[j] = __builtin_fmaf(lsum[j], alpha, psum);
            pm[j] *= alpha;
            if constexpr (BITS == 16) {
#pragma unroll
                for (int c = 0; c < 32; ++c) o[j][c] *= alpha;
            } else {
                alpha_v[j] = alpha;
            }
            // slot of token t in the value layout: (t & 3) * 8 + (t >> 2)
            float* pl = plds + (row * HPR + j) * 32;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int i = 0; i < NTH; ++i) {
                    const int t = 16 * hh + (fx ^ i);
                    pl[(t & 3) * 8 + (t >> 2)] = pt[hh * NTH + i];
                }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int j = 0; j < HPR; ++j) {
            const float* pl = plds + (row * HPR + j) * 32;
            const float4 pa = *reinterpret_cast<const float4*>(pl + tq * 8);
            const float4 pb = *reinterpret_cast<const float4*>(pl + tq * 8 + 4);
            pw[j][0] = pa.x; pw[j][1] = pa.y; pw[j][2] = pa.z; pw[j][3] = pa.w;
            pw[j][4] = pb.x; pw[j][5] = pb.y; pw[j][6] = pb.z; pw[j][7] = pb.w;
        }
    };

    // ---- INT-b pieces
    auto key_meta = [&](const uint4* m4, auto cvt_tag) {   // rows: scale lo, scale hi, min lo, min hi
        constexpr bool CVT = decltype(cvt_tag)::value;
        const float4 s0 = as_f4(m4[0]), s1 = as_f4(m4[1]), n0 = as_f4(m4[2]), n1 = as_f4(m4[3]);
        const float ks[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const float kmn[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
#pragma unroll
        for (int j = 0; j < HPR; ++j) {
            float bias = 0.f, sw = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bias = __builtin_fmaf(qs[j][e], kmn[e], bias);
                kw[j][e] = CVT ? qs[j][e] * ks[e] : qs[j][e] * ks[e] * 0.0625f;
                sw += kw[j][e];
            }
            if constexpr (CVT) {
                koff[j] = bias;
            } else {
                koff[j] = __builtin_fmaf(-1024.f, sw, bias);
                koff64[j] = __builtin_fmaf(-256.f, sw, bias);
            }
        }
    };
    // 4 key-code rows of one half (INT4).  Field f of word w is the code of
    // position 8w + f; the shifts bring fields (0, 4), (1, 5), (2, 6), (3, 7)
    // of a word to bits 4-7 of its low / high half.
    auto key_half_int4 = [&](const uint4* rows) {
#pragma unroll
        for (int j = 0; j < HPR; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][r] = koff[j];
        if constexpr (CVT4) {
            // field g of a word: byte g/2 of its low (g even) or high (g odd) nibbles
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int w = i >> 1;
                const uint32_t ws[4] = {rows[i].x, rows[i].y, rows[i].z, rows[i].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = ws[e] & 0x0F0F0F0Fu, hi = (ws[e] >> 4) & 0x0F0F0F0Fu;
                    const float c[8] = {cvt_ub<0>(lo), cvt_ub<0>(hi), cvt_ub<1>(lo), cvt_ub<1>(hi),
                                        cvt_ub<2>(lo), cvt_ub<2>(hi), cvt_ub<3>(lo), cvt_ub<3>(hi)};
#pragma unroll
                    for (int j = 0; j < HPR; ++j) {
                        const float wq = kw[j][4 * (i & 1) + e];
#pragma unroll
                        for (int g = 0; g < 8; ++g) acc[j][8 * w + g] = __builtin_fmaf(wq, c[g], acc[j][8 * w + g]);
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int w = i >> 1;
            const uint32_t ws[4] = {rows[i].x, rows[i].y, rows[i].z, rows[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = ws[e];
                const uint32_t y[4] = {((x << 4) & 0x00F000F0u) | vmagic, (x & 0x00F000F0u) | vmagic,
                                       ((x >> 4) & 0x00F000F0u) | vmagic, ((x >> 8) & 0x00F000F0u) | vmagic};
#pragma unroll
                for (int j = 0; j < HPR; ++j) {
                    const float wq = kw[j][4 * (i & 1) + e];
#pragma unroll
                    for (int f = 0; f < 4; ++f) {
                        acc[j][8 * w + f] = __builtin_fmaf(wq, lo16(y[f]), acc[j][8 * w + f]);
                        acc[j][8 * w + 4 + f] = __builtin_fmaf(wq, hi16(y[f]), acc[j][8 * w + 4 + f]);
                    }
                }
            }
        }
    };
    // 2 key-code rows of one half (INT2).  Field f of the word is the code
    // of position f; shifted copies bring fields (2s, 2s+1) and (2s+8, 2s+9)
    // to bits 4-5 / 6-7 of the low / high half (weights w/16 and w/64).
    auto key_half_int2 = [&](const uint4* rows) {
#pragma unroll
        for (int j = 0; j < HPR; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][r] = (r & 1) ? koff64[j] : koff[j];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t ws[4] = {rows[i].x, rows[i].y, rows[i].z, rows[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = ws[e];
                const uint32_t src[4] = {x << 4, x, x >> 4, x >> 8};
#pragma unroll
                for (int sh = 0; sh < 4; ++sh) {
                    const uint32_t ya = (src[sh] & 0x00300030u) | vmagic;
                    const uint32_t yb = (src[sh] & 0x00C000C0u) | vmagic;
#pragma unroll
                    for (int j = 0; j < HPR; ++j) {
                        const float w16 = kw[j][4 * i + e], w64 = w16 * 0.25f;
                        acc[j][2 * sh] = __builtin_fmaf(w16, lo16(ya), acc[j][2 * sh]);
                        acc[j][2 * sh + 8] = __builtin_fmaf(w16, hi16(ya), acc[j][2 * sh + 8]);
                        acc[j][2 * sh + 1] = __builtin_fmaf(w64, lo16(yb), acc[j][2 * sh + 1]);
                        acc[j][2 * sh + 9] = __builtin_fmaf(w64, hi16(yb), acc[j][2 * sh + 9]);
                    }
                }
            }
        }
    };
    auto take_half = [&](int hh) {
#pragma unroll
        for (int j = 0; j < HPR; ++j) {
            reduce_half<S>(acc[j]);
#pragma unroll
            for (int i = 0; i < NTH; ++i) sc[j][hh * NTH + i] = acc[j][i];
        }
    };
    auto value_meta = [&](const uint4* m4, auto cvt_tag) {   // (scale, min) of tokens t_{2r}, t_{2r+1}
        constexpr bool CVT = decltype(cvt_tag)::value;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float4 sm = as_f4(m4[m >> 1]);
            const float s = (m & 1) ? sm.z : sm.x;
            const float mn = (m & 1) ? sm.w : sm.y;
#pragma unroll
            for (int j = 0; j < HPR; ++j) {
                pm[j] = __builtin_fmaf(pw[j][m], mn, pm[j]);
                pw[j][m] = CVT ? pw[j][m] * s : pw[j][m] * s * 0.0625f;
            }
        }
    };
    // row m: token tq + 4m; word u holds channels 8u .. 8u+7 of the group
    auto values_int4 = [&](const uint4* rows) {
        if constexpr (CVT4) {
#pragma unroll
            for (int j = 0; j < HPR; ++j)
#pragma unroll
                for (int c = 0; c < 32; ++c) o[j][c] *= alpha_v[j];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const uint32_t ws[4] = {rows[m].x, rows[m].y, rows[m].z, rows[m].w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t lo = ws[u] & 0x0F0F0F0Fu, hi = (ws[u] >> 4) & 0x0F0F0F0Fu;
                    const float c[8] = {cvt_ub<0>(lo), cvt_ub<0>(hi), cvt_ub<1>(lo), cvt_ub<1>(hi),
                                        cvt_ub<2>(lo), cvt_ub<2>(hi), cvt_ub<3>(lo), cvt_ub<3>(hi)};
#pragma unroll
                    for (int j = 0; j < HPR; ++j) {
                        const float wv = pw[j][m];
#pragma unroll
                        for (int g = 0; g < 8; ++g) o[j][8 * u + g] = __builtin_fmaf(wv, c[g], o[j][8 * u + g]);
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < HPR; ++j) {
            float sw = 0.f;
#pragma unroll
            for (int m = 0; m < 8; ++m) sw += pw[j][m];
            const float off = 1024.f * sw;
#pragma unroll
            for (int c = 0; c < 32; ++c) o[j][c] = __builtin_fmaf(o[j][c], alpha_v[j], -off);
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint32_t ws[4] = {rows[m].x, rows[m].y, rows[m].z, rows[m].w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t x = ws[u];
                const uint32_t y[4] = {((x << 4) & 0x00F000F0u) | vmagic, (x & 0x00F000F0u) | vmagic,
                                       ((x >> 4) & 0x00F000F0u) | vmagic, ((x >> 8) & 0x00F000F0u) | vmagic};
#pragma unroll
                for (int j = 0; j < HPR; ++j) {
                    const float wv = pw[j][m];
#pragma unroll
                    for (int f = 0; f < 4; ++f) {
                        o[j][8 * u + f] = __builtin_fmaf(wv, lo16(y[f]), o[j][8 * u + f]);
                        o[j][8 * u + 4 + f] = __builtin_fmaf(wv, hi16(y[f]), o[j][8 * u + 4 + f]);
                    }
                }
            }
        }
    };
    // row r: tokens t_{2r} (dwords 0,1), t_{2r+1} (dwords 2,3); word u holds
    // channels 16u .. 16u+15 of the group
    auto values_int2 = [&](const uint4* rows) {
#pragma unroll
        for (int j = 0; j < HPR; ++j) {
            float sw = 0.f;
#pragma unroll
            for (int m = 0; m < 8; ++m) sw += pw[j][m];
            const float off16 = 1024.f * sw, off64 = 256.f * sw;
#pragma unroll
            for (int c = 0; c < 32; ++c) o[j][c] = __builtin_fmaf(o[j][c], alpha_v[j], (c & 1) ? -off64 : -off16);
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint4 cw = rows[m >> 1];
            const uint32_t ws[2] = {(m & 1) ? cw.z : cw.x, (m & 1) ? cw.w : cw.y};
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t x = ws[u];
                const uint32_t src[4] = {x << 4, x, x >> 4, x >> 8};
#pragma unroll
                for (int sh = 0; sh < 4; ++sh) {
                    const uint32_t ya = (src[sh] & 0x00300030u) | vmagic;
                    const uint32_t yb = (src[sh] & 0x00C000C0u) | vmagic;
#pragma unroll
                    for (int j = 0; j < HPR; ++j) {
                        const float w16 = pw[j][m], w64 = w16 * 0.25f;
                        o[j][16 * u + 2 * sh] = __builtin_fmaf(w16, lo16(ya), o[j][16 * u + 2 * sh]);
                        o[j][16 * u + 2 * sh + 8] = __builtin_fmaf(w16, hi16(ya), o[j][16 * u + 2 * sh + 8]);
                        o[j][16 * u + 2 * sh + 1] = __builtin_fmaf(w64, lo16(yb), o[j][16 * u + 2 * sh + 1]);
                        o[j][16 * u + 2 * sh + 9] = __builtin_fmaf(w64, hi16(yb), o[j][16 * u + 2 * sh + 9]);
                    }
                }
            }
        }
    };

    // ---- FP16 pieces: 8 key rows (q . k with v_dot2) or 8 value rows
    auto keys_fp16 = [&](const uint4* rows, int r0) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
#pragma unroll
            for (int j = 0; j < HPR; ++j) {
                float a = __builtin_amdgcn_fdot2(as_h2(rows[r].x), as_h2(qw[j][0]), 0.f, false);
                a = __builtin_amdgcn_fdot2(as_h2(rows[r].y), as_h2(qw[j][1]), a, false);
                a = __builtin_amdgcn_fdot2(as_h2(rows[r].z), as_h2(qw[j][2]), a, false);
                a = __builtin_amdgcn_fdot2(as_h2(rows[r].w), as_h2(qw[j][3]), a, false);
                acc[j][r0 + r] = a;
            }
        }
    };
    auto values_fp16 = [&](const uint4* rows, int mbase) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int cb = 8 * (r & 3);
            const uint32_t ws[4] = {rows[r].x, rows[r].y, rows[r].z, rows[r].w};
#pragma unroll
            for (int j = 0; j < HPR; ++j) {
                const float pr = pw[j][mbase + (r >> 2)];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[j][cb + 2 * e] = __builtin_fmaf(pr, lo_h(ws[e]), o[j][cb + 2 * e]);
                    o[j][cb + 2 * e + 1] = __builtin_fmaf(pr, hi_h(ws[e]), o[j][cb + 2 * e + 1]);
                }
            }
        }
    };

    // one phase's arithmetic on the rows in `cur`
    auto compute_phase = [&](auto bits_tag, int ph, const uint4* cur, bool valid) {
        constexpr int BITS = decltype(bits_tag)::value;
        if constexpr (BITS == 4) {
            if (ph == 0) {
                key_meta(cur, std::integral_constant<bool, CVT4>{});
                key_half_int4(cur + 4);
                take_half(0);
            } else if (ph == 1) {
                key_half_int4(cur);
                take_half(1);
                softmax_step(bits_tag, valid);
                value_meta(cur + 4, std::integral_constant<bool, CVT4>{});
            } else {
                values_int4(cur);
            }
        } else if constexpr (BITS == 2) {
            if (ph == 0) {
                key_meta(cur, std::false_type{});
                key_half_int2(cur + 4);
                take_half(0);
                key_half_int2(cur + 6);
                take_half(1);
                softmax_step(bits_tag, valid);
            } else {
                value_meta(cur, std::false_type{});
                values_int2(cur + 4);
            }
        } else {
            if (ph < 4) {
                keys_fp16(cur, 8 * (ph & 1));
                if (ph & 1) {
                    take_half(ph >> 1);
                    if (ph == 3) {
#pragma unroll
                        for (int j = 0; j < HPR; ++j)
#pragma unroll
                            for (int i = 0; i < 2 * NTH; ++i) sc[j][i] *= p.qscale;
                        softmax_step(bits_tag, valid);
                    }
                }
            } else {
                values_fp16(cur, 2 * (ph - 4));
            }
        }
    };

    // ---- unit loop.  Every phase's loads are issued one phase ahead, into
    // the other of two 8-row register buffers; the last phase of a unit
    // prefetches the first phase of the next unit this wavefront holds a
    // ticket for (or, when there is none, a stand-in read of this unit's
    // first bytes, which keeps the loop free of a branch whose merge point
    // would make the compiler wait for every outstanding load).  Tickets are taken in
    // increasing order, so a wavefront meets the segments in the order FP16,
    // INT4, INT2 and the three loops below run once each.
    auto run_unit = [&](auto bits_tag, auto par_tag, const uint8_t* ub, uint32_t vo, const uint8_t* ubn,
                        uint32_t von, bool valid) {
        constexpr int BITS = decltype(bits_tag)::value;
        constexpr int PAR = decltype(par_tag)::value;
        constexpr int NPH = n_phases<BITS>();
#pragma unroll
        for (int ph = 0; ph < NPH; ++ph) {
            uint4* cur = ((ph + PAR) & 1) ? bufB : bufA;
            uint4* nxt = ((ph + PAR) & 1) ? bufA : bufB;
            if (ph + 1 < NPH) load_rows8<D>(nxt, ub, vo, ph + 1);
            else load_rows8<D>(nxt, ubn, von, 0);
            __builtin_amdgcn_sched_barrier(0);
            compute_phase(bits_tag, ph, cur, valid);
        }
    };

    // one step: process unit U (whose first phase is in the buffer of parity
    // PAR) and move to the next ticket; with no next unit the prefetch reads
    // the first 16 bytes of this unit's rows with every lane (one cache line
    // per load instead of the unit's phase: the codes are loaded
    // nontemporally, so a re-read of the phase would go back to HBM)
    auto step = [&](auto bits_tag, auto par_tag, int k, int segg_k, int ubase_k) {
        const int Un = grab();
        uint32_t von = 0;
        const uint8_t* ubn = ub;
        if (Un < U1) ubn = unit_addr(Un, von);
        const bool valid = (U - ubase_k) * GPI + gslot < segg_k;
        run_unit(bits_tag, par_tag, ub, vo, ubn, von, valid);
        U = Un;
        ub = ubn;
        vo = von;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    {   // FP16 (even phase count: buffer parity is kept)
        const int end = min(U1, su.ubase[0] + su.nu[0]);
        while (U < end) step(std::integral_constant<int, 16>{}, I0{}, 0, su.segg[0], su.ubase[0]);
    }
    // the FP16 keys used the raw fp16 query; the INT-b keys take fp32 weights
#pragma unroll
    for (int j = 0; j < HPR; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qs[j][2 * e] = lo_h(qw[j][e]) * p.qscale;
            qs[j][2 * e + 1] = hi_h(qw[j][e]) * p.qscale;
        }
    {   // INT4 (odd phase count: parity flips every unit, so units go in pairs)
        const int end = min(U1, su.ubase[1] + su.nu[1]);
        bool flipped = false;
        while (U < end) {
            step(std::integral_constant<int, 4>{}, I0{}, 1, su.segg[1], su.ubase[1]);
            if (U >= end) { flipped = true; break; }
            step(std::integral_constant<int, 4>{}, I1{}, 1, su.segg[1], su.ubase[1]);
        }
        if (flipped) {
            // the next unit's first phase landed in bufB
#pragma unroll
            for (int i = 0; i < 8; ++i) bufA[i] = bufB[i];
        }
    }
    {   // INT2 (even phase count)
        const int end = min(U1, su.ubase[2] + su.nu[2]);
        while (U < end) step(std::integral_constant<int, 2>{}, I0{}, 2, su.segg[2], su.ubase[2]);
    }

    // ---------------- merge rows of the same heads, then lanes of the same value group
#pragma unroll
    for (int j = 0; j < HPR; ++j) {
#pragma unroll
        for (int c = 0; c < 32; ++c) o[j][c] += pm[j];
        float Mx = M[j];
#pragma unroll
        for (int off = S; off < 64; off <<= 1) Mx = fmaxf(Mx, __shfl_xor(Mx, off));
        const float rs = (M[j] == -INFINITY) ? 0.f : fast_exp2(M[j] - Mx);
        float l = lsum[j] * rs;
#pragma unroll
        for (int off = 1; off < S; off <<= 1) l += __shfl_xor(l, off);
#pragma unroll
        for (int off = S; off < 64; off <<= 1) l += __shfl_xor(l, off);
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            float v = o[j][c] * rs;
#pragma unroll
            for (int off = NG; off < S; off <<= 1) v += __shfl_xor(v, off);
#pragma unroll
            for (int off = S; off < 64; off <<= 1) v += __shfl_xor(v, off);
            o[j][c] = v;
        }
        // ---------------- the wavefront's record of head j, for the workgroup merge
        if (row == 0 && tq == 0) {
            float* r = rec + ((size_t)wave * HB + j) * RECF;
            float4* o4 = reinterpret_cast<float4*>(r + 32 * G);
#pragma unroll
            for (int c = 0; c < 8; ++c)
                o4[c] = make_float4(o[j][4 * c], o[j][4 * c + 1], o[j][4 * c + 2], o[j][4 * c + 3]);
            if (G == 0) {
                r[D] = Mx;
                r[D + 1] = l;
            }
        }
    }
    __syncthreads();
    constexpr int QPR = D / 4;
    if ((int)threadIdx.x < HB * QPR) {
        const int mh = threadIdx.x / QPR, qd = threadIdx.x % QPR;
        float m = -INFINITY, l = 0.f, oo[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int wv = 0; wv < kAttnWaves; ++wv) {
            const float* r = rec + ((size_t)wv * HB + mh) * RECF;
            const float4 x = *reinterpret_cast<const float4*>(r + 4 * qd);
            const float o2[4] = {x.x, x.y, x.z, x.w};
            merge_run<4>(m, l, oo, r[D], r[D + 1], o2);
        }
        float* dst = p.part + ((size_t)slot * HB + mh) * RECF;
        *reinterpret_cast<float4*>(dst + 4 * qd) = make_float4(oo[0], oo[1], oo[2], oo[3]);
        if (qd == 0) *reinterpret_cast<float4*>(dst + D) = make_float4(m, l, 0.f, 0.f);
    }
    __syncthreads();
}


// ---------------------------------------------------------------- four query heads per KV head
// With four query heads per KV head the two rows of a row pair share one
// group block and split its data, not its heads: row hs takes the key tokens
// of position bit 3 equal to hs in each half (through the token xor: the
// lane's key words of position block hs ^ top) and the value channels
// 16hs .. 16hs+15 of each group, and both rows serve all four heads.  Every
// code is unpacked once, for four FMAs, and every lane loads only the rows
// (or the half cells) it uses: an FP16 unit takes 4 load phases, an INT4 or
// INT2 unit 2.
//
// The key state of a lane lists its heads in the order j ^ sg, sg = 2 in the
// lanes of the upper half of a row (top) and 0 otherwise, so that the first
// butterfly step of the reduce-scatter, which pairs lanes of opposite top,
// hands each lane two of the four heads without a select.  Value state (o,
// pm, the value weights) is in natural head order.
template <int D>
__device__ __forceinline__ void run_piece_g4(const AttnParams& p, const SeqUnits<D, 4>& su, int b, int h, int U0,
                                             int U1, int tbase, int slot, int* ctr, float* plds, float* rec) {
    constexpr int HB = 4;
    constexpr int S = D / 8;
    constexpr int R = 64 / S;          // rows per wave
    constexpr int NG = D / 32;         // value groups per token
    constexpr int GPI = R / 2;         // group blocks per unit: one per row pair
    constexpr int NTH = 16 / S;        // tokens per lane, head and key half after the reduce-scatter
    constexpr int RECF = D + 4;
    constexpr uint32_t ROWB = (uint32_t)S * 16u;
    constexpr int FIRST = S == 16 ? kDppRowMirror : kDppRowHalfMirror;   // partner of opposite top
    static_assert(GPI == SeqUnits<D, HB>::GPI, "unit geometry");

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = lane / S, L = lane % S;
    const int hs = row & 1, gslot = row >> 1;
    const int G = L % NG, tq = L / NG;
    const int fx = tok_xor(S, L);
    const bool top = L >= S / 2;
    const int sg = top ? 2 : 0;
    const int ws = hs ^ (top ? 1 : 0);   // the lane's key position block (bit 3 of the position)
    const int bh = b * p.Hkv + h;

    const size_t gpc = (size_t)(p.C / kGroup);
    const uint8_t* seg16 = p.pool[0] + (size_t)bh * p.cap[0] * gpc * group_bytes(16, D);
    const uint8_t* seg4 = p.pool[1] + (size_t)bh * p.cap[1] * gpc * group_bytes(4, D);
    const uint8_t* seg2 = p.pool[2] + (size_t)bh * p.cap[2] * gpc * group_bytes(2, D);

    // per-lane byte offsets inside a group block
    const uint32_t k16 = (uint32_t)(8 * ws) * ROWB;                 // FP16 key rows 16hh + 8ws + i
    const uint32_t v16 = (uint32_t)(32 + 2 * hs) * ROWB;            // FP16 value rows 32 + 4m + 2hs + k
    const uint32_t k4 = (uint32_t)(2 * ws) * ROWB;                  // INT4 key code rows 4 + 4hh + 2ws + i
    const uint32_t v4 = 16u * ROWB + 8u * (uint32_t)hs;             // INT4 value code rows 16 + m, bytes 8hs..
    const uint32_t psel = ws ? 0x07060302u : 0x05040100u;          // INT2 keys: the 16-bit half of block ws

    uint4 bufA[8], bufB[8];
    auto grab = [&]() -> int {
        int t = 0;
        if (lane == 0) t = atomicAdd(ctr, 1);
        return U0 + (__builtin_amdgcn_readfirstlane(t) - tbase);
    };
    auto unit_addr = [&](int U, uint32_t& voff) -> const uint8_t* {
        int k = 0, u = U;
        const uint8_t* base = seg16;
        uint32_t gb = (uint32_t)group_bytes(16, D);
        if (U >= su.ubase[2]) {
            k = 2; u = U - su.ubase[2]; base = seg2; gb = (uint32_t)group_bytes(2, D);
        } else if (U >= su.ubase[1]) {
            k = 1; u = U - su.ubase[1]; base = seg4; gb = (uint32_t)group_bytes(4, D);
        }
        const int segg = k == 0 ? su.segg[0] : (k == 1 ? su.segg[1] : su.segg[2]);
        const bool live = u * GPI + gslot < segg;
        voff = (live ? (uint32_t)gslot * gb : 0u) + (uint32_t)L * 16u;
        return base + (size_t)u * GPI * gb;
    };
    typedef unsigned u32x2_nt __attribute__((ext_vector_type(2)));
    auto ld8 = [](const uint8_t* a) -> uint2 {
        const u32x2_nt x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt*>(a));
        return make_uint2(x.x, x.y);
    };
    // The rows of load phase ph >= 1 of a unit of BITS-bit codes (phase 0,
    // whose unit may be of any segment, is load_first below).
    //   FP16: 1 = the lane's 8 key rows of half 1, 2 and 3 = its value rows of
    //         tokens tq + 4m, m = 0..3 and 4..7 (two channel octets each);
    //   INT4: 1 = value meta rows, then the lane's half cell of the 8 value
    //         code rows;
    //   INT2: 1 = value meta and value code rows.
    auto load_phase = [&](auto bits_tag, uint4* buf, const uint8_t* base, uint32_t voff, int ph) {
        constexpr int BITS = decltype(bits_tag)::value;
        const uint8_t* a = base + voff;
        if constexpr (BITS == 16) {
            if (ph == 1) {
#pragma unroll
                for (int i = 0; i < 8; ++i) buf[i] = ld16(a + k16 + (uint32_t)(16 + i) * ROWB);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    buf[i] = ld16(a + v16 + (uint32_t)(16 * (ph - 2) + 4 * (i >> 1) + (i & 1)) * ROWB);
            }
        } else if constexpr (BITS == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) buf[i] = ld16(a + (uint32_t)(12 + i) * ROWB);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint2 x = ld8(a + v4 + (uint32_t)(2 * i) * ROWB);
                const uint2 y = ld8(a + v4 + (uint32_t)(2 * i + 1) * ROWB);
                buf[4 + i] = make_uint4(x.x, x.y, y.x, y.y);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) buf[i] = ld16(a + (uint32_t)(8 + i) * ROWB);
        }
    };

    // Phase 0 of a unit of any segment k (wave-uniform) without a branch:
    // the rows are uniform (FP16 0-7, INT4 0-5 and 8-9, INT2 0-7) and the
    // lane's position-block offset applies to the FP16 rows and the INT4 code
    // rows.
    auto load_first = [&](uint4* buf, const uint8_t* base, uint32_t voff, int k) {
        const uint32_t va = voff + (k == 0 ? k16 : 0u);
        const uint32_t vb = voff + (k == 0 ? k16 : (k == 1 ? k4 : 0u));
        const uint32_t r6 = (k == 1 ? 8u : 6u) * ROWB;
#pragma unroll
        for (int i = 0; i < 4; ++i) buf[i] = ld16(base + va + (uint32_t)i * ROWB);
        buf[4] = ld16(base + vb + 4u * ROWB);
        buf[5] = ld16(base + vb + 5u * ROWB);
        buf[6] = ld16(base + r6 + vb);
        buf[7] = ld16(base + r6 + vb + ROWB);
    };
    auto seg_of = [&](int U_) { return U_ >= su.ubase[2] ? 2 : (U_ >= su.ubase[1] ? 1 : 0); };

    int U = grab();
    uint32_t vo = 0;
    const uint8_t* ub = seg16;
    if (U < U1) {
        ub = unit_addr(U, vo);
        load_first(bufA, ub, vo, seg_of(U));
    }

    // query channels 8L..8L+7 of the four heads, in key-state order
    uint32_t qw[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 qc =
            *reinterpret_cast<const uint4*>(p.q + ((size_t)b * p.Hq + h * p.hpk + p.hoff + (j ^ sg)) * D + 8 * L);
        qw[j][0] = qc.x; qw[j][1] = qc.y; qw[j][2] = qc.z; qw[j][3] = qc.w;
    }
    float qs[4][8];        // q * log2(e)/sqrt(d) in fp32 (INT-b keys), key-state order

    float M[2];            // running max of heads j ^ sg (j = 0, 1): uniform over the row pair's holders
    float lsum[2];         // this lane's share of their softmax denominators
    float o[4][16];        // value channels 32G + 16hs + c, natural head order
    float pm[4];           // sum_t p_t * mn_t over this lane's value tokens
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        M[j] = -INFINITY;
        lsum[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        pm[j] = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) o[j][c] = 0.f;
    }
    float sc[2][2 * NTH];  // key scores of heads j ^ sg: half 0, then half 1
    float pw[4][8];        // value weights of tokens tq + 4m: p (FP16), p * scale (INT-b)
    float koff[4];         // initial key accumulators: sum_j q_j mn_j
    float acc[4][8];       // key partial sums of the lane's 8 positions of one half

    // Reduce-scatter of one half over the S lanes of a row: the first step
    // pairs lanes of opposite top (same tokens, heads swapped), the others
    // halve the positions as the token xor dictates.
    auto take_half = [&](int hh) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 8; ++g) acc[j][g] += dpp<FIRST>(acc[j + 2][g]);
        if constexpr (S == 16) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int g = 0; g < 4; ++g) acc[j][g] += dpp<kDppRowHalfMirror>(acc[j][g + 4]);
#pragma unroll
                for (int g = 0; g < 2; ++g) acc[j][g] += dpp<kDppXor2>(acc[j][g + 2]);
                acc[j][0] += dpp<kDppXor1>(acc[j][1]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int g = 0; g < 4; ++g) acc[j][g] += dpp<kDppXor2>(acc[j][g + 4]);
#pragma unroll
                for (int g = 0; g < 2; ++g) acc[j][g] += dpp<kDppXor1>(acc[j][g + 2]);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < NTH; ++g) sc[j][hh * NTH + g] = acc[j][g];
    };
    // max over the lanes of the row pair that hold the same heads
    auto pair_max = [&](float v) {
        v = fmaxf(v, dpp<kDppXor1>(v));
        v = fmaxf(v, dpp<kDppXor2>(v));
        if constexpr (S == 16) {
            v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
            // the other row of the pair: v_permlane16_swap of v with itself
            // gives each pair of rows its even row's values in the first
            // result and its odd row's in the second
            const auto sw = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v),
                                                             __builtin_bit_cast(unsigned, v), false, false);
            v = fmaxf(__builtin_bit_cast(float, sw[0]), __builtin_bit_cast(float, sw[1]));
        } else {
            v = fmaxf(v, dpp<0x128>(v));   // row_ror:8, the other row of the pair
        }
        return v;
    };
    // the values of heads 0..3 (natural order) from x[j] of heads j ^ sg,
    // j = 0, 1, here and at the first-step partner (heads j ^ sg ^ 2)
    auto natural4 = [&](const float* x, float* nat) {
        const float y0 = dpp<FIRST>(x[0]), y1 = dpp<FIRST>(x[1]);
        nat[0] = top ? y0 : x[0];
        nat[1] = top ? y1 : x[1];
        nat[2] = top ? x[0] : y0;
        nat[3] = top ? x[1] : y1;
    };

    auto softmax_step = [&](bool valid) {
        float al[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float mloc = -INFINITY;
#pragma unroll
            for (int i = 0; i < 2 * NTH; ++i) {
                if (!valid) sc[j][i] = -INFINITY;
                mloc = fmaxf(mloc, sc[j][i]);
            }
            mloc = pair_max(mloc);
            const float Mn = fmaxf(M[j], mloc);
            al[j] = (Mn == -INFINITY) ? 1.f : fast_exp2(M[j] - Mn);
            M[j] = Mn;
            float pt[2 * NTH];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 2 * NTH; ++i) {
                pt[i] = valid ? fast_exp2(sc[j][i] - Mn) : 0.f;
                psum += pt[i];
            }
            lsum[j] = __builtin_fmaf(lsum[j], al[j], psum);
            // slot of token t in the value layout: (t & 3) * 8 + (t >> 2)
            float* pl = plds + (gslot * HB + (j ^ sg)) * 32;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int g = 0; g < NTH; ++g) {
                    const int t = 16 * hh + 8 * hs + ((g ^ fx) & 7);
                    pl[(t & 3) * 8 + (t >> 2)] = pt[hh * NTH + g];
                }
        }
        // the value state is rescaled only when some head's maximum rose
        // (the factor is exactly 1 otherwise)
        if (__ballot(al[0] != 1.f || al[1] != 1.f)) {
            float an[4];
            natural4(al, an);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pm[j] *= an[j];
#pragma unroll
                for (int c = 0; c < 16; ++c) o[j][c] *= an[j];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float* pl = plds + (gslot * HB + j) * 32;
            const float4 pa = *reinterpret_cast<const float4*>(pl + tq * 8);
            const float4 pb = *reinterpret_cast<const float4*>(pl + tq * 8 + 4);
            pw[j][0] = pa.x; pw[j][1] = pa.y; pw[j][2] = pa.z; pw[j][3] = pa.w;
            pw[j][4] = pb.x; pw[j][5] = pb.y; pw[j][6] = pb.z; pw[j][7] = pb.w;
        }
    };

    // ---- INT-b pieces (codes converted to fp32 by v_cvt_f32_ubyte, once for the four heads)
    // The key weight of channel e and head j is q_j * s_e, formed where it
    // is used from the scale rows that stay in the phase buffer (a second
    // time for the second half), which keeps 32 weights out of the registers.
    auto key_meta = [&](const uint4* m4) {   // rows: scale lo, scale hi, min lo, min hi
        const float4 n0 = as_f4(m4[2]), n1 = as_f4(m4[3]);
        const float kmn[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float bias = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) bias = __builtin_fmaf(qs[j][e], kmn[e], bias);
            koff[j] = bias;
        }
    };
    auto key_scale = [](const uint4* m4, int ch) {
        const uint4 r = m4[ch >> 2];
        const uint32_t x = (ch & 3) == 0 ? r.x : (ch & 3) == 1 ? r.y : (ch & 3) == 2 ? r.z : r.w;
        return __builtin_bit_cast(float, x);
    };
    // the lane's 2 INT4 key rows of one half: word e of row ii holds channel
    // 4ii + e at its 8 positions g (nibble g)
    auto key_half_int4 = [&](const uint4* m4, const uint4* rows) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < 8; ++g) acc[j][g] = koff[j];
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const uint32_t wd[4] = {rows[ii].x, rows[ii].y, rows[ii].z, rows[ii].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = wd[e] & 0x0F0F0F0Fu, hi = (wd[e] >> 4) & 0x0F0F0F0Fu;
                const float c[8] = {cvt_ub<0>(lo), cvt_ub<0>(hi), cvt_ub<1>(lo), cvt_ub<1>(hi),
                                    cvt_ub<2>(lo), cvt_ub<2>(hi), cvt_ub<3>(lo), cvt_ub<3>(hi)};
                const float ks = key_scale(m4, 4 * ii + e);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float wq = qs[j][4 * ii + e] * ks;
#pragma unroll
                    for (int g = 0; g < 8; ++g) acc[j][g] = __builtin_fmaf(wq, c[g], acc[j][g]);
                }
            }
        }
    };
    // the 2 INT2 key rows of one half: word e of row ii holds channel 4ii + e
    // at positions 0..15 (bits 2f); the lane takes positions 8ws .. 8ws+7,
    // the 16-bit half ws of the word, pairing two words in one register
    auto key_half_int2 = [&](const uint4* m4, const uint4* rows) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < 8; ++g) acc[j][g] = koff[j];
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const uint32_t wd[4] = {rows[ii].x, rows[ii].y, rows[ii].z, rows[ii].w};
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
                // bytes: [word 2e2, half ws] [word 2e2+1, half ws]
                const uint32_t y = __builtin_amdgcn_perm(wd[2 * e2 + 1], wd[2 * e2], psel);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    // byte 0: position k, byte 1: k + 4 of word 2e2; bytes 2, 3 the same of word 2e2+1
                    const uint32_t z = (y >> (2 * k)) & 0x03030303u;
                    const float c0 = cvt_ub<0>(z), c1 = cvt_ub<1>(z), c2 = cvt_ub<2>(z), c3 = cvt_ub<3>(z);
                    const float sa = key_scale(m4, 4 * ii + 2 * e2), sb = key_scale(m4, 4 * ii + 2 * e2 + 1);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float wa = qs[j][4 * ii + 2 * e2] * sa, wb = qs[j][4 * ii + 2 * e2 + 1] * sb;
                        acc[j][k] = __builtin_fmaf(wa, c0, acc[j][k]);
                        acc[j][k + 4] = __builtin_fmaf(wa, c1, acc[j][k + 4]);
                        acc[j][k] = __builtin_fmaf(wb, c2, acc[j][k]);
                        acc[j][k + 4] = __builtin_fmaf(wb, c3, acc[j][k + 4]);
                    }
                }
            }
        }
    };
    auto value_meta = [&](const uint4* m4) {   // (scale, min) of tokens t_{2r}, t_{2r+1}
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float4 sm = as_f4(m4[m >> 1]);
            const float s = (m & 1) ? sm.z : sm.x;
            const float mn = (m & 1) ? sm.w : sm.y;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pm[j] = __builtin_fmaf(pw[j][m], mn, pm[j]);
                pw[j][m] *= s;
            }
        }
    };
    // token tq + 4m: dwords 2m, 2m + 1 of the buffer (channels 16hs + 8uu + f)
    auto values_int4 = [&](const uint4* rows) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint4 cw = rows[m >> 1];
            const uint32_t wd[2] = {(m & 1) ? cw.z : cw.x, (m & 1) ? cw.w : cw.y};
#pragma unroll
            for (int uu = 0; uu < 2; ++uu) {
                const uint32_t lo = wd[uu] & 0x0F0F0F0Fu, hi = (wd[uu] >> 4) & 0x0F0F0F0Fu;
                const float c[8] = {cvt_ub<0>(lo), cvt_ub<0>(hi), cvt_ub<1>(lo), cvt_ub<1>(hi),
                                    cvt_ub<2>(lo), cvt_ub<2>(hi), cvt_ub<3>(lo), cvt_ub<3>(hi)};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float wv = pw[j][m];
#pragma unroll
                    for (int g = 0; g < 8; ++g) o[j][8 * uu + g] = __builtin_fmaf(wv, c[g], o[j][8 * uu + g]);
                }
            }
        }
    };
    // row r: tokens t_{2r} (dwords 0, 1), t_{2r+1} (dwords 2, 3); dword u of a
    // token holds channels 16u .. 16u+15 of the group, the lane takes u = hs
    auto values_int2 = [&](const uint4* rows) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint4 cw = rows[m >> 1];
            const uint32_t x = (m & 1) ? (hs ? cw.w : cw.z) : (hs ? cw.y : cw.x);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // byte q: channel 4q + k
                const uint32_t z = (x >> (2 * k)) & 0x03030303u;
                const float c[4] = {cvt_ub<0>(z), cvt_ub<1>(z), cvt_ub<2>(z), cvt_ub<3>(z)};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float wv = pw[j][m];
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) o[j][4 * q4 + k] = __builtin_fmaf(wv, c[q4], o[j][4 * q4 + k]);
                }
            }
        }
    };

    // ---- FP16 pieces: the lane's 8 key rows of one half (q . k with v_dot2),
    // or its 8 value rows of tokens tq + 4m, m = 4mb .. 4mb + 3
    auto keys_fp16 = [&](const uint4* rows) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float a = __builtin_amdgcn_fdot2(as_h2(rows[i].x), as_h2(qw[j][0]), 0.f, false);
                a = __builtin_amdgcn_fdot2(as_h2(rows[i].y), as_h2(qw[j][1]), a, false);
                a = __builtin_amdgcn_fdot2(as_h2(rows[i].z), as_h2(qw[j][2]), a, false);
                a = __builtin_amdgcn_fdot2(as_h2(rows[i].w), as_h2(qw[j][3]), a, false);
                acc[j][i] = a;
            }
    };
    auto values_fp16 = [&](const uint4* rows, int mb) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int m = 4 * mb + (i >> 1), cb = 8 * (i & 1);
            const uint32_t wd[4] = {rows[i].x, rows[i].y, rows[i].z, rows[i].w};
            float f[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[2 * e] = lo_h(wd[e]);
                f[2 * e + 1] = hi_h(wd[e]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float pr = pw[j][m];
#pragma unroll
                for (int c = 0; c < 8; ++c) o[j][cb + c] = __builtin_fmaf(pr, f[c], o[j][cb + c]);
            }
        }
    };

    auto compute_phase = [&](auto bits_tag, int ph, const uint4* cur, bool valid) {
        constexpr int BITS = decltype(bits_tag)::value;
        if constexpr (BITS == 16) {
            if (ph < 2) {
                keys_fp16(cur);
                take_half(ph);
                if (ph == 1) {
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int i = 0; i < 2 * NTH; ++i) sc[j][i] *= p.qscale;
                    softmax_step(valid);
                }
            } else {
                values_fp16(cur, ph - 2);
            }
        } else {
            if (ph == 0) {
                key_meta(cur);
                if constexpr (BITS == 4) key_half_int4(cur, cur + 4);
                else key_half_int2(cur, cur + 4);
                take_half(0);
                if constexpr (BITS == 4) key_half_int4(cur, cur + 6);
                else key_half_int2(cur, cur + 6);
                take_half(1);
                softmax_step(valid);
            } else {
                value_meta(cur);
                if constexpr (BITS == 4) values_int4(cur + 4);
                else values_int2(cur + 4);
            }
        }
    };

    // ---- unit loop: as in the general path, loads one phase ahead in the
    // other buffer; every segment has an even phase count here
    auto run_unit = [&](auto bits_tag, const uint8_t* ub_, uint32_t vo_, int kn, const uint8_t* ubn, uint32_t von,
                        bool valid) {
        constexpr int BITS = decltype(bits_tag)::value;
        constexpr int NPH = BITS == 16 ? 4 : 2;
#pragma unroll
        for (int ph = 0; ph < NPH; ++ph) {
            uint4* cur = (ph & 1) ? bufB : bufA;
            uint4* nxt = (ph & 1) ? bufA : bufB;
            if (ph + 1 < NPH) load_phase(bits_tag, nxt, ub_, vo_, ph + 1);
            else load_first(nxt, ubn, von, kn);   // the next unit, or a stand-in re-read of this one
            __builtin_amdgcn_sched_barrier(0);
            compute_phase(bits_tag, ph, cur, valid);
        }
    };
    auto step = [&](auto bits_tag, int segg_k, int ubase_k) {
        constexpr int BITS = decltype(bits_tag)::value;
        const int Un = grab();
        uint32_t von = 0;   // no next unit: every lane re-reads the unit's first cell (one line per load)
        const uint8_t* ubn = ub;
        int kn = expert_of_bits(BITS);
        if (Un < U1) {
            ubn = unit_addr(Un, von);
            kn = seg_of(Un);
        }
        const bool valid = (U - ubase_k) * GPI + gslot < segg_k;
        run_unit(bits_tag, ub, vo, kn, ubn, von, valid);
        U = Un;
        ub = ubn;
        vo = von;
    };
    {
        const int end = min(U1, su.ubase[0] + su.nu[0]);
        while (U < end) step(std::integral_constant<int, 16>{}, su.segg[0], su.ubase[0]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qs[j][2 * e] = lo_h(qw[j][e]) * p.qscale;
            qs[j][2 * e + 1] = hi_h(qw[j][e]) * p.qscale;
        }
    {
        const int end = min(U1, su.ubase[1] + su.nu[1]);
        while (U < end) step(std::integral_constant<int, 4>{}, su.segg[1], su.ubase[1]);
    }
    {
        const int end = min(U1, su.ubase[2] + su.nu[2]);
        while (U < end) step(std::integral_constant<int, 2>{}, su.segg[2], su.ubase[2]);
    }

    // ---------------- merge the lanes and row pairs of each head
    float Mn4[4], ln4[4];
    natural4(M, Mn4);
#pragma unroll
    for (int j = 0; j < 4; ++j) ln4[j] = ((j >> 1) == (top ? 1 : 0)) ? lsum[j & 1] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float Mx = Mn4[j];
#pragma unroll
        for (int off = 2 * S; off < 64; off <<= 1) Mx = fmaxf(Mx, __shfl_xor(Mx, off));

        const float rs = (Mn4[j] == -INFINITY) ? 0.f : fast_exp2(Mn4[j] - Mx);
        float l = ln4[j] * rs;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) l += __shfl_xor(l, off);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            float v = (o[j][c] + pm[j]) * rs;
#pragma unroll
            for (int off = NG; off < S; off <<= 1) v += __shfl_xor(v, off);
#pragma unroll
            for (int off = 2 * S; off < 64; off <<= 1) v += __shfl_xor(v, off);
            o[j][c] = v;
        }
        if (gslot == 0 && tq == 0) {
            float* r = rec + ((size_t)wave * HB + j) * RECF;
            float4* o4 = reinterpret_cast<float4*>(r + 32 * G + 16 * hs);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                o4[c] = make_float4(o[j][4 * c], o[j][4 * c + 1], o[j][4 * c + 2], o[j][4 * c + 3]);
            if (G == 0 && hs == 0) {
                r[D] = Mx;
                r[D + 1] = l;
            }
        }
    }
    __syncthreads();
    constexpr int QPR = D / 4;
    if ((int)threadIdx.x < HB * QPR) {
        const int mh = threadIdx.x / QPR, qd = threadIdx.x % QPR;
        float m = -INFINITY, l = 0.f, oo[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int wv = 0; wv < kAttnWaves; ++wv) {
            const float* r = rec + ((size_t)wv * HB + mh) * RECF;
            const float4 x = *reinterpret_cast<const float4*>(r + 4 * qd);
            const float o2[4] = {x.x, x.y, x.z, x.w};
            merge_run<4>(m, l, oo, r[D], r[D + 1], o2);
        }
        float* dst = p.part + ((size_t)slot * HB + mh) * RECF;
        *reinterpret_cast<float4*>(dst + 4 * qd) = make_float4(oo[0], oo[1], oo[2], oo[3]);
        if (qd == 0) *reinterpret_cast<float4*>(dst + D) = make_float4(m, l, 0.f, 0.f);
    }
    __syncthreads();
}

}  // namespace

// Persistent workgroups of kAttnWaves wavefronts.  Workgroup w takes the cost
// range [w*T/G, (w+1)*T/G) of the end-to-end (sequence, head) streams (T
// in all) and, for every stream whose unit starts fall in it, runs
// those units as one piece and leaves the piece's partial at record
// (sequence*Hkv + head) + w.
template <int D, int HB>
__global__ __launch_bounds__(64 * kAttnWaves, kAttnWaves / 4) void attn_tile_kernel(AttnParams p) {
    __shared__ int ctr;
    __shared__ float plds_all[kAttnWaves][(64 / (D / 8)) * attn_heads_per_row(HB) * 32];
    __shared__ __align__(16) float rec[kAttnWaves * HB * (D + 4)];
    const int w = blockIdx.x;
    const int lane = threadIdx.x & 63;
    if (threadIdx.x == 0) ctr = 0;
    __syncthreads();
    // Split.  With at most 64 sequences one pass over seg_count gives the
    // total, the prefix offsets and this workgroup's first sequence;
    // otherwise a second pass finds the sequence.
    int total, off, incl = 0, v = 0;
    int cnt[3] = {0, 0, 0};
    if (p.B <= 64) {
        if (lane < p.B) {
#pragma unroll
            for (int k = 0; k < 3; ++k) cnt[k] = p.seg_count[lane * 3 + k];
            SeqUnits<D, HB> sl;
            sl.init_counts(p, cnt[0], cnt[1], cnt[2]);
            v = sl.cost * p.Hkv;
        }
        incl = wave_incl_sum(v);
        total = __builtin_amdgcn_readlane(incl, 63);
    } else {
        total = total_cost<D, HB>(p);
    }
    if (total == 0) return;
    const int G = used_workgroups(p, total);
    if (w >= G) return;
    const int lo = split_point(w, total, G);
    const int hi = split_point(w + 1, total, G);
    int b;
    SeqUnits<D, HB> su;
    if (p.B <= 64) {
        const unsigned long long hit = __ballot(lane < p.B && incl > lo);
        b = __builtin_ctzll(hit);
        off = __builtin_amdgcn_readlane(incl - v, b);
        su.init_counts(p, __builtin_amdgcn_readlane(cnt[0], b), __builtin_amdgcn_readlane(cnt[1], b),
                       __builtin_amdgcn_readlane(cnt[2], b));
    } else {
        b = seq_containing<D, HB>(p, lo, off);
        if (b >= p.B) return;
        su.init(p, b);
    }
    int h = (int)((unsigned)(lo - off) / (unsigned)su.cost);
    off += h * su.cost;
    float* plds = plds_all[threadIdx.x >> 6];
    int tbase = 0;   // tickets taken by earlier pieces
    while (off < hi) {
        const int U0 = su.first_at_or_after(lo - off);
        const int U1 = su.first_at_or_after(hi - off);
        if (U0 < U1) {
            if constexpr (HB == 4)
                run_piece_g4<D>(p, su, b, h, U0, U1, tbase, b * p.Hkv + h + w, &ctr, plds, rec);
            else
                run_piece<D, HB>(p, su, b, h, U0, U1, tbase, b * p.Hkv + h + w, &ctr, plds, rec);
            tbase += U1 - U0 + kAttnWaves;
        }
        off += su.cost;
        if (++h == p.Hkv) {
            h = 0;
            if (++b >= p.B) break;
            su.init(p, b);
        }
    }
}

// Merge the piece partials (and the fp16 tail) of one (sequence, KV head)
// into the outputs of its HB query heads.  The pieces of (b, h) are those of
// the workgroups owning its first and its last unit and every workgroup in
// between, at records (b*Hkv + h) + w.  512 threads: thread (hb, qd, tgi)
// owns channel quad qd of query head hb and merges pieces tgi, tgi + TG, ...
// online, with its loads batched so that they are in flight together; the TG
// threads of one (head, quad) are adjacent lanes, so their states then meet
// in a butterfly of lane exchanges.  All heads are merged at once.
//
// Finding the pieces takes a load of the segment counts and the split
// arithmetic, and the records can only be loaded after that.  When the
// streams have equal cost (one sequence, or sequences of equal mix) the first
// owner of stream bh is floor(bh*G/(B*Hkv)) up to rounding, so every thread
// first loads its share of the TG records from one below that guess on;
// when the true pieces lie inside that window (the common case) the merge
// uses them and waits for one round of loads instead of two.
template <int D, int HB>
__global__ __launch_bounds__(512) void attn_combine_kernel(AttnParams p) {
    constexpr int NT = 512;
    constexpr int QPR = D / 4;            // float4 quads per record
    constexpr int TG = NT / (QPR * HB);   // piece groups per (head, quad): adjacent lanes
    static_assert(TG >= 4 && TG <= 32 && (TG & (TG - 1)) == 0, "butterfly width");
    constexpr int BATCH = 2;
    __shared__ float ts[HB][4096];        // tail scores (log2 domain)
    __shared__ int s_range[2];
    const int bh = blockIdx.x;
    const int b = bh / p.Hkv, h = bh % p.Hkv;
    const int tid = threadIdx.x, tgi = tid % TG, qd = (tid / TG) % QPR, hb = tid / (TG * QPR);
    const int hq = h * p.hpk + p.hoff + hb;
    const int nslots = p.B * p.Hkv + p.G;   // records in the workspace (per query head of the group)
    const int wg = max(0, (int)(((long long)bh * p.G) / (p.B * p.Hkv)) - 1);
    float2 sml;
    float4 sov;
    {
        const int slot = min(bh + wg + tgi, nslots - 1);
        const float* rec = p.part + ((size_t)slot * HB + hb) * (D + 4);
        sml = *reinterpret_cast<const float2*>(rec + D);
        sov = *reinterpret_cast<const float4*>(rec + 4 * qd);
    }
    if (tid < 64) {
        int w0 = 0, np = 0;
        const int total = total_cost<D, HB>(p);
        if (total > 0) {
            SeqUnits<D, HB> su;
            su.init(p, b);
            if (su.units > 0) {
                const int G = used_workgroups(p, total);
                const int first = seq_offset<D, HB>(p, b) + h * su.cost;
                const int last = first + su.unit_start(su.units - 1);
                w0 = owner_of(first, total, G);
                np = owner_of(last, total, G) - w0 + 1;
            }
        }
        if (tid == 0) {
            s_range[0] = w0;
            s_range[1] = np;
        }
    }
    if (p.tail_len > 0) {
        // scores of the tail tokens for every head of the group
        const uint16_t* tk = p.tail_k + (size_t)bh * p.tail_stride * D;
        for (int i = tid; i < HB * p.tail_len; i += NT) {
            const int th = i / p.tail_len, t = i % p.tail_len;
            const uint16_t* qp = p.q + ((size_t)b * p.Hq + h * p.hpk + p.hoff + th) * D;
            float s = 0.f;
            for (int c = 0; c < D; ++c)
                s = __builtin_fmaf((float)__builtin_bit_cast(_Float16, qp[c]),
                                   (float)__builtin_bit_cast(_Float16, tk[(size_t)t * D + c]), s);
            ts[th][t] = s * p.qscale;
        }
    }
    __syncthreads();
    const int w0 = s_range[0], npiece = s_range[1];
    const bool spec = w0 >= wg && w0 + npiece <= wg + TG;    // all pieces inside the loaded window
    float m = -INFINITY, l = 0.f;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    if (spec) {
        // piece wg + tgi - w0 (a valid piece's slot is always below nslots)
        const int v = wg + tgi - w0;
        if (v >= 0 && v < npiece) {
            const float o2[4] = {sov.x, sov.y, sov.z, sov.w};
            merge_run<4>(m, l, o, sml.x, sml.y, o2);
        }
    } else for (int v0 = tgi; v0 < npiece; v0 += TG * BATCH) {
        float2 ml[BATCH];
        float4 ov[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int v = v0 + j * TG;
            const float* rec = p.part + ((size_t)(bh + w0 + (v < npiece ? v : v0)) * HB + hb) * (D + 4);
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
        const uint16_t* tv = p.tail_v + (size_t)bh * p.tail_stride * D + 4 * qd;
        for (int t = tgi; t < p.tail_len; t += TG) {
            float vf[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) vf[c] = (float)__builtin_bit_cast(_Float16, tv[(size_t)t * D + c]);
            merge_run<4>(m, l, o, ts[hb][t], 1.f, vf);
        }
    }
    // the TG states of this (head, quad): butterfly over adjacent lanes
#pragma unroll
    for (int off = 1; off < TG; off <<= 1) {
        const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
        const float o2[4] = {__shfl_xor(o[0], off), __shfl_xor(o[1], off), __shfl_xor(o[2], off),
                             __shfl_xor(o[3], off)};
        merge_run<4>(m, l, o, m2, l2, o2);
    }
    if (tgi == 0) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        *reinterpret_cast<float4*>(p.out + ((size_t)b * p.Hq + hq) * D + 4 * qd) =
            make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    }
}

hipError_t launch_attention(const AttnParams& ap, int D, int HB, hipStream_t st) {
    const dim3 grid(ap.G);
    const dim3 cgrid(ap.B * ap.Hkv);
#define MKV_ATTN_CASE(DD, HH)                                                          \
    if (D == DD && HB == HH) {                                                         \
        attn_tile_kernel<DD, HH><<<grid, 64 * kAttnWaves, 0, st>>>(ap);                \
        attn_combine_kernel<DD, HH><<<cgrid, 512, 0, st>>>(ap);                        \
    } else
    MKV_ATTN_CASE(128, 1) MKV_ATTN_CASE(128, 2) MKV_ATTN_CASE(128, 4)
    MKV_ATTN_CASE(64, 1) MKV_ATTN_CASE(64, 2) MKV_ATTN_CASE(64, 4)
    return hipErrorInvalidValue;
#undef MKV_ATTN_CASE
    return hipGetLastError();
}

}  // namespace mkv
