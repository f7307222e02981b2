// Internal definitions shared by the kernels of libmkv.so (not part of the
// C ABI).  The packed-cache layout documented in include/mkv.h is expressed
// here once, as index functions used by both the writer (quantize/pack) and
// the reader (decode attention).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mkv {

constexpr int kGroup = 32;   // tokens per group block / values per quant group

// Expert index <-> bitwidth.
__host__ __device__ constexpr int bits_of_expert(int k) { return k == 0 ? 16 : (k == 1 ? 4 : 2); }
__host__ __device__ constexpr int expert_of_bits(int b) { return b == 16 ? 0 : (b == 4 ? 1 : (b == 2 ? 2 : -1)); }

// Rows (of S 16-byte cells) in each section of a group block.
// INT-b: [key meta 4][key codes 2b][value meta 4][value codes 2b]
// FP16:  [keys 32][values 32]
__host__ __device__ constexpr int kc_rows(int bits) { return bits == 16 ? 32 : 2 * bits; }
__host__ __device__ constexpr int vc_rows(int bits) { return bits == 16 ? 32 : 2 * bits; }
__host__ __device__ constexpr int meta_rows(int bits) { return bits == 16 ? 0 : 4; }
__host__ __device__ constexpr int group_rows(int bits) { return kc_rows(bits) + vc_rows(bits) + 2 * meta_rows(bits); }
__host__ __device__ constexpr int km_row0(int bits) { return 0; }
__host__ __device__ constexpr int kc_row0(int bits) { return meta_rows(bits); }
__host__ __device__ constexpr int vm_row0(int bits) { return meta_rows(bits) + kc_rows(bits); }
__host__ __device__ constexpr int vc_row0(int bits) { return 2 * meta_rows(bits) + kc_rows(bits); }

__host__ __device__ constexpr int lane_slots(int d) { return d / 8; }
__host__ __device__ constexpr size_t group_bytes(int bits, int d) {
    return (size_t)group_rows(bits) * lane_slots(d) * 16;
}

// Token permutation of the key rows/fields of lane slot L (S = d/8 slots).
// Field position r (0..31) of lane slot L holds token tok_of(S, L, r): the
// two halves r < 16 and r >= 16 keep their tokens (0..15 and 16..31) and
// inside a half the position is xor-ed with tok_xor(S, L).  The xor masks
// make the reduce-scatter of the q.k partial sums of one half over the S
// lanes of a row select-free: at every butterfly step each lane keeps the
// low half of its registers and its DPP partner's high half holds the same
// tokens.
__host__ __device__ constexpr int tok_xor(int S, int L) {
    return S == 16 ? ((L & 1) * 1) ^ (((L >> 1) & 1) * 2) ^ (((L >> 2) & 1) * 7) ^ (((L >> 3) & 1) * 12)
                   : ((L & 1) * 2) ^ (((L >> 1) & 1) * 4) ^ (((L >> 2) & 1) * 14);
}
__host__ __device__ constexpr int tok_of(int S, int L, int r) { return (r & 16) | ((r & 15) ^ tok_xor(S, L)); }

// Inclusive prefix sum over the 64 lanes of a wavefront: Hillis-Steele
// inside each row of 16 lanes (row shifts fill with 0), then lane 15 of rows
// 0 and 2 is added to rows 1 and 3 and lane 31 to rows 2 and 3 (row
// broadcasts).  Every lane must be active.
__device__ __forceinline__ int wave_incl_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return x;
}

// Sum over the 64 lanes, wave-uniform.
__device__ __forceinline__ int wave_sum(int x) { return __builtin_amdgcn_readlane(wave_incl_sum(x), 63); }

// Values: lane slot L covers value group G = L % NG and tokens tq + 4m,
// tq = L / NG, m = 0..7 (NG = d/32).
__host__ __device__ constexpr int vslot_of(int tq, int G, int NG) { return tq * NG + G; }

}  // namespace mkv
