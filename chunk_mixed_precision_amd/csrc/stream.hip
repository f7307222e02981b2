// Copies for the streaming decode loop: one token's rows into the fp16 tail
// that attention reads, and a pool re-laid out for a larger capacity when a
// bitwidth segment outgrows it (MoQAE "Overall framework": the context is
// cut into equal chunks as it grows).  Plain strided row copies with
// 16-byte vector accesses.
#include "mkv_internal.h"
#include "mkv_kernels.h"

namespace mkv {

// Row r (of `rows`) of `row_bytes` bytes: src + r*spitch -> dst + r*dpitch.
// Every pointer, pitch and row length is a multiple of 16 bytes.
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint8_t* __restrict__ src, size_t spitch,
                                                        uint8_t* __restrict__ dst, size_t dpitch,
                                                        size_t row_bytes, int rows) {
    const size_t vec_per_row = row_bytes / 16;
    const size_t total = vec_per_row * (size_t)rows;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
        const size_t r = i / vec_per_row, v = i % vec_per_row;
        const uint4 x = *reinterpret_cast<const uint4*>(src + r * spitch + v * 16);
        *reinterpret_cast<uint4*>(dst + r * dpitch + v * 16) = x;
    }
}

hipError_t launch_copy_rows(const void* src, size_t spitch, void* dst, size_t dpitch, size_t row_bytes, int rows,
                            hipStream_t st) {
    const size_t total = row_bytes / 16 * (size_t)rows;
    if (total == 0) return hipSuccess;
    const size_t blocks = (total + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
    copy_rows_kernel<<<grid, 256, 0, st>>>(static_cast<const uint8_t*>(src), spitch, static_cast<uint8_t*>(dst),
                                           dpitch, row_bytes, rows);
    return hipGetLastError();
}

}  // namespace mkv
