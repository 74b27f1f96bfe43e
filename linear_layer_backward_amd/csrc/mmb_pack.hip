// mmb_pack.hip -- row-pitch copies for the MFMA path on shapes whose rows
// are not whole 16-byte vectors (C or OC not a multiple of 8 in bf16, 4 in
// fp32): the tiles read and write 16-byte vectors along rows, so such a
// tensor is copied into a zero-padded pitch first (pack) and, for the
// outputs, copied back afterwards (unpack).  HBM-bound element copies; a
// row per block row, consecutive threads on consecutive elements.
#include "mmb_internal.h"

namespace mmb {
namespace {

constexpr int kCopyThreads = 256;

template <typename T>
__global__ __launch_bounds__(kCopyThreads) void pack_rows(T* __restrict__ dst, long long ld_dst,
                                                          const T* __restrict__ src,
                                                          long long ld_src, long long rows,
                                                          int cols) {
    for (long long r = blockIdx.y; r < rows; r += gridDim.y)
        for (long long c = (long long)blockIdx.x * kCopyThreads + threadIdx.x; c < ld_dst;
             c += (long long)gridDim.x * kCopyThreads)
            dst[r * ld_dst + c] = c < cols ? src[r * ld_src + c] : T(0);
}

template <typename T>
__global__ __launch_bounds__(kCopyThreads) void unpack_rows(T* __restrict__ dst, long long ld_dst,
                                                            const T* __restrict__ src,
                                                            long long ld_src, long long rows,
                                                            int cols) {
    for (long long r = blockIdx.y; r < rows; r += gridDim.y)
        for (long long c = (long long)blockIdx.x * kCopyThreads + threadIdx.x; c < cols;
             c += (long long)gridDim.x * kCopyThreads)
            dst[r * ld_dst + c] = src[r * ld_src + c];
}

dim3 copy_grid(long long rows, long long cols) {
    const long long bx = (cols + kCopyThreads - 1) / kCopyThreads;
    return dim3((unsigned)(bx < 64 ? bx : 64), (unsigned)(rows < 32768 ? rows : 32768));
}

}  // namespace

hipError_t launch_pack(void* dst, long long ld_dst, const void* src, long long ld_src,
                       long long rows, int cols, int es, hipStream_t s) {
    if (rows <= 0 || ld_dst <= 0) return hipSuccess;
    const dim3 g = copy_grid(rows, ld_dst);
    if (es == 2)
        hipLaunchKernelGGL(pack_rows<uint16_t>, g, dim3(kCopyThreads), 0, s, (uint16_t*)dst, ld_dst,
                           (const uint16_t*)src, ld_src, rows, cols);
    else
        hipLaunchKernelGGL(pack_rows<uint32_t>, g, dim3(kCopyThreads), 0, s, (uint32_t*)dst, ld_dst,
                           (const uint32_t*)src, ld_src, rows, cols);
    return hipGetLastError();
}

hipError_t launch_unpack(void* dst, long long ld_dst, const void* src, long long ld_src,
                         long long rows, int cols, int es, hipStream_t s) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const dim3 g = copy_grid(rows, cols);
    if (es == 2)
        hipLaunchKernelGGL(unpack_rows<uint16_t>, g, dim3(kCopyThreads), 0, s, (uint16_t*)dst,
                           ld_dst, (const uint16_t*)src, ld_src, rows, cols);
    else
        hipLaunchKernelGGL(unpack_rows<uint32_t>, g, dim3(kCopyThreads), 0, s, (uint32_t*)dst,
                           ld_dst, (const uint32_t*)src, ld_src, rows, cols);
    return hipGetLastError();
}

}  // namespace mmb
