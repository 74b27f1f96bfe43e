// mmb_pack.hip -- row-pitch copies for the MFMA path on shapes whose rows
// are not whole 16-byte vectors (C or OC not a multiple of 8 in bf16, 4 in
// fp32): the tiles read and write 16-byte vectors along rows, so such a
// tensor is copied into a zero-padded pitch first (pack) and, for the
// outputs, copied back afterwards (unpack).  HBM-bound copies, a row per
// block row: pack writes whole 16-byte vectors (the destination pitch is a
// multiple of the vector), unpack goes element by element (its destination
// rows are not vector aligned).  Source and destination buffers are 16-byte
// aligned.
#include "mmb_internal.h"

namespace mmb {
namespace {

constexpr int kCopyThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Output dword j of a vector whose source starts B bytes into the 32-byte
// window lo:hi (two aligned 16-byte loads): bytes B + 4j .. B + 4j + 3.
template <int B>
__device__ __forceinline__ u32x4 window(const u32x4& lo, const u32x4& hi) {
    const uint32_t w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    constexpr int K = B / 4, SUB = B % 4;
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = SUB ? __builtin_amdgcn_alignbyte(w[K + j + 1], w[K + j], SUB) : w[K + j];
    return o;
}

// Pack: one thread per 16-byte vector of a padded row.  Source row r starts
// at element r * ld_src, s elements past a 16-byte boundary (s is the same
// for the whole row, so the shift below is a uniform branch); a vector that
// lies inside the row's `cols` elements is cut out of two aligned 16-byte
// loads, the one holding the row end and the zero pad go element by element.
// The last row also goes element by element: there, the second aligned load
// of a vector could reach past the end of the source.
template <typename T>
__global__ __launch_bounds__(kCopyThreads) void pack_rows(T* __restrict__ dst, long long ld_dst,
                                                          const T* __restrict__ src,
                                                          long long ld_src, long long rows,
                                                          int cols) {
    constexpr int VEC = 16 / (int)sizeof(T);
    const long long nvec = ld_dst / VEC;   // ld_dst is a multiple of VEC
    for (long long r = blockIdx.y; r < rows; r += gridDim.y) {
        const long long a0 = r * ld_src;
        const int sb = (int)(a0 % VEC) * (int)sizeof(T);   // byte offset past alignment
        const bool vec_ok = r + 1 < rows && ld_src >= 2 * VEC;
        for (long long v = (long long)blockIdx.x * kCopyThreads + threadIdx.x; v < nvec;
             v += (long long)gridDim.x * kCopyThreads) {
            const long long c0 = v * VEC;
            u32x4 o;
            if (vec_ok && c0 + VEC <= cols) {
                const u32x4* p = (const u32x4*)(src + (a0 + c0 - sb / (int)sizeof(T)));
                const u32x4 lo = p[0], hi = p[1];
                switch (sb) {
                    case 0: o = lo; break;
                    case 2: o = window<2>(lo, hi); break;
                    case 4: o = window<4>(lo, hi); break;
                    case 6: o = window<6>(lo, hi); break;
                    case 8: o = window<8>(lo, hi); break;
                    case 10: o = window<10>(lo, hi); break;
                    case 12: o = window<12>(lo, hi); break;
                    default: o = window<14>(lo, hi); break;
                }
            } else {
                T e[VEC];
#pragma unroll
                for (int k = 0; k < VEC; ++k) e[k] = c0 + k < cols ? src[a0 + c0 + k] : T(0);
                o = __builtin_bit_cast(u32x4, e);
            }
            *(u32x4*)(dst + r * ld_dst + c0) = o;
        }
    }
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
    const dim3 g = copy_grid(rows, ld_dst / (16 / es));
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
