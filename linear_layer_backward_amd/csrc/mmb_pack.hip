// mmb_pack.hip -- row-pitch copies for the MFMA path on tensors whose rows
// are not whole 16-byte vectors (C or OC not a multiple of 8 in bf16, 4 in
// fp32) or whose address is not 16-byte aligned: the tiles read and write
// 16-byte vectors along rows, so such a tensor is copied into an aligned,
// zero-padded pitch first (pack) and, for the outputs, copied back
// afterwards (unpack).  HBM-bound copies, a row per block row, both moving
// whole 16-byte vectors cut out of aligned loads wherever a row allows.
// Packed buffers are 16-byte aligned with pitches a multiple of the vector;
// the caller's buffers are aligned to their element size.
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
// sb bytes past a 16-byte boundary (sb, taken from the row's address, is the
// same for the whole row, so the shift below is a uniform branch); a vector
// that lies inside the row's `cols` elements is cut out of two aligned
// 16-byte loads, the one holding the row end and the zero pad go element by
// element.  The first aligned load of a row may start up to 14 bytes before
// the row, inside the same 16-byte block (never on another page); the last
// row goes element by element, since there the second aligned load of a
// vector could reach past the end of the source.
template <typename T>
__global__ __launch_bounds__(kCopyThreads) void pack_rows(T* __restrict__ dst, long long ld_dst,
                                                          const T* __restrict__ src,
                                                          long long ld_src, long long rows,
                                                          int cols) {
    constexpr int VEC = 16 / (int)sizeof(T);
    const long long nvec = ld_dst / VEC;   // ld_dst is a multiple of VEC
    for (long long r = blockIdx.y; r < rows; r += gridDim.y) {
        const long long a0 = r * ld_src;
        const int sb = (int)((uintptr_t)(src + a0) % 16);   // byte offset past alignment
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

// Unpack: the mirror of pack, one thread per 16-byte aligned vector of a
// destination row.  Destination row r starts db bytes past a 16-byte
// boundary (uniform for the row), so its aligned vectors begin `lead`
// elements in; a vector wholly inside the row's `cols` elements is cut out
// of two aligned 16-byte loads of the packed source row (which starts
// aligned) and stored whole.  The elements before the first aligned vector
// and after the last one share their 16-byte blocks with the neighbouring
// rows and go element by element (one thread per row does them), as does a
// vector whose second source load would leave the padded source row.
template <typename T>
__global__ __launch_bounds__(kCopyThreads) void unpack_rows(T* __restrict__ dst, long long ld_dst,
                                                            const T* __restrict__ src,
                                                            long long ld_src, long long rows,
                                                            int cols) {
    constexpr int VEC = 16 / (int)sizeof(T);
    for (long long r = blockIdx.y; r < rows; r += gridDim.y) {
        T* drow = dst + r * ld_dst;
        const T* srow = src + r * ld_src;
        const int db = (int)((uintptr_t)drow % 16);
        const int lead = db ? (16 - db) / (int)sizeof(T) : 0;
        const long long lead_c = lead < cols ? lead : cols;
        const long long nfull = (cols - lead_c) / VEC;
        const int sb = (lead % VEC) * (int)sizeof(T);   // source bytes past alignment
        for (long long t = (long long)blockIdx.x * kCopyThreads + threadIdx.x; t <= nfull;
             t += (long long)gridDim.x * kCopyThreads) {
            if (t == nfull) {   // the row's partial blocks at both ends
                for (long long k = 0; k < lead_c; ++k) drow[k] = srow[k];
                for (long long k = lead_c + nfull * VEC; k < cols; ++k) drow[k] = srow[k];
                continue;
            }
            const long long e0 = lead_c + t * VEC;
            const long long a0 = e0 - sb / (int)sizeof(T);   // aligned source start
            if (sb != 0 && a0 + 2 * VEC > ld_src) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) drow[e0 + k] = srow[e0 + k];
                continue;
            }
            const u32x4* p = (const u32x4*)(srow + a0);
            const u32x4 lo = p[0];
            u32x4 o;
            switch (sb) {
                case 0: o = lo; break;
                case 2: o = window<2>(lo, p[1]); break;
                case 4: o = window<4>(lo, p[1]); break;
                case 6: o = window<6>(lo, p[1]); break;
                case 8: o = window<8>(lo, p[1]); break;
                case 10: o = window<10>(lo, p[1]); break;
                case 12: o = window<12>(lo, p[1]); break;
                default: o = window<14>(lo, p[1]); break;
            }
            *(u32x4*)(drow + e0) = o;
        }
    }
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
    const dim3 g = copy_grid(rows, cols / (16 / es) + 1);
    if (es == 2)
        hipLaunchKernelGGL(unpack_rows<uint16_t>, g, dim3(kCopyThreads), 0, s, (uint16_t*)dst,
                           ld_dst, (const uint16_t*)src, ld_src, rows, cols);
    else
        hipLaunchKernelGGL(unpack_rows<uint32_t>, g, dim3(kCopyThreads), 0, s, (uint32_t*)dst,
                           ld_dst, (const uint32_t*)src, ld_src, rows, cols);
    return hipGetLastError();
}

}  // namespace mmb
