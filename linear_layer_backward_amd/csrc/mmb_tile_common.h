// mmb_tile_common.h -- pieces shared by the MFMA tile kernels: vector types,
// buffer-resource loads with zero fill, the output epilogue, and the
// deterministic split-K finish (last arriver sums the partial tiles in split
// order).
#pragma once

#include "mmb_internal.h"
#include "mmb_numeric.h"

namespace mmb {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;            // 4 wave64s per workgroup
constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past any num_records

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zeros without touching memory (gfx9 descriptor, dword3 0x00020000).
// Callers keep every offset they use below 2^31 by rebasing `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long long bytes) {
    const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffffLL ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// ---- epilogue: four consecutive outputs, D = old + v, rounded once --------
__device__ __forceinline__ void store4(float* d, f32x4 v) {
    *(f32x4*)d = *(const f32x4*)d + v;
}
__device__ __forceinline__ void store4(bf16_t* d, f32x4 v) {
    const u32x2 old = *(const u32x2*)d;
    f32x4 o = v;
    o[0] += __uint_as_float(old[0] << 16);
    o[1] += __uint_as_float(old[0] & 0xffff0000u);
    o[2] += __uint_as_float(old[1] << 16);
    o[3] += __uint_as_float(old[1] & 0xffff0000u);
    u32x2 r;
    r[0] = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
    r[1] = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
    *(u32x2*)d = r;
}

// ---- split-K ---------------------------------------------------------------
// The MB x NB accumulator blocks of a workgroup, stored as 4-float groups in
// fragment order: thread tid's group q of block (mb, nb) lives at
// ((mb * NB + nb) * 4 + q) * 1024 + tid * 4, so each store instruction of a
// wave writes 1 KB contiguously.
template <int MB, int NB>
__device__ __forceinline__ void publish_partial(float* wt, const f32x16 (&acc)[MB][NB], int tid) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = {acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1],
                                 acc[mb][nb][4 * q + 2], acc[mb][nb][4 * q + 3]};
                *(f32x4*)(wt + ((mb * NB + nb) * 4 + q) * (kThreads * 4) + tid * 4) = v;
            }
}

// Take a ticket for the tile; true in every thread of the workgroup that
// arrives last.  The partials (and anything else) written before the call
// are visible to that workgroup.
__device__ __forceinline__ bool arrive_last(int* counter, int splits, int* s_flag) {
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) *s_flag = atomicAdd(counter, 1) == splits - 1;
    __syncthreads();
    const bool last = *s_flag;
    if (last) __threadfence();
    return last;
}

// acc <- p_0 + p_1 + ... + p_{S-1} (this workgroup's own partial taken from
// registers), the same order whichever split arrives last.
template <int MB, int NB>
__device__ __forceinline__ void sum_partials(const float* w0, int splits, int split, int tile_floats,
                                             f32x16 (&acc)[MB][NB], int tid) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int off = ((mb * NB + nb) * 4 + q) * (kThreads * 4) + tid * 4;
                const f32x4 mine = {acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1],
                                    acc[mb][nb][4 * q + 2], acc[mb][nb][4 * q + 3]};
                f32x4 s = split == 0 ? mine : *(const f32x4*)(w0 + off);
                for (int sp = 1; sp < splits; ++sp)
                    s += sp == split ? mine
                                     : *(const f32x4*)(w0 + (long long)sp * tile_floats + off);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[mb][nb][4 * q + r] = s[r];
            }
}

// Output of the MB x NB blocks: block (mb, nb) register r of lane l is
// D[m0 + mb*32 + (l & 31)][n0 + nb*32 + 8*(r/4) + 4*(l/32) + r%4].
template <typename T, int MB, int NB>
__device__ __forceinline__ void write_tile(T* D, long long ldd, int M, int N, int m0, int n0,
                                           const f32x16 (&acc)[MB][NB], int lane) {
    const int lr = lane & 31, half = lane >> 5;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = m0 + mb * 32 + lr;
        if (m >= M) continue;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + nb * 32 + 8 * q + 4 * half;
                if (n >= N) continue;
                const f32x4 v = {acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1],
                                 acc[mb][nb][4 * q + 2], acc[mb][nb][4 * q + 3]};
                store4(D + (long long)m * ldd + n, v);
            }
    }
}

}  // namespace mmb
