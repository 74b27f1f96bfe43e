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

// ---- masks without branches -------------------------------------------------
// kOOB when i >= n (so that offset | mask is out of any buffer range), else 0
__device__ __forceinline__ uint32_t oob_if_ge(int i, int n) {
    return ~(uint32_t)((i - n) >> 31) & kOOB;
}

// Agent-coherent (sc1) 16-byte store / load: visible to workgroups on other
// XCDs once the store has completed (s_waitcnt), with no L2 write-back or
// invalidate of unrelated lines.
constexpr int kAgentCoherent = 16;   // cache-policy bit SC1
__device__ __forceinline__ void store16_agent(__amdgpu_buffer_rsrc_t r, uint32_t voff, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, 0, kAgentCoherent);
}
__device__ __forceinline__ f32x4 load16_agent(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kAgentCoherent));
}

// ---- output tile --------------------------------------------------------------
// Block (mb, nb) register r of lane l holds D[m0 + mb*32 + (l & 31)]
// [n0 + nb*32 + 8*(r/4) + 4*(l/32) + r%4].  D = old + acc, rounded once.  All
// old values are loaded first (one round trip), then the sums are stored;
// rows >= M and columns >= N are masked through out-of-range offsets.
template <typename T> struct OutVec;
template <> struct OutVec<float> { typedef u32x4 type; };
template <> struct OutVec<bf16_t> { typedef u32x2 type; };

__device__ __forceinline__ u32x4 out_load(__amdgpu_buffer_rsrc_t r, uint32_t off, float) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 out_load(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16_t) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ void out_store(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 old,
                                          f32x4 v) {
    const f32x4 o = __builtin_bit_cast(f32x4, old) + v;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), r, off, 0, 0);
}
__device__ __forceinline__ void out_store(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 old,
                                          f32x4 v) {
    f32x4 o = v;
    o[0] += __uint_as_float(old[0] << 16);
    o[1] += __uint_as_float(old[0] & 0xffff0000u);
    o[2] += __uint_as_float(old[1] << 16);
    o[3] += __uint_as_float(old[1] & 0xffff0000u);
    u32x2 w;
    w[0] = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
    w[1] = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, 0);
}

template <typename T, int MB, int NB>
__device__ __forceinline__ void write_tile(T* D, long long ldd, int M, int N, int m0, int n0,
                                           const f32x16 (&acc)[MB][NB], int lane) {
    const int lr = lane & 31, half = lane >> 5;
    const long long base = (long long)m0 * ldd + n0;
    const auto r = make_rsrc(D + base, ((long long)M * ldd - base) * (long long)sizeof(T));
    auto offset = [&](int mb, int nb, int q) {
        const int m = mb * 32 + lr, n = nb * 32 + 8 * q + 4 * half;
        return (uint32_t)((m * ldd + n) * (long long)sizeof(T)) | oob_if_ge(m0 + m, M) |
               oob_if_ge(n0 + n, N);
    };
    // one row of blocks per batch of loads bounds the registers in flight
    constexpr int CH = 1;
#pragma unroll
    for (int mb0 = 0; mb0 < MB; mb0 += CH) {
        typename OutVec<T>::type old[CH][NB][4];
#pragma unroll
        for (int i = 0; i < CH; ++i)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int q = 0; q < 4; ++q) old[i][nb][q] = out_load(r, offset(mb0 + i, nb, q), T{});
#pragma unroll
        for (int i = 0; i < CH; ++i)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int mb = mb0 + i;
                    const f32x4 v = {acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1],
                                     acc[mb][nb][4 * q + 2], acc[mb][nb][4 * q + 3]};
                    out_store(r, offset(mb, nb, q), old[i][nb][q], v);
                }
    }
}

// ---- split-K ---------------------------------------------------------------
// A workgroup's partial tile (fp32), in fragment order: thread tid's group q
// of block (mb, nb) lives at float ((mb * NB + nb) * 4 + q) * 4 * NT + tid * 4
// (NT threads per workgroup), so each wave store writes 1 KB contiguously.
template <int MB, int NB, int NT>
__device__ __forceinline__ void publish_partial(float* wt, const f32x16 (&acc)[MB][NB], int tid) {
    const auto r = make_rsrc(wt, (long long)MB * NB * 4 * NT * 16);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = {acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1],
                                 acc[mb][nb][4 * q + 2], acc[mb][nb][4 * q + 3]};
                store16_agent(r, (uint32_t)((((mb * NB + nb) * 4 + q) * NT + tid) * 16), v);
            }
}

// Take the tile's ticket once this workgroup's agent-coherent stores have
// completed; true (in every thread) for the workgroup that arrives last.
__device__ __forceinline__ bool arrive_last(int* counter, int splits, int* s_flag) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) *s_flag = atomicAdd(counter, 1) == splits - 1;
    __syncthreads();
    return *s_flag;
}

// acc <- p_0 + p_1 + ... + p_{S-1}, every partial (this workgroup's own
// included) read back with agent-coherent loads and added in split order, so
// the bits do not depend on which split arrives last.  Up to 8 groups of 4
// floats are fetched per batch of loads.
template <int MB, int NB, int NT>
__device__ __forceinline__ void sum_partials(const float* w0, int splits, int tile_floats,
                                             f32x16 (&acc)[MB][NB], int tid) {
    constexpr int NG = MB * NB * 4;          // 4-float groups per thread
    constexpr int BATCH = NG >= 32 ? 8 : NG / 2;
    static_assert(NG % BATCH == 0, "whole batches");
#pragma unroll
    for (int b0 = 0; b0 < NG; b0 += BATCH) {
        f32x4 sum[BATCH];
        for (int sp = 0; sp < splits; ++sp) {
            const auto r = make_rsrc(w0 + (long long)sp * tile_floats, (long long)tile_floats * 4);
            f32x4 v[BATCH];
#pragma unroll
            for (int g = 0; g < BATCH; ++g)
                v[g] = load16_agent(r, (uint32_t)(((b0 + g) * NT + tid) * 16));
#pragma unroll
            for (int g = 0; g < BATCH; ++g) sum[g] = sp == 0 ? v[g] : sum[g] + v[g];
        }
#pragma unroll
        for (int g = 0; g < BATCH; ++g) {
            const int q = (b0 + g) & 3, blk = (b0 + g) >> 2;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[blk / NB][blk % NB][4 * q + e] = sum[g][e];
        }
    }
}

// dbias partials: thread tid's column of this split, and the ordered sum of
// all splits' values for the last arriver (agent-coherent, 4 bytes each).
__device__ __forceinline__ void publish_bias(float* wb, float v) {
    __hip_atomic_store(wb, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float sum_bias(const float* wb, int splits, int stride) {
    float s = 0.f;
    for (int sp = 0; sp < splits; ++sp) {
        const float v = __hip_atomic_load(wb + (long long)sp * stride, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        s = sp == 0 ? v : s + v;
    }
    return s;
}

}  // namespace mmb
