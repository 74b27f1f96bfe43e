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
// Cache-policy bit NT (non-temporal): for output tiles that nothing in the
// launch reads again, so that they do not displace the operand slabs that
// later tiles reuse in L2.
constexpr int kStreamOut = 2;
__device__ __forceinline__ void store16_agent(__amdgpu_buffer_rsrc_t r, uint32_t voff, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, 0, kAgentCoherent);
}
__device__ __forceinline__ f32x4 load16_agent(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kAgentCoherent));
}

// ---- output tile --------------------------------------------------------------
// Block (mb, nb) register r of lane l holds D[m0 + mb*32 + (l & 31)]
// [n0 + nb*32 + 8*(r/4) + 4*(l/32) + r%4] (m0, n0: the wave's block origin);
// D = old + acc, rounded once.
//
// The tile is staged through LDS, so that global memory sees whole rows:
// the old tile (BM x BN elements of T) is loaded with 16-byte vectors, one
// row of BN elements per BN * sizeof(T) / 16 lanes, into LDS (rows padded
// by 16 bytes so that the 32 rows of one MFMA output block fall on distinct
// banks); every lane adds its accumulators to the old values of its fragment
// positions (wave block at rows wm0.., columns wn0..) and rounds once in
// place; the tile then goes back in the same row-contiguous pattern.  Stored
// straight from the MFMA layout, one wave instruction touches 32 rows and 16
// or 32 bytes of each.  Rows >= M and 16-byte groups >= N are masked through
// out-of-range offsets (N is a multiple of the 16-byte group on this path).
// `smem` holds at least out_lds_bytes<T, BM, BN>() bytes; the call begins
// with a barrier, after which the caller's earlier LDS contents are dead.
template <typename T, int BM, int BN>
constexpr int out_pitch() { return BN * (int)sizeof(T) + 16; }
template <typename T, int BM, int BN>
constexpr int out_lds_bytes() { return BM * out_pitch<T, BM, BN>(); }

__device__ __forceinline__ void add_round_store(char* pos, const f32x4& v, float) {
    f32x4 o = *(const f32x4*)pos;
    o += v;
    *(f32x4*)pos = o;
}
__device__ __forceinline__ void add_round_store(char* pos, const f32x4& v, bf16_t) {
    const u32x2 old = *(const u32x2*)pos;
    f32x4 o = v;
    o[0] += __uint_as_float(old[0] << 16);
    o[1] += __uint_as_float(old[0] & 0xffff0000u);
    o[2] += __uint_as_float(old[1] << 16);
    o[3] += __uint_as_float(old[1] & 0xffff0000u);
    u32x2 w;
    w[0] = f32x2_to_bf16x2_bits(o[0], o[1]);
    w[1] = f32x2_to_bf16x2_bits(o[2], o[3]);
    *(u32x2*)pos = w;
}

// bf16 with stochastic rounding: the 4 values take bits 0..15, 16..31, ...
// of `bits` (one word of the element block, see sr_block).
__device__ __forceinline__ void add_round_store_sr(char* pos, const f32x4& v, uint64_t bits) {
    const u32x2 old = *(const u32x2*)pos;
    f32x4 o = v;
    o[0] += __uint_as_float(old[0] << 16);
    o[1] += __uint_as_float(old[0] & 0xffff0000u);
    o[2] += __uint_as_float(old[1] << 16);
    o[3] += __uint_as_float(old[1] & 0xffff0000u);
    u32x2 w;
    w[0] = sr_bf16_bits(o[0], (uint32_t)bits & 0xFFFFu) |
           (sr_bf16_bits(o[1], (uint32_t)(bits >> 16) & 0xFFFFu) << 16);
    w[1] = sr_bf16_bits(o[2], (uint32_t)(bits >> 32) & 0xFFFFu) |
           (sr_bf16_bits(o[3], (uint32_t)(bits >> 48) & 0xFFFFu) << 16);
    *(u32x2*)pos = w;
}

// Global 16-byte offsets of the epilogue's row-contiguous passes: thread tid
// moves group tid % CHUNKS of row tid / CHUNKS + ROWS_PER_PASS * i in pass i.
// Offsets are relative to out_rsrc(); rows >= M and groups >= N are masked.
template <typename T, int NT, int BM, int BN>
struct OutMap {
    static constexpr int VEC = 16 / (int)sizeof(T);   // elements per 16-byte group
    static constexpr int CHUNKS = BN / VEC;            // 16-byte groups per row
    static_assert(NT % CHUNKS == 0 && BM % (NT / CHUNKS) == 0, "whole rows per pass");
    static constexpr int ROWS_PER_PASS = NT / CHUNKS;
    static constexpr int PASSES = BM / ROWS_PER_PASS;
};
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(T* D, long long ldd, int M, int m0, int n0) {
    const long long base = (long long)m0 * ldd + n0;
    return make_rsrc(D + base, ((long long)M * ldd - base) * (long long)sizeof(T));
}
template <typename T, int NT, int BM, int BN>
__device__ __forceinline__ uint32_t out_off(long long ldd, int M, int N, int m0, int n0, int tid, int i) {
    typedef OutMap<T, NT, BM, BN> OM;
    const int ch = tid % OM::CHUNKS, row = tid / OM::CHUNKS + OM::ROWS_PER_PASS * i;
    return (uint32_t)((row * ldd + OM::VEC * ch) * (long long)sizeof(T)) |
           oob_if_ge(n0 + OM::VEC * ch, N) | oob_if_ge(m0 + row, M);
}

// Second half of the epilogue, once LDS holds the base tile (the old output,
// or the bias rows) and a barrier has published it: every lane adds its
// accumulators at its fragment positions and rounds once in place, then the
// tile goes out row-contiguously.  SR: stochastic rounding to bf16 with the
// elements' Philox bits under (seed, tag) instead of round to nearest.
template <typename T, int MB, int NB, int NT, int BM, int BN, bool SR = false>
__device__ __forceinline__ void add_round_write(T* D, long long ldd, int M, int N, int m0, int n0,
                                                const f32x16 (&acc)[MB][NB], char* smem, int tid,
                                                int lane, int wm0, int wn0, uint64_t seed = 0,
                                                uint64_t tag = 0) {
    static_assert(!SR || sizeof(T) == 2, "stochastic rounding is for bf16 outputs");
    typedef OutMap<T, NT, BM, BN> OM;
    constexpr int PITCH = out_pitch<T, BM, BN>();
    const auto r = out_rsrc(D, ldd, M, m0, n0);
    const int ch = tid % OM::CHUNKS, row0 = tid / OM::CHUNKS;
    const int lr = lane & 31, half = lane >> 5;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            uint64_t bits[4] = {0, 0, 0, 0};
            if constexpr (SR)
                sr_block(seed, tag, (uint64_t)(m0 + wm0 + mb * 32 + lr),
                         (uint64_t)(n0 + wn0 + nb * 32 + 4 * half), bits);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = wm0 + mb * 32 + lr, col = wn0 + nb * 32 + 8 * q + 4 * half;
                const f32x4 a = {acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1], acc[mb][nb][4 * q + 2],
                                 acc[mb][nb][4 * q + 3]};
                if constexpr (SR)
                    add_round_store_sr(smem + row * PITCH + (int)sizeof(T) * col, a, bits[q]);
                else
                    add_round_store(smem + row * PITCH + (int)sizeof(T) * col, a, T{});
            }
        }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < OM::PASSES; ++i) {
        const int row = row0 + OM::ROWS_PER_PASS * i;
        __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4*)(smem + row * PITCH + 16 * ch), r,
                                              out_off<T, NT, BM, BN>(ldd, M, N, m0, n0, tid, i), 0, 0);
    }
}

// beta = 1: D = old + acc.  With PRE > 0, passes 0 .. PRE-1 of the old tile
// were already loaded by the caller (pre[i], loaded from out_rsrc() at
// out_off(.., i)).
template <typename T, int MB, int NB, int NT, int BM, int BN, int PRE = 0, bool SR = false>
__device__ __forceinline__ void write_tile_lds(T* D, long long ldd, int M, int N, int m0, int n0,
                                               const f32x16 (&acc)[MB][NB], char* smem, int tid,
                                               int lane, int wm0, int wn0,
                                               const u32x4* pre = nullptr, uint64_t seed = 0,
                                               uint64_t tag = 0) {
    typedef OutMap<T, NT, BM, BN> OM;
    constexpr int PITCH = out_pitch<T, BM, BN>();
    constexpr int PASSES = OM::PASSES;
    static_assert(PRE >= 0 && PRE <= PASSES, "preloaded passes");
    const auto r = out_rsrc(D, ldd, M, m0, n0);
    const int ch = tid % OM::CHUNKS, row0 = tid / OM::CHUNKS;
    __syncthreads();
    // the preloaded passes go to LDS first, so that their registers are free
    // for the loads of the others
#pragma unroll
    for (int i = 0; i < PRE; ++i)
        *(u32x4*)(smem + (row0 + OM::ROWS_PER_PASS * i) * PITCH + 16 * ch) = pre[i];
    u32x4 v[PASSES];
#pragma unroll
    for (int i = PRE; i < PASSES; ++i)
        v[i] = buffer_load16(r, out_off<T, NT, BM, BN>(ldd, M, N, m0, n0, tid, i), 0);
#pragma unroll
    for (int i = PRE; i < PASSES; ++i)
        *(u32x4*)(smem + (row0 + OM::ROWS_PER_PASS * i) * PITCH + 16 * ch) = v[i];
    __syncthreads();
    add_round_write<T, MB, NB, NT, BM, BN, SR>(D, ldd, M, N, m0, n0, acc, smem, tid, lane, wm0, wn0,
                                               seed, tag);
}

// beta = 0 with a bias row (the forward product): D[m, n] = acc + bias[n],
// rounded once; bias == nullptr adds nothing.  Every LDS row of the tile
// starts as the bias slice [n0, n0 + BN), so the add/round pass is the one of
// the beta = 1 epilogue.  bias is 16-byte aligned and holds bias_len >= N
// elements, zero past N and whole 16-byte groups (a packed copy when N is
// not a multiple of the group): the buffer range checks whole dwords, so a
// range ending inside the last group would read its last bf16 pair as zero.
template <typename T, int MB, int NB, int NT, int BM, int BN>
__device__ __forceinline__ void write_tile_bias(T* D, long long ldd, int M, int N, int m0, int n0,
                                                const f32x16 (&acc)[MB][NB], char* smem, int tid,
                                                int lane, int wm0, int wn0, const T* bias,
                                                long long bias_len) {
    typedef OutMap<T, NT, BM, BN> OM;
    constexpr int PITCH = out_pitch<T, BM, BN>();
    const int ch = tid % OM::CHUNKS, row0 = tid / OM::CHUNKS;
    const auto rb = make_rsrc(bias + (bias ? n0 : 0),
                              bias ? (bias_len - n0) * (long long)sizeof(T) : 0);
    const u32x4 b = buffer_load16(rb, (uint32_t)(16 * ch) | oob_if_ge(n0 + OM::VEC * ch, N), 0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < OM::PASSES; ++i)
        *(u32x4*)(smem + (row0 + OM::ROWS_PER_PASS * i) * PITCH + 16 * ch) = b;
    __syncthreads();
    add_round_write<T, MB, NB, NT, BM, BN>(D, ldd, M, N, m0, n0, acc, smem, tid, lane, wm0, wn0);
}

// beta = 0 with the bias added in registers (the bf16 forward): D = acc +
// bias[n], rounded once, with no bias rows in LDS.  bv[nb][q] holds the 4
// bias values (bf16) of the lane's columns n0 + wn0 + nb*32 + 8q + 4*(lane/32)
// .. +3, loaded by load_bias_frags from a bias of bias_len elements as for
// write_tile_bias (zeros past N or without a bias); the
// tile then leaves LDS row-contiguously as in add_round_write, with
// non-temporal stores (measured 2-3 % faster on the forward; no change on
// the backward's epilogues, which keep the default policy).
template <int NB>
__device__ __forceinline__ void load_bias_frags(const bf16_t* bias, int N, long long bias_len, int n0,
                                                int wn0, int lane, u32x2 (&bv)[NB][4]) {
    const auto rb = make_rsrc(bias + (bias ? n0 : 0), bias ? (bias_len - n0) * 2 : 0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int col = wn0 + nb * 32 + 8 * q + 4 * (lane >> 5);
            bv[nb][q] = __builtin_amdgcn_raw_buffer_load_b64(
                rb, (uint32_t)(2 * col) | oob_if_ge(n0 + col, N), 0, 0);
        }
}

template <int MB, int NB, int NT, int BM, int BN>
__device__ __forceinline__ void bias_round_write(bf16_t* D, long long ldd, int M, int N, int m0,
                                                 int n0, const f32x16 (&acc)[MB][NB], char* smem,
                                                 int tid, int lane, int wm0, int wn0,
                                                 const u32x2 (&bv)[NB][4]) {
    typedef OutMap<bf16_t, NT, BM, BN> OM;
    constexpr int PITCH = out_pitch<bf16_t, BM, BN>();
    const auto r = out_rsrc(D, ldd, M, m0, n0);
    const int ch = tid % OM::CHUNKS, row0 = tid / OM::CHUNKS;
    const int lr = lane & 31, half = lane >> 5;
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = wm0 + mb * 32 + lr, col = wn0 + nb * 32 + 8 * q + 4 * half;
                const u32x2 b = bv[nb][q];
                const float o0 = acc[mb][nb][4 * q] + __uint_as_float(b[0] << 16);
                const float o1 = acc[mb][nb][4 * q + 1] + __uint_as_float(b[0] & 0xffff0000u);
                const float o2 = acc[mb][nb][4 * q + 2] + __uint_as_float(b[1] << 16);
                const float o3 = acc[mb][nb][4 * q + 3] + __uint_as_float(b[1] & 0xffff0000u);
                u32x2 w;
                w[0] = f32x2_to_bf16x2_bits(o0, o1);
                w[1] = f32x2_to_bf16x2_bits(o2, o3);
                *(u32x2*)(smem + row * PITCH + 2 * col) = w;
            }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < OM::PASSES; ++i) {
        const int row = row0 + OM::ROWS_PER_PASS * i;
        __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4*)(smem + row * PITCH + 16 * ch), r,
                                              out_off<bf16_t, NT, BM, BN>(ldd, M, N, m0, n0, tid, i),
                                              0, kStreamOut);
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
// the bits do not depend on which split arrives last.  The whole of p_0 is
// fetched at once (into the accumulators, whose values were published), then
// each further partial in batches of up to 16 groups of 4 floats, so that one
// partial costs about one round trip to memory.
template <int MB, int NB, int NT>
__device__ __forceinline__ void sum_partials(const float* w0, int splits, int tile_floats,
                                             f32x16 (&acc)[MB][NB], int tid) {
    constexpr int NG = MB * NB * 4;          // 4-float groups per thread
    constexpr int BATCH = NG > 16 ? 16 : NG;
    static_assert(NG % BATCH == 0, "whole batches");
    f32x4 sum[NG];
    {
        const auto r = make_rsrc(w0, (long long)tile_floats * 4);
#pragma unroll
        for (int g = 0; g < NG; ++g) sum[g] = load16_agent(r, (uint32_t)((g * NT + tid) * 16));
    }
    for (int sp = 1; sp < splits; ++sp) {
        const auto r = make_rsrc(w0 + (long long)sp * tile_floats, (long long)tile_floats * 4);
#pragma unroll
        for (int b0 = 0; b0 < NG; b0 += BATCH) {
            f32x4 v[BATCH];
#pragma unroll
            for (int g = 0; g < BATCH; ++g)
                v[g] = load16_agent(r, (uint32_t)(((b0 + g) * NT + tid) * 16));
#pragma unroll
            for (int g = 0; g < BATCH; ++g) sum[b0 + g] += v[g];
        }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int q = g & 3, blk = g >> 2;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[blk / NB][blk % NB][4 * q + e] = sum[g][e];
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
