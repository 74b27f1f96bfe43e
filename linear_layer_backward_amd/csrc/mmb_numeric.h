// mmb_numeric.h -- storage types and conversions of the HIP path.
//
// bfloat16 is the upper half of an IEEE binary32: widening is a 16-bit shift
// (exact); narrowing is gfx950's v_cvt_pk_bf16_f32, which rounds to nearest,
// ties to even, under the default round mode of a HIP kernel, and keeps NaN
// a NaN (branch-free: two values per instruction).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmb {

struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// lo in bits 0..15, hi in bits 16..31
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_bits_to_f32(x.bits); }

// ---- stochastic rounding to bf16 ---------------------------------------------
// The llm.c encoder page writes bf16 parameter gradients with stochastic
// rounding under a deterministic per-element seed.  The random bits here come
// from Philox-4x64 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011), keyed by (seed, tag):
// element (row, col) of a row-major gradient uses bits 16*(col%4).. of word
// (col%32)/8 of the block with counter (row, 2*(col/32) + (col/4)%2, 0, 0),
// so the 16 elements that one lane owns in a 32-column MFMA block share one
// block.  x rounds to the upper half of bits(x) + r16 (away from zero with
// probability discarded/65536); non-finite values round to nearest.

__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
        const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
        const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
        k0 += W0;
        k1 += W1;
    }
}

// The Philox block of the 16 elements of row `row`, columns
// 32*(col/32) + 8q + 4*half + e (q, e = 0..3), half = (col/4) % 2.
__device__ __forceinline__ void sr_block(uint64_t seed, uint64_t tag, uint64_t row, uint64_t col,
                                         uint64_t (&w)[4]) {
    w[0] = row;
    w[1] = 2 * (col / 32) + (col / 4) % 2;
    w[2] = 0;
    w[3] = 0;
    philox4x64_10(w, seed, tag);
}

// bf16 bits of x stochastically rounded with r16 (0 .. 65535).
__device__ __forceinline__ uint32_t sr_bf16_bits(float x, uint32_t r16) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7F800000u) == 0x7F800000u) return __builtin_bit_cast(uint16_t, (__bf16)x);
    return (u + r16) >> 16;
}

// One element on its own (dbias, the generic path): its block, its 16 bits.
__device__ __forceinline__ uint32_t sr_bf16_element(float x, uint64_t seed, uint64_t tag,
                                                    uint64_t row, uint64_t col) {
    uint64_t w[4];
    sr_block(seed, tag, row, col, w);
    return sr_bf16_bits(x, (uint32_t)(w[(col % 32) / 8] >> (16 * (col % 4))) & 0xFFFFu);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
    return bf16_t{(uint16_t)f32_to_bf16_bits(x)};
}

}  // namespace mmb
