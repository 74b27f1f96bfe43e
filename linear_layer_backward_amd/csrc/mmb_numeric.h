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

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
    return bf16_t{(uint16_t)f32_to_bf16_bits(x)};
}

}  // namespace mmb
