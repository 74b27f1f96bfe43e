// mmb_numeric.h -- storage types and conversions of the HIP path.
//
// bfloat16 is the upper half of an IEEE binary32: widening is a 16-bit shift
// (exact); narrowing rounds to nearest, ties to even, on the bit pattern, and
// keeps NaN a quiet NaN.
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
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;  // NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_bits_to_f32(x.bits); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
    return bf16_t{(uint16_t)f32_to_bf16_bits(x)};
}

}  // namespace mmb
