// mmb_generic.hip -- the generic path: one thread per output element, fp32
// accumulation, any shape and any alignment.  It serves the calls the MFMA
// tiles cannot take even through packed copies: C or OC above 2^22 (beyond
// the tiles' 32-bit slab offsets), or a buffer not aligned to its element
// size.
//
// Operation: llm.c page "dev/cuda/matmul_backward.cu" -- the dinp and
// dweight GEMMs of matmul_backward1 (beta = 1) and the one-thread-per-channel
// bias kernel matmul_backward_bias_kernel_naive (assigning dbias); and the
// forward product out = inp . W^T + bias that the launcher's comments recall.
#include "mmb_internal.h"
#include "mmb_numeric.h"

namespace mmb {
namespace {

constexpr int kBlock = 256;

// dinp[r,i] = old + sum_o dout[r,o] * weight[o,i]; block = one row r and 256
// consecutive i, so weight reads coalesce and dout[r,o] is a broadcast.
template <typename T>
__global__ __launch_bounds__(kBlock) void generic_dinp(T* __restrict__ dinp,
                                                       const T* __restrict__ dout,
                                                       const T* __restrict__ weight,
                                                       int C, int OC) {
    const long long r = blockIdx.y;
    const int i = blockIdx.x * kBlock + threadIdx.x;
    if (i >= C) return;
    const T* d = dout + r * OC;
    float acc = 0.f;
    for (int o = 0; o < OC; ++o)
        acc = fmaf(to_f32(d[o]), to_f32(weight[(long long)o * C + i]), acc);
    T* out = dinp + r * C + i;
    *out = from_f32<T>(to_f32(*out) + acc);
}

// dweight[o,i] = old + sum_r dout[r,o] * inp[r,i]; block = one channel o and
// 256 consecutive i.  SR: bf16 stochastic rounding (element (o0 + o, i), tag 1).
template <typename T, bool SR = false>
__global__ __launch_bounds__(kBlock) void generic_dweight(T* __restrict__ dweight,
                                                          const T* __restrict__ dout,
                                                          const T* __restrict__ inp,
                                                          int BT, int C, int OC, long long o0 = 0,
                                                          unsigned long long seed = 0) {
    const long long o = blockIdx.y;
    const int i = blockIdx.x * kBlock + threadIdx.x;
    if (i >= C) return;
    float acc = 0.f;
    for (long long r = 0; r < BT; ++r)
        acc = fmaf(to_f32(dout[r * OC + o]), to_f32(inp[r * C + i]), acc);
    T* out = dweight + o * C + i;
    if constexpr (SR)
        *out = T{(uint16_t)sr_bf16_element(to_f32(*out) + acc, seed, 1, (uint64_t)(o0 + o),
                                           (uint64_t)i)};
    else
        *out = from_f32<T>(to_f32(*out) + acc);
}

// dbias[o] = sum_r dout[r,o]: one thread per channel, reads coalesce along o.
template <typename T, bool SR = false>
__global__ __launch_bounds__(kBlock) void generic_dbias(T* __restrict__ dbias,
                                                        const T* __restrict__ dout,
                                                        int BT, int OC, unsigned long long seed = 0) {
    const int o = blockIdx.x * kBlock + threadIdx.x;
    if (o >= OC) return;
    float acc = 0.f;
    for (long long r = 0; r < BT; ++r) acc += to_f32(dout[r * OC + o]);
    if constexpr (SR)
        dbias[o] = T{(uint16_t)sr_bf16_element(acc, seed, 2, 0, (uint64_t)o)};
    else
        dbias[o] = from_f32<T>(acc);
}

// Forward: out[r,o] = sum_i inp[r,i] * weight[o,i] (+ bias[o]), assigned;
// block = one row r and 256 consecutive o (inp[r,i] is a broadcast).
template <typename T>
__global__ __launch_bounds__(kBlock) void generic_forward(T* __restrict__ out,
                                                          const T* __restrict__ inp,
                                                          const T* __restrict__ weight,
                                                          const T* __restrict__ bias,
                                                          int C, int OC) {
    const long long r = blockIdx.y;
    const int o = blockIdx.x * kBlock + threadIdx.x;
    if (o >= OC) return;
    const T* x = inp + r * C;
    const T* w = weight + (long long)o * C;
    float acc = 0.f;
    for (int i = 0; i < C; ++i) acc = fmaf(to_f32(x[i]), to_f32(w[i]), acc);
    if (bias != nullptr) acc += to_f32(bias[o]);
    out[r * OC + o] = from_f32<T>(acc);
}

template <typename T>
hipError_t launch_forward(void* out, const void* inp, const void* weight, const void* bias,
                          int BT, int C, int OC, hipStream_t s) {
    const unsigned gx = (unsigned)((OC + kBlock - 1) / kBlock);
    const int kRowsPerLaunch = 65535;   // grid.y limit
    for (int r0 = 0; r0 < BT; r0 += kRowsPerLaunch) {
        const int rows = BT - r0 < kRowsPerLaunch ? BT - r0 : kRowsPerLaunch;
        hipLaunchKernelGGL(generic_forward<T>, dim3(gx, rows), dim3(kBlock), 0, s,
                           (T*)out + (long long)r0 * OC, (const T*)inp + (long long)r0 * C,
                           (const T*)weight, (const T*)bias, C, OC);
    }
    return hipGetLastError();
}

template <typename T, bool SR = false>
hipError_t launch(void* dinp, void* dweight, void* dbias, const void* dout,
                  const void* inp, const void* weight, int BT, int C, int OC,
                  hipStream_t s, unsigned long long seed = 0) {
    const dim3 block(kBlock);
    const unsigned gx = (unsigned)((C + kBlock - 1) / kBlock);
    // grid.y is limited to 65535 by the hardware dispatcher: chunk the rows
    const int kRowsPerLaunch = 65535;
    for (int r0 = 0; r0 < BT; r0 += kRowsPerLaunch) {
        const int rows = BT - r0 < kRowsPerLaunch ? BT - r0 : kRowsPerLaunch;
        hipLaunchKernelGGL(generic_dinp<T>, dim3(gx, rows), block, 0, s,
                           (T*)dinp + (long long)r0 * C, (const T*)dout + (long long)r0 * OC,
                           (const T*)weight, C, OC);
    }
    for (int o0 = 0; o0 < OC; o0 += kRowsPerLaunch) {
        const int rows = OC - o0 < kRowsPerLaunch ? OC - o0 : kRowsPerLaunch;
        hipLaunchKernelGGL((generic_dweight<T, SR>), dim3(gx, rows), block, 0, s,
                           (T*)dweight + (long long)o0 * C, (const T*)dout + o0,
                           (const T*)inp, BT, C, OC, (long long)o0, seed);
    }
    if (dbias != nullptr)
        hipLaunchKernelGGL((generic_dbias<T, SR>), dim3((OC + kBlock - 1) / kBlock), block, 0, s,
                           (T*)dbias, (const T*)dout, BT, OC, seed);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_generic(int dtype, void* dinp, void* dweight, void* dbias,
                          const void* dout, const void* inp, const void* weight,
                          int BT, int C, int OC, hipStream_t s, bool sr,
                          unsigned long long seed) {
    if (dtype == 0) return launch<float>(dinp, dweight, dbias, dout, inp, weight, BT, C, OC, s);
    if (sr)
        return launch<bf16_t, true>(dinp, dweight, dbias, dout, inp, weight, BT, C, OC, s, seed);
    return launch<bf16_t>(dinp, dweight, dbias, dout, inp, weight, BT, C, OC, s);
}

hipError_t launch_fwd_generic(int dtype, void* out, const void* inp, const void* weight,
                              const void* bias, int BT, int C, int OC, hipStream_t s) {
    if (dtype == 0) return launch_forward<float>(out, inp, weight, bias, BT, C, OC, s);
    return launch_forward<bf16_t>(out, inp, weight, bias, BT, C, OC, s);
}

}  // namespace mmb
