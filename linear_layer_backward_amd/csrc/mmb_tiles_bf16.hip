// mmb_tiles_bf16.hip -- bf16-storage / fp32-accumulate MFMA tiles of the
// linear-layer backward pass (dinp and dweight GEMMs with beta = 1, dbias
// fused into the dweight units of output column tile 0), one launch.
//
// Operation: llm.c page "dev/cuda/matmul_backward.cu", launcher
// matmul_backward1 (the two GEMMs) and the bias kernels (column sums of dout).
//
// gfx950 design (one workgroup = 4 wave64s = one 256 x 192 output tile; each
// wave owns a 128 x 96 quarter = 4 x 3 blocks of v_mfma_f32_32x32x16_bf16):
//  * Staging: global -> VGPR -> LDS, two LDS stages of K depth 64 (64 KB
//    each), loads of stage k+1 in flight during the MFMAs of stage k, one
//    barrier per stage.  All loads are raw buffer loads: a lane whose 16-byte
//    vector is outside the operand gets offset 2^31 and reads zeros, so the
//    loop has no branches.
//  * LDS keeps each operand in its memory orientation:
//      - dout for dinp (K-contiguous rows): [256 rows][64 k], 128-byte rows,
//        16-byte chunk c stored at c ^ (row & 7); MFMA fragments are one
//        ds_read_b128 per lane.
//      - weight, inp and dout-for-dweight (M/N-contiguous rows): [64 k][256
//        columns], 512-byte rows, chunk c stored at c ^ {0,10,4,14}[row & 3];
//        MFMA fragments are two ds_read_b64_tr_b16 per lane, the gfx950 LDS
//        transpose read (lane l of each 16-lane group receives element l%4
//        of the 8 bytes read by lane 4e + (l%16)/4, e = 0..3, giving four
//        consecutive K values of one column).  No VALU transposes.
//    Both swizzles keep the 16-lane groups of the transpose reads and the
//    8-lane groups of the 16-byte writes on distinct banks.
//  * The MFMA "A" input is the N-side fragment, so each lane's accumulator
//    registers hold 4 consecutive output columns (8-byte bf16 epilogue).
//  * dbias: dweight units of column tile 0 sum the dout vectors they stage
//    (fp32), combine lanes l and l+32 by a shuffle and the 4 waves through
//    LDS in a fixed order.
//  * Split K (dweight's K = B*T): fp32 partial tiles in the workspace, the
//    last arriver adds them in split order, adds the old output and rounds
//    once to bf16.
#include "mmb_tile_common.h"

namespace mmb {
namespace {

constexpr int BM = 256, BN = 192, BK = 64;
constexpr int WM = 128, WN = 96, MB = WM / 32, NB = WN / 32;
constexpr int KC_PITCH = 128;   // K-contiguous LDS row: BK bf16
constexpr int MN_PITCH = 512;   // M/N-contiguous LDS row: up to 256 bf16
constexpr int REGION = 32768;   // one operand of one stage
constexpr int STAGE = 2 * REGION;
constexpr int LDS_BYTES = 2 * STAGE;
static_assert(BM * KC_PITCH == REGION && BK * MN_PITCH == REGION, "regions");

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) char lds_char;

// chunk XOR of M/N-contiguous rows, by row & 3: {0, 10, 4, 14}
__device__ __forceinline__ int sw_mn(int row) { return (0xE4A0 >> ((row & 3) << 2)) & 0xF; }

__device__ __forceinline__ int kc_addr(int row, int chunk) {
    return row * KC_PITCH + ((chunk ^ (row & 7)) << 4);
}
__device__ __forceinline__ int mn_addr(int row, int chunk) {
    return row * MN_PITCH + ((chunk ^ sw_mn(row)) << 4);
}

__device__ __forceinline__ bf16x4 tr_read(const char* region, int byte) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)((lds_char*)region + byte));
}

// MFMA fragment (8 consecutive K of one row) of a K-contiguous region:
// lane l reads row xb + (l & 31), K chunk 2s + (l >> 5).
__device__ __forceinline__ bf16x8 frag_kc(const char* region, int xb, int s, int lane) {
    const int row = xb + (lane & 31);
    return __builtin_bit_cast(bf16x8, *(const u32x4*)(region + kc_addr(row, 2 * s + (lane >> 5))));
}

// The same fragment from an M/N-contiguous region with two transpose reads:
// lane L of group G = L/16 addresses row 16s + 8(G/2) + 4h + (L/4)%4, columns
// xb + 16(G%2) + 4(L%4) .. +3 (h = 0, 1).
__device__ __forceinline__ bf16x8 frag_mn(const char* region, int xb, int s, int lane) {
    const int G = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
    const int row = 16 * s + 8 * (G >> 1) + e;
    const int col = xb + 16 * (G & 1) + 4 * q;
    const int byte = row * MN_PITCH + ((((col >> 3) ^ sw_mn(row)) << 4) | (((col >> 2) & 1) << 3));
    const bf16x4 lo = tr_read(region, byte);
    const bf16x4 hi = tr_read(region, byte + 4 * MN_PITCH);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// AK: A (M side) is K-contiguous in memory (dinp: dout rows); otherwise it
// is M-contiguous (dweight: dout^T).  B (N side) is always N-contiguous
// (weight for dinp, inp for dweight).  Leading dimensions: dout OC, weight
// and inp C, output C.
template <bool AK>
__device__ __forceinline__ void run_unit(const TilesParams& p, const GemmPlan& g, int4 u,
                                         char* smem, int* s_flag) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int tile_m = u.y, tile_n = u.z, split = u.w;
    const int M = g.M, N = g.N, Kd = g.K;
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int kt0 = (int)((long long)split * g.kiters / g.splits);
    const int kt1 = (int)((long long)(split + 1) * g.kiters / g.splits);

    const bf16_t* A = (const bf16_t*)p.dout;
    const bf16_t* Bp = (const bf16_t*)(AK ? p.weight : p.inp);
    bf16_t* D = (bf16_t*)(AK ? p.dinp : p.dweight);
    const long long lda = p.OC, ldb = p.C, ldd = p.C;
    const long long a_elems = (long long)p.BT * p.OC;
    const long long b_elems = AK ? (long long)p.OC * p.C : (long long)p.BT * p.C;
    const bool do_bias = !AK && p.dbias != nullptr && tile_n == 0;

    // Staging geometry, fixed per thread.  Row masking comes from the buffer
    // range (every operand ends at its last valid K row, or for dinp's A at
    // row M); column masking from a precomputed out-of-range column offset,
    // so the load loop has no selects for the compiler to turn into branches.
    //   A, K-contiguous:  rows (tid>>3) + 32j, chunk tid&7 (K masked by AND)
    //   A, M-contiguous:  K-rows (tid>>5) + 8j, chunk tid&31
    //   B (waves 0-2):    K-rows tid/24 + 8j, chunk tid%24
    const int a_c = AK ? (tid & 7) : (tid & 31);
    const int a_r = AK ? (tid >> 3) : (tid >> 5);
    const bool b_on = wave < 3;                     // wave-uniform
    const int b_c = tid % 24, b_r = tid / 24;
    const uint32_t a_coff = AK ? (uint32_t)(a_c * 16)
                               : (m0 + 8 * a_c < M ? (uint32_t)((m0 + 8 * a_c) * 2) : kOOB);
    const uint32_t b_coff = n0 + 8 * b_c < N ? (uint32_t)((n0 + 8 * b_c) * 2) : kOOB;
    const uint32_t a_rstride = (uint32_t)((AK ? 32 : 8) * lda * 2);
    const uint32_t a_roff = (uint32_t)(a_r * lda * 2);
    const uint32_t b_rstride = (uint32_t)(8 * ldb * 2);
    const uint32_t b_roff = (uint32_t)(b_r * ldb * 2);

    u32x4 ra[8], rb[8];
    float bsum[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) bsum[x] = 0.f;

    auto load = [&](int kt) {
        const int k0 = kt * BK;
        {
            const long long off0 = AK ? (long long)m0 * lda + k0 : (long long)k0 * lda;
            const auto r = make_rsrc(A + off0, (a_elems - off0) * 2);
#pragma unroll
            for (int j = 0; j < 8; ++j) ra[j] = buffer_load16(r, a_roff + j * a_rstride + a_coff, 0);
            if constexpr (AK) {
                // K tail inside a row: zero the vectors at or past K
                const uint32_t keep = (uint32_t)((k0 + 8 * a_c - Kd) >> 31);
#pragma unroll
                for (int j = 0; j < 8; ++j) ra[j] &= keep;
            }
        }
        if (b_on) {
            const long long off0 = (long long)k0 * ldb;
            const auto r = make_rsrc(Bp + off0, (b_elems - off0) * 2);
#pragma unroll
            for (int j = 0; j < 8; ++j) rb[j] = buffer_load16(r, b_roff + j * b_rstride + b_coff, 0);
        }
    };

    auto store = [&](int stage) {
        char* sa = smem + stage * STAGE;
        char* sb = sa + REGION;
        if constexpr (AK) {
#pragma unroll
            for (int j = 0; j < 8; ++j) *(u32x4*)(sa + kc_addr(a_r + 32 * j, a_c)) = ra[j];
        } else {
            if (do_bias) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        bsum[2 * d] += __uint_as_float(ra[j][d] << 16);
                        bsum[2 * d + 1] += __uint_as_float(ra[j][d] & 0xffff0000u);
                    }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) *(u32x4*)(sa + mn_addr(a_r + 8 * j, a_c)) = ra[j];
        }
        if (b_on) {
#pragma unroll
            for (int j = 0; j < 8; ++j) *(u32x4*)(sb + mn_addr(b_r + 8 * j, b_c)) = rb[j];
        }
    };

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int wm0 = (wave & 1) * WM, wn0 = (wave >> 1) * WN;

    load(kt0);
    store(0);
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
        const int cur = (kt - kt0) & 1;
        const bool more = kt + 1 < kt1;
        if (more) load(kt + 1);
        const char* sa = smem + cur * STAGE;
        const char* sb = sa + REGION;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            bf16x8 fa[NB], fb[MB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) fa[nb] = frag_mn(sb, wn0 + nb * 32, s, lane);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                fb[mb] = AK ? frag_kc(sa, wm0 + mb * 32, s, lane) : frag_mn(sa, wm0 + mb * 32, s, lane);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[nb], fb[mb], acc[mb][nb],
                                                                          0, 0, 0);
        }
        if (more) store(cur ^ 1);
        __syncthreads();
    }

    // dbias of this unit's 256 columns: lanes l, l^32 share a column chunk;
    // the 4 waves meet in LDS (the stages are free after the last barrier)
    float bias = 0.f;
    if (do_bias) {
        float* red = (float*)smem;
#pragma unroll
        for (int x = 0; x < 8; ++x) bsum[x] += __shfl_xor(bsum[x], 32);
        if (lane < 32) {
#pragma unroll
            for (int x = 0; x < 8; ++x) red[wave * BM + lane * 8 + x] = bsum[x];
        }
        __syncthreads();
        bias = ((red[tid] + red[BM + tid]) + red[2 * BM + tid]) + red[3 * BM + tid];
    }

    if (g.splits > 1) {
        const int tile = tile_m * g.tiles_n + tile_n;
        float* w0 = p.ws + g.ws_base + (long long)tile * g.splits * (BM * BN);
        publish_partial<MB, NB>(w0 + (long long)split * (BM * BN), acc, tid);
        float* wb = p.ws_bias + (long long)tile_m * g.splits * BM;
        if (do_bias) wb[split * BM + tid] = bias;
        if (!arrive_last(p.counters + g.tile_base + tile, g.splits, s_flag)) return;
        sum_partials<MB, NB>(w0, g.splits, split, BM * BN, acc, tid);
        if (do_bias) {
            float s = split == 0 ? bias : wb[tid];
            for (int sp = 1; sp < g.splits; ++sp) s += sp == split ? bias : wb[sp * BM + tid];
            bias = s;
        }
        if (tid == 0) p.counters[g.tile_base + tile] = 0;
    }

    write_tile<bf16_t, MB, NB>(D, ldd, M, N, m0 + wm0, n0 + wn0, acc, lane);
    if (do_bias && m0 + tid < M) ((bf16_t*)p.dbias)[m0 + tid] = from_f32<bf16_t>(bias);
}

__global__ __launch_bounds__(kThreads, 1) void mmb_tiles_bf16_kernel(TilesParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
    __shared__ int s_flag;
    const int4 u = p.units[blockIdx.x];
    if (u.x == UNIT_DINP)
        run_unit<true>(p, p.g[UNIT_DINP], u, smem, &s_flag);
    else
        run_unit<false>(p, p.g[UNIT_DWEIGHT], u, smem, &s_flag);
}

}  // namespace

hipError_t launch_tiles_bf16(const TilesParams& p, hipStream_t s) {
    if (p.n_units <= 0) return hipSuccess;
    hipLaunchKernelGGL(mmb_tiles_bf16_kernel, dim3(p.n_units), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace mmb
