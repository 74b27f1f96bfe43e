// mmb_tiles_bf16.hip -- bf16-storage / fp32-accumulate MFMA tiles of the
// linear-layer backward pass (dinp and dweight GEMMs with beta = 1, dbias
// fused into the dweight units of output column tile 0), one launch.
//
// Operation: llm.c page "dev/cuda/matmul_backward.cu", launcher
// matmul_backward1 (the two GEMMs) and the bias kernels (column sums of dout).
//
// gfx950 design (one workgroup = 4 wave64s = one 256 x 192 output tile; each
// wave owns a 128 x 96 quarter = 4 x 3 blocks of v_mfma_f32_32x32x16_bf16):
//  * Staging: operands go from HBM straight into LDS with buffer loads in LDS
//    mode (16 bytes per lane, no VGPR staging), through a ring of NS stages
//    of K depth 32 (32 KB each).  NS-1 stages are in flight while one is
//    consumed; each wave waits for its own loads with an explicit vmcnt and
//    one barrier per stage publishes the stage and retires the previous one.
//    These loads are issued from inline assembly because the compiler would
//    otherwise wait for every outstanding LDS load before any LDS read.
//  * A lane whose 16-byte vector lies outside the operand gets buffer offset
//    2^31 and writes zeros; rows past the end fall outside the buffer range.
//  * LDS keeps each operand in its memory orientation:
//      - dout for dinp (K-contiguous): [256 rows][32 k], 64-byte rows, chunk
//        c stored at c ^ ((row >> 1) & 3) ^ ((row >> 3) & 1); fragments are
//        ds_read_b128.
//      - weight, inp and dout-for-dweight (M/N-contiguous): [32 k][256
//        columns], 512-byte rows, chunk c stored at c ^ {0,10,4,14}[row & 3];
//        fragments are two ds_read_b64_tr_b16 per lane, the gfx950 LDS
//        transpose read (lane l of each 16-lane group receives element l%4
//        of the 8 bytes read by lane 4e + (l%16)/4, e = 0..3, i.e. four
//        consecutive K values of one column).  No VALU transposes.
//    Both swizzles keep the 8-lane groups of 16-byte reads and the 16-lane
//    groups of transpose reads on distinct banks.
//  * The MFMA "A" input is the N-side fragment, so each lane's accumulator
//    registers hold 4 consecutive output columns (8-byte bf16 epilogue).
//  * dbias: dweight units of column tile 0 also read their dout stage from
//    LDS and sum it in fp32; lanes l and l+32 combine by a shuffle and the
//    4 waves through LDS in a fixed order.
//  * Split K (dweight's K = B*T): fp32 partial tiles in the workspace, the
//    last arriver adds them in split order, adds the old output and rounds
//    once to bf16.
#include "mmb_tile_common.h"

namespace mmb {
namespace {

constexpr int BM = 256, BN = 192, BK = 32;
constexpr int WM = 128, WN = 96, MB = WM / 32, NB = WN / 32;
constexpr int NS = 4;            // LDS stages in the ring
constexpr int KC_PITCH = 64;     // K-contiguous LDS row: BK bf16
constexpr int MN_PITCH = 512;    // M/N-contiguous LDS row: up to 256 bf16
constexpr int REGION = 16384;    // one operand of one stage
constexpr int STAGE = 2 * REGION;
constexpr int LDS_BYTES = NS * STAGE;
constexpr int LOADS_PER_STAGE = 8;  // 16-byte-per-lane loads per wave per stage
static_assert(BM * KC_PITCH == REGION && BK * MN_PITCH == REGION, "regions");
static_assert(REGION / (4 * 1024) * 2 == LOADS_PER_STAGE, "loads per wave");

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// chunk XOR of M/N-contiguous rows, by row & 3: {0, 10, 4, 14}
__device__ __forceinline__ int sw_mn(int row) { return (0xE4A0 >> ((row & 3) << 2)) & 0xF; }
// chunk XOR of K-contiguous rows: distinct over any 8 rows of equal parity
// and any 16 rows of equal row % 4 (both 32- and 64-bank LDS)
__device__ __forceinline__ int sw_kc(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }

__device__ __forceinline__ bf16x4 tr_read(const char* region, int byte) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)((lds_char*)region + byte));
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(size_t)((const lds_char*)p);
}

// Buffer descriptor words (gfx9 raw buffer, dword3 0x00020000) over
// [base, base + bytes), num_records clamped below 2^31.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, long long bytes) {
    const uint64_t a = (uint64_t)base;
    const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffffLL ? 0x7fffffff : (int)bytes);
    return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), n, 0x00020000};
}

// 16 bytes per lane from buffer offset voff into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(i32x4 r, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(r), "s"(lds) : "memory", "m0");
}

// Wait until at most n of this wave's loads are outstanding (n uniform).
__device__ __forceinline__ void wait_loads(int n) {
    if (n >= 3 * LOADS_PER_STAGE) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else if (n >= 2 * LOADS_PER_STAGE) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (n >= LOADS_PER_STAGE) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// MFMA fragment (8 consecutive K of one row) of a K-contiguous region:
// lane l reads row xb + (l & 31), K chunk 2s + (l >> 5).
__device__ __forceinline__ bf16x8 frag_kc(const char* region, int xb, int s, int lane) {
    const int row = xb + (lane & 31);
    const int chunk = (2 * s + (lane >> 5)) ^ sw_kc(row);
    return __builtin_bit_cast(bf16x8, *(const u32x4*)(region + row * KC_PITCH + (chunk << 4)));
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
    const int nk = kt1 - kt0;

    const bf16_t* A = (const bf16_t*)p.dout;
    const bf16_t* Bp = (const bf16_t*)(AK ? p.weight : p.inp);
    bf16_t* D = (bf16_t*)(AK ? p.dinp : p.dweight);
    const long long lda = p.OC, ldb = p.C, ldd = p.C;
    const long long a_elems = (long long)p.BT * p.OC;
    const long long b_elems = AK ? (long long)p.OC * p.C : (long long)p.BT * p.C;
    const bool do_bias = !AK && p.dbias != nullptr && tile_n == 0;

    // Load geometry.  Wave w's i-th load of a region fills its 1 KB block
    // 4w + i; lane p lands at byte 16p of the block, so the lane fetches the
    // global vector that belongs there under the swizzle.
    //   K-contiguous A: block rows 16(4w+i) + p/4, physical chunk p%4
    //   M/N-contiguous: block rows 2(4w+i) + p/32, physical chunk p%32
    uint32_t a_off[4], b_off[4];
    int a_kc = 0;   // K-contiguous A: K offset (elements) of this lane's vector
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (AK) {
            const int row = 64 * wave + 16 * i + (lane >> 2);
            const int c = (lane & 3) ^ sw_kc(row);
            a_kc = 8 * c;
            a_off[i] = (uint32_t)(row * lda * 2 + c * 16);
        } else {
            const int row = 2 * (4 * wave + i) + (lane >> 5);
            const int c = (lane & 31) ^ sw_mn(row);
            const int col = m0 + 8 * c;
            a_off[i] = col < M ? (uint32_t)((row * lda + col) * 2) : kOOB;
        }
        {
            const int row = 2 * (4 * wave + i) + (lane >> 5);
            const int c = (lane & 31) ^ sw_mn(row);
            const int col = n0 + 8 * c;
            b_off[i] = (c < BN / 8 && col < N) ? (uint32_t)((row * ldb + col) * 2) : kOOB;
        }
    }
    const uint32_t smem_lds = lds_offset(smem);

    auto issue = [&](int kt, int stage) {
        const int k0 = kt * BK;
        const uint32_t la = smem_lds + stage * STAGE + wave * 4096;
        const uint32_t lb = la + REGION;
        const long long oa = AK ? (long long)m0 * lda + k0 : (long long)k0 * lda;
        const i32x4 ra = rsrc_words(A + oa, (a_elems - oa) * 2);
        // K tail inside a K-contiguous row: vectors at or past K read zeros
        const uint32_t kmask = AK ? (~(uint32_t)((k0 + a_kc - Kd) >> 31) & kOOB) : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(ra, a_off[i] | kmask, la + i * 1024);
        const long long ob = (long long)k0 * ldb;
        const i32x4 rb = rsrc_words(Bp + ob, (b_elems - ob) * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16(rb, b_off[i], lb + i * 1024);
    };

    f32x16 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    float bsum[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) bsum[x] = 0.f;
    // dbias: thread t sums column chunk t & 31 over K-rows (t >> 5) + 8j
    const int bias_c = tid & 31, bias_r = tid >> 5;
    const int bias_byte = bias_r * MN_PITCH + ((bias_c ^ sw_mn(bias_r)) << 4);

    const int wm0 = (wave & 1) * WM, wn0 = (wave >> 1) * WN;

    // Fragments of one 16-deep substep.
    struct Frag {
        bf16x8 a[NB];   // N side (MFMA input A)
        bf16x8 b[MB];   // M side (MFMA input B)
    };
    auto read_sub = [&](int stage, int k, Frag& f) {
        const char* sa = smem + stage * STAGE;
        const char* sb = sa + REGION;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) f.a[nb] = frag_mn(sb, wn0 + nb * 32, k, lane);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            f.b[mb] = AK ? frag_kc(sa, wm0 + mb * 32, k, lane) : frag_mn(sa, wm0 + mb * 32, k, lane);
    };
    auto bias_add = [&](int stage) {
        const char* sa = smem + stage * STAGE;
#pragma unroll
        for (int j = 0; j < BK / 8; ++j) {
            const u32x4 v = *(const u32x4*)(sa + bias_byte + j * 8 * MN_PITCH);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                bsum[2 * d] += __uint_as_float(v[d] << 16);
                bsum[2 * d + 1] += __uint_as_float(v[d] & 0xffff0000u);
            }
        }
    };
    auto mma_sub = [&](const Frag& f) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[nb], f.b[mb], acc[mb][nb],
                                                                      0, 0, 0);
    };

    // Ring of NS stages, NS-1 loaded ahead.  Iteration `it`: read the second
    // substep of stage it while the MFMAs of its first substep run; then one
    // barrier publishes stage it+1 (each wave has waited for its own loads
    // of it) and retires stage it-1 (all its fragments were read before),
    // whose buffer takes the loads of stage it+NS-1; then the first substep
    // of stage it+1 is read while the MFMAs of the second substep of it run.
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
        if (i < nk) issue(kt0 + i, i);
    Frag fa, fb;
    if (nk > 0) {
        const int issued = nk < NS - 1 ? nk : NS - 1;
        wait_loads((issued - 1) * LOADS_PER_STAGE);
        __syncthreads();
        read_sub(0, 0, fa);
        if (do_bias) bias_add(0);
    }
    for (int it = 0; it < nk; ++it) {
        read_sub(it % NS, 1, fb);
        mma_sub(fa);
        __builtin_amdgcn_sched_barrier(0);
        if (it + 1 < nk) {
            const int ahead = nk - it - 2 < NS - 3 ? nk - it - 2 : NS - 3;
            wait_loads(ahead * LOADS_PER_STAGE);
            __syncthreads();
            if (it + NS - 1 < nk) issue(kt0 + it + NS - 1, (it + NS - 1) % NS);
            __builtin_amdgcn_sched_barrier(0);
            read_sub((it + 1) % NS, 0, fa);
            if (do_bias) bias_add((it + 1) % NS);
        }
        mma_sub(fb);
        __builtin_amdgcn_sched_barrier(0);
    }

    // dbias of this unit's 256 columns: lanes l, l^32 share a column chunk;
    // the 4 waves meet in LDS once every wave is done with the ring
    float bias = 0.f;
    if (do_bias) {
        float* red = (float*)smem;
#pragma unroll
        for (int x = 0; x < 8; ++x) bsum[x] += __shfl_xor(bsum[x], 32);
        __syncthreads();
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
        float* wb = p.ws_bias + (long long)tile_m * g.splits * BM + tid;
        if (do_bias) publish_bias(wb + split * BM, bias);
        if (!arrive_last(p.counters + g.tile_base + tile, g.splits, s_flag)) return;
        sum_partials<MB, NB>(w0, g.splits, BM * BN, acc, tid);
        if (do_bias) bias = sum_bias(wb, g.splits, BM);
        if (tid == 0) p.counters[g.tile_base + tile] = 0;
    }

    write_tile<bf16_t, MB, NB>(D, ldd, M, N, m0 + wm0, n0 + wn0, acc, lane);
    if (do_bias && m0 + tid < M) ((bf16_t*)p.dbias)[m0 + tid] = from_f32<bf16_t>(bias);
}

__global__ __launch_bounds__(kThreads, 1) void mmb_tiles_bf16_kernel(TilesParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
    // the split-K ticket flag lives in the ring, used only after the K loop
    // (the dbias reduction uses the first 4 KB)
    int* s_flag = (int*)(smem + 8192);
    const int4 u = p.units[blockIdx.x];
    if (u.x == UNIT_DINP)
        run_unit<true>(p, p.g[UNIT_DINP], u, smem, s_flag);
    else
        run_unit<false>(p, p.g[UNIT_DWEIGHT], u, smem, s_flag);
}

}  // namespace

int tiles_bf16_bk() { return BK; }

hipError_t launch_tiles_bf16(const TilesParams& p, hipStream_t s) {
    if (p.n_units <= 0) return hipSuccess;
    hipLaunchKernelGGL(mmb_tiles_bf16_kernel, dim3(p.n_units), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace mmb
