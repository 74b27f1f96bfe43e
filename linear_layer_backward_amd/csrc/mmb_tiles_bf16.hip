// mmb_tiles_bf16.hip -- bf16-storage / fp32-accumulate MFMA tiles of the
// linear-layer backward pass (dinp and dweight GEMMs with beta = 1, dbias
// fused into the dweight units of output column tile 0), one launch.
//
// Operation: llm.c page "dev/cuda/matmul_backward.cu", launcher
// matmul_backward1 (the two GEMMs) and the bias kernels (column sums of dout).
//
// gfx950 design (one workgroup = 8 wave64s = one 256 x 256 output tile; wave
// w owns the 128 x 64 block at rows 128 (w & 1), columns 64 (w >> 1), i.e.
// 4 x 2 blocks of v_mfma_f32_32x32x16_bf16):
//  * Two waves per SIMD.  A single wave cannot keep the matrix unit busy:
//    between its own MFMAs it also has to issue the LDS reads, the loads and
//    their waits; a second wave on the same SIMD issues MFMAs while the
//    first one waits.
//  * Staging: operands go from HBM straight into LDS with buffer loads in LDS
//    mode (16 bytes per lane, no VGPR staging), two stages of K depth 64
//    (64 KB each).  K depth 64 makes every K-contiguous row one full 128-byte
//    line.  The loads of a stage are issued two stages ahead; each wave waits
//    for its own loads with an explicit vmcnt and one barrier per stage
//    publishes them.  The barrier sits before the last 16-deep substep of a
//    stage, so the next stage's first fragments are read while that
//    substep's MFMAs run.  The loads are issued from inline assembly because
//    the compiler would otherwise wait for every outstanding LDS load before
//    any LDS read.
//  * A lane whose 16-byte vector lies outside the operand gets buffer offset
//    2^31 and writes zeros; rows past the end fall outside the buffer range.
//  * LDS keeps each operand in its memory orientation:
//      - dout for dinp (K-contiguous): [256 rows][64 k], 128-byte rows, chunk
//        c stored at c ^ (row & 7) ^ ((row >> 3) & 1); fragments are
//        ds_read_b128.
//      - weight, inp and dout-for-dweight (M/N-contiguous): [64 k][256
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
//    8 waves through LDS in a fixed order.
//  * Split K (dweight's K = B*T): fp32 partial tiles in the workspace, the
//    last arriver adds them in split order, adds the old output and rounds
//    once to bf16.
#include "mmb_tile_common.h"

namespace mmb {
namespace {

constexpr int NT = 512, NW = NT / 64;          // 8 waves, two per SIMD
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WM = 128, WN = 64, MB = WM / 32, NB = WN / 32;
constexpr int KC_PITCH = 128;    // K-contiguous LDS row: BK bf16 (one 128-byte line)
constexpr int MN_PITCH = 512;    // M/N-contiguous LDS row: 256 bf16
constexpr int REGION = 32768;    // one operand of one stage
constexpr int STAGE = 2 * REGION;
constexpr int PF_SLOT = 2 * STAGE;          // 1 KB sink for the L2 prefetch loads
constexpr int LDS_BYTES = PF_SLOT + 1024;
constexpr int LOADS = REGION / (NW * 1024); // 1 KB loads per wave per operand per stage
static_assert(BM * KC_PITCH == REGION && BK * MN_PITCH == REGION, "regions");
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
static_assert(MB * NB * 16 * NT == BM * BN, "accumulators cover the tile");

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// chunk XOR of 512-byte M/N-contiguous rows, by row & 3: {0, 10, 4, 14}
__device__ __forceinline__ int sw_mn(int row) { return (0xE4A0 >> ((row & 3) << 2)) & 0xF; }
// chunk XOR of K-contiguous rows: distinct over any 8 consecutive rows and
// over the 8 rows of equal parity among any 16 (32- and 64-bank LDS)
__device__ __forceinline__ int sw_kc(int row) { return (row & 7) ^ ((row >> 3) & 1); }

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

// The compiler reserves m0 and warns when an asm statement clobbers it;
// these statements set it themselves right before the one instruction that
// reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from buffer offset voff into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(i32x4 r, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(r), "s"(lds) : "memory", "m0");
}

// 4 bytes per lane into LDS at lds + 4 * lane: only used to pull lines into
// the caches ahead of the real loads.
__device__ __forceinline__ void touch4(i32x4 r, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(r), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until this wave has at most N loads outstanding.
template <int N>
__device__ __forceinline__ void wait_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
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

    // Load geometry.  Wave w's i-th load of a region fills 1 KB block
    // LOADS * w + i; lane p lands at byte 16p of the block, so the lane
    // fetches the global vector that belongs there under the swizzle.
    //   K-contiguous A: block rows 8 * block + p/8, physical chunk p%8
    //   M/N-contiguous: block rows 2 * block + p/32, physical chunk p%32
    uint32_t a_off[LOADS], b_off[LOADS];
    int a_kc[LOADS];   // K-contiguous A: K offset of the lane's vector in load i
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int blk = LOADS * wave + i;
        const int row = 2 * blk + (lane >> 5);
        if constexpr (AK) {
            const int krow = 8 * blk + (lane >> 3);
            const int c = (lane & 7) ^ sw_kc(krow);
            a_kc[i] = 8 * c;
            a_off[i] = (uint32_t)(krow * lda * 2 + c * 16);
        } else {
            const int col = m0 + 8 * ((lane & 31) ^ sw_mn(row));
            a_off[i] = col < M ? (uint32_t)((row * lda + col) * 2) : kOOB;
        }
        const int col = n0 + 8 * ((lane & 31) ^ sw_mn(row));
        b_off[i] = col < N ? (uint32_t)((row * ldb + col) * 2) : kOOB;
    }
    // L2 prefetch geometry: one 4-byte touch per 128-byte line of a stage;
    // waves 0-3 cover A, waves 4-7 cover B, one load per wave per stage.
    //   K-contiguous A: row 64(w % 4) + p (one line per row)
    //   M/N-contiguous: row 16(w % 4) + p/4, line p%4 (4 lines per 512-byte row)
    const bool pf_a = wave < 4;
    uint32_t pf_off;
    {
        const int w4 = wave & 3;
        const int row = 16 * w4 + (lane >> 2);
        const int col = 64 * (lane & 3);
        if (pf_a) {
            if constexpr (AK) pf_off = (uint32_t)((64 * w4 + lane) * lda * 2);
            else pf_off = m0 + col < M ? (uint32_t)((row * lda + m0 + col) * 2) : kOOB;
        } else {
            pf_off = n0 + col < N ? (uint32_t)((row * ldb + n0 + col) * 2) : kOOB;
        }
    }
    const uint32_t smem_lds = lds_offset(smem);

    auto a_origin = [&](int kt) { return AK ? (long long)m0 * lda + kt * BK : (long long)kt * BK * lda; };
    // Stage kt into LDS buffer `stage`; a stage past the end (kt >= kt1)
    // still issues its loads, over an empty range, so that every wave's
    // count of outstanding loads follows one fixed pattern.
    auto issue = [&](int kt, int stage) {
        const bool live = kt < kt1;
        const int k0 = kt * BK;
        const uint32_t la = smem_lds + stage * STAGE + wave * (LOADS * 1024);
        const uint32_t lb = la + REGION;
        const long long oa = a_origin(kt);
        const i32x4 ra = rsrc_words(A + oa, live ? (a_elems - oa) * 2 : 0);
        // K tail inside a K-contiguous row: vectors at or past K read zeros
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const uint32_t kmask = AK ? oob_if_ge(k0 + a_kc[i], Kd) : 0u;
            dma16(ra, a_off[i] | kmask, la + i * 1024);
        }
        const long long ob = (long long)k0 * ldb;
        const i32x4 rb = rsrc_words(Bp + ob, live ? (b_elems - ob) * 2 : 0);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) dma16(rb, b_off[i], lb + i * 1024);
    };
    // Pull stage kt's lines into the caches (one load per wave; past the end
    // it reads nothing).
    auto prefetch = [&](int kt) {
        const bool live = kt < kt1;
        const long long oa = a_origin(kt);
        const long long ob = (long long)kt * BK * ldb;
        const i32x4 r = pf_a ? rsrc_words(A + oa, live ? (a_elems - oa) * 2 : 0)
                             : rsrc_words(Bp + ob, live ? (b_elems - ob) * 2 : 0);
        touch4(r, pf_off, smem_lds + PF_SLOT);
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
    // dbias: thread t sums column chunk t & 31 over K-rows (t >> 5) + 16j
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
        for (int j = 0; j < BK / 16; ++j) {
            const u32x4 v = *(const u32x4*)(sa + bias_byte + j * 16 * MN_PITCH);
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

    // Ring of two stages.  Loads per wave, in issue order: stage 0, stage 1,
    // touch of stage 2, then per iteration `it` the loads of stage it+2 and
    // the touch of stage it+3.  Iteration it runs the substeps of stage it
    // (buffer it & 1); before its last substep every wave waits for its own
    // loads of stage it+1 (only the newest touch may still fly), and one
    // barrier makes stage it+1 visible and retires buffer it & 1, which then
    // takes the loads of stage it+2 while the last substep runs.
    if (nk > 0) {
        issue(kt0, 0);
        issue(kt0 + 1, 1);
        prefetch(kt0 + 2);
        wait_loads<2 * LOADS + 1>();   // stage 0 landed (this wave's part)
        __syncthreads();
        Frag f0, f1;
        read_sub(0, 0, f0);
        for (int it = 0; it < nk; ++it) {
            const int cur = it & 1;
            if (do_bias) bias_add(cur);
            read_sub(cur, 1, f1);
            mma_sub(f0);
            read_sub(cur, 2, f0);
            mma_sub(f1);
            read_sub(cur, 3, f1);
            mma_sub(f0);
            __builtin_amdgcn_sched_barrier(0);
            wait_loads<1>();           // stage it+1 landed (this wave's part)
            __syncthreads();
            issue(kt0 + it + 2, cur);
            prefetch(kt0 + it + 3);
            __builtin_amdgcn_sched_barrier(0);
            if (it + 1 < nk) read_sub(cur ^ 1, 0, f0);
            mma_sub(f1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    wait_loads<0>();   // no load may land in LDS after the workgroup moves on

    // dbias of this unit's 256 columns: lanes l, l^32 share a column chunk;
    // the 8 waves meet in LDS once every wave is done with the ring
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
        if (tid < BM) {
            bias = red[tid];
#pragma unroll
            for (int w = 1; w < NW; ++w) bias += red[w * BM + tid];
        }
    }

    if (g.splits > 1) {
        const int tile = tile_m * g.tiles_n + tile_n;
        float* w0 = p.ws + g.ws_base + (long long)tile * g.splits * (BM * BN);
        publish_partial<MB, NB, NT>(w0 + (long long)split * (BM * BN), acc, tid);
        float* wb = p.ws_bias + (long long)tile_m * g.splits * BM + tid;
        if (do_bias && tid < BM) publish_bias(wb + split * BM, bias);
        if (!arrive_last(p.counters + g.tile_base + tile, g.splits, s_flag)) return;
        sum_partials<MB, NB, NT>(w0, g.splits, BM * BN, acc, tid);
        if (do_bias && tid < BM) bias = sum_bias(wb, g.splits, BM);
        if (tid == 0) p.counters[g.tile_base + tile] = 0;
    }

    write_tile<bf16_t, MB, NB>(D, ldd, M, N, m0 + wm0, n0 + wn0, acc, lane);
    if (do_bias && tid < BM && m0 + tid < M) ((bf16_t*)p.dbias)[m0 + tid] = from_f32<bf16_t>(bias);
}

__global__ __launch_bounds__(NT, 1) void mmb_tiles_bf16_kernel(TilesParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
    // the split-K ticket flag lives in the ring, used only after the K loop
    // (the dbias reduction uses the first 8 KB)
    int* s_flag = (int*)(smem + 8192);
    const int4 u = p.units[blockIdx.x];
    if (u.x == UNIT_DINP)
        run_unit<true>(p, p.g[UNIT_DINP], u, smem, s_flag);
    else
        run_unit<false>(p, p.g[UNIT_DWEIGHT], u, smem, s_flag);
}

}  // namespace

int tiles_bf16_bk() { return BK; }
int tiles_bf16_bn() { return BN; }

hipError_t launch_tiles_bf16(const TilesParams& p, hipStream_t s) {
    if (p.n_units <= 0) return hipSuccess;
    hipLaunchKernelGGL(mmb_tiles_bf16_kernel, dim3(p.n_units), dim3(NT), 0, s, p);
    return hipGetLastError();
}

}  // namespace mmb
