// mmb_tiles_bf16.hip -- bf16-storage / fp32-accumulate MFMA tiles of the
// linear-layer backward pass (dinp and dweight GEMMs with beta = 1, dbias
// fused into the dweight units of output column tile 0), one launch; and of
// the forward product out = inp . W^T + bias (both operands K-contiguous,
// beta = 0, the bias added in the epilogue), a launch of its own.
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
//  * Staging: each wave moves 8 KB of every 64 KB stage (K depth 64) from
//    HBM to registers with 16-byte buffer loads and from there to LDS; two
//    LDS stages plus the stage in flight in registers.  The loads of a stage
//    are spread over the whole iteration before the one that writes them to
//    LDS, so every load has an iteration to land and the memory pipeline
//    sees a steady stream instead of one burst per stage (a wave whose load
//    cannot issue stalls, MFMAs included).  K depth 64 makes every
//    K-contiguous row one full 128-byte line.  One barrier per stage, before
//    its last 16-deep substep, publishes the next stage, so that stage's
//    first fragments are read while the last substep's MFMAs run.
//  * A lane whose 16-byte vector lies outside the operand gets buffer offset
//    2^31 and loads zeros; rows past the end fall outside the buffer range.
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
//  * A unit that writes its own tile fetches the old tile inside the K
//    loop, in load slots that would otherwise fetch past the last stage, so
//    that the beta = 1 epilogue waits on no load.
#include <type_traits>

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
// the ring, or the whole output tile in the epilogue
constexpr int OUT_BYTES = out_lds_bytes<bf16_t, BM, BN>();
constexpr int LDS_BYTES = 2 * STAGE > OUT_BYTES ? 2 * STAGE : OUT_BYTES;
constexpr int LOADS = REGION / (NW * 1024); // 1 KB loads per wave per operand per stage
static_assert(BM * KC_PITCH == REGION && BK * MN_PITCH == REGION, "regions");
static_assert(LDS_BYTES <= 160 * 1024, "LDS");
static_assert(MB * NB * 16 * NT == BM * BN, "accumulators cover the tile");

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) char lds_char;

// chunk XOR of 512-byte M/N-contiguous rows, by row & 3: {0, 10, 4, 14}
__device__ __forceinline__ int sw_mn(int row) { return (0xE4A0 >> ((row & 3) << 2)) & 0xF; }
// chunk XOR of K-contiguous rows: distinct over any 8 consecutive rows and
// over the 8 rows of equal parity among any 16 (32- and 64-bank LDS)
__device__ __forceinline__ int sw_kc(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ bf16x4 tr_read(const char* region, int byte) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)((lds_char*)region + byte));
}

// Scheduling pattern of one substep (8 MFMAs): the two LDS stores behind the
// first two MFMAs, then two fragment reads after each MFMA from the third
// on, the two loads last.  Spreading the reads keeps the LDS queue short for
// the other wave on the SIMD; measured 4-5 % faster than the compiler's own
// order.
template <int READS>
__device__ __forceinline__ void interleave_substep() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        if (i < 2) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // LDS store
        if (i >= 2 && i - 2 < READS / 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS read
        if (i >= 6) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
    }
}

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

// The three GEMMs these tiles run, with the orientation of their operands in
// memory (leading dimensions: dout OC, weight and inp C):
//   DINP     D = dinp [BT,C]  += dout [BT,OC] . weight [OC,C]   A K-contiguous, B N-contiguous
//   DWEIGHT  D = dweight[OC,C] += dout^T . inp [BT,C]           A M-contiguous, B N-contiguous
//   FWD      D = out [BT,OC]   = inp [BT,C] . weight^T + bias   A K-contiguous, B K-contiguous
// (FWD: out = inp . W^T, the forward product whose gradients the other two are.)
enum class Op { DINP, DWEIGHT, FWD };

// SR: the output (dweight) and dbias are rounded stochastically (Philox bits
// under p.seed, tags 1 and 2) instead of to nearest.
template <Op OP, bool SR = false>
__device__ __forceinline__ void run_unit(const TilesParams& p, const GemmPlan& g, int4 u, int4 v,
                                         char* smem, int* s_flag) {
    static_assert(!SR || OP == Op::DWEIGHT, "stochastic rounding is for the parameter gradients");
    constexpr bool AK = OP != Op::DWEIGHT;   // A rows K-contiguous (dout rows, inp rows)
    constexpr bool BKC = OP == Op::FWD;      // B rows K-contiguous (weight rows)
    constexpr bool BETA1 = OP != Op::FWD;    // gradients accumulate; the forward assigns
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int tile_m = u.y, tile_n = u.z, split = u.w;
    const int M = g.M, N = g.N, Kd = g.K;
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    // K iterations [kt0, kt1) of a tile cut into `splits` units; the tile's
    // partial sums (if any) start at workspace slot `slot`
    const int kt0 = v.x, kt1 = v.y, splits = v.z, slot = v.w;
    const int nk = kt1 - kt0;

    const bf16_t* A = (const bf16_t*)(OP == Op::FWD ? p.inp : p.dout);
    const bf16_t* Bp = (const bf16_t*)(OP == Op::DWEIGHT ? p.inp : p.weight);
    bf16_t* D = (bf16_t*)(OP == Op::DINP ? p.dinp : OP == Op::DWEIGHT ? p.dweight : p.out);
    // row pitches: dout (out) rows ldo, the C-wide tensors' rows ldc
    const long long lda = OP == Op::FWD ? p.ldc : p.ldo, ldb = p.ldc, ldd = OP == Op::FWD ? p.ldo : p.ldc;
    const long long a_elems = (long long)p.BT * lda;
    const long long b_elems = OP == Op::DWEIGHT ? (long long)p.BT * ldb : (long long)p.OC * ldb;
    const bool do_bias = OP == Op::DWEIGHT && p.dbias != nullptr && tile_n == 0;

    // Load geometry.  Wave w's i-th load of a region fills 1 KB block
    // LOADS * w + i; lane p lands at byte 16p of the block, so the lane
    // fetches the global vector that belongs there under the swizzle.
    //   K-contiguous: block rows 8 * block + p/8, physical chunk p%8
    //   M/N-contiguous: block rows 2 * block + p/32, physical chunk p%32
    uint32_t a_off[LOADS], b_off[LOADS];
    int a_kc[LOADS], b_kc[LOADS];   // K-contiguous: K offset of the lane's vector in load i
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
        if constexpr (BKC) {
            const int krow = 8 * blk + (lane >> 3);
            const int c = (lane & 7) ^ sw_kc(krow);
            b_kc[i] = 8 * c;
            b_off[i] = (uint32_t)(krow * ldb * 2 + c * 16);
        } else {
            const int col = n0 + 8 * ((lane & 31) ^ sw_mn(row));
            b_kc[i] = 0;
            b_off[i] = col < N ? (uint32_t)((row * ldb + col) * 2) : kOOB;
        }
    }

    auto a_origin = [&](int kt) { return AK ? (long long)m0 * lda + kt * BK : (long long)kt * BK * lda; };
    auto b_origin = [&](int kt) { return BKC ? (long long)n0 * ldb + kt * BK : (long long)(kt * BK) * ldb; };
    // Global -> register staging of stage kt, chunk pair j (load j of each
    // operand).  A stage past the end (kt >= kt1) still issues its loads, over
    // an empty range (they return zeros), so that every wave's count of
    // outstanding loads follows one fixed pattern.
    u32x4 stg_a[LOADS], stg_b[LOADS];
    auto load_pair = [&](int kt, int j) {
        const bool live = kt < kt1;
        const int k0 = kt * BK;
        const long long oa = a_origin(kt);
        const auto ra = make_rsrc(A + oa, live ? (a_elems - oa) * 2 : 0);
        // K tail inside a K-contiguous row: vectors at or past K read zeros
        const uint32_t kmask = AK ? oob_if_ge(k0 + a_kc[j], Kd) : 0u;
        stg_a[j] = buffer_load16(ra, a_off[j] | kmask, 0);
        const long long ob = b_origin(kt);
        const auto rb = make_rsrc(Bp + ob, live ? (b_elems - ob) * 2 : 0);
        const uint32_t kmask_b = BKC ? oob_if_ge(k0 + b_kc[j], Kd) : 0u;
        stg_b[j] = buffer_load16(rb, b_off[j] | kmask_b, 0);
    };
    // Old output tile, passes p0 + 2j and p0 + 2j + 1 of the epilogue, into
    // the staging registers of pair j (an empty range for units that publish
    // a partial; the forward has no old tile).
    const bool own_write = BETA1 && splits <= 1;
    const long long out_base = (long long)m0 * ldd + n0;
    const auto ro = make_rsrc(D + out_base, own_write ? ((long long)M * ldd - out_base) * 2 : 0);
    auto load_out_pair = [&](int j, int p0) {
        stg_a[j] = buffer_load16(ro, out_off<bf16_t, NT, BM, BN>(ldd, M, N, m0, n0, tid, p0 + 2 * j), 0);
        stg_b[j] = buffer_load16(ro, out_off<bf16_t, NT, BM, BN>(ldd, M, N, m0, n0, tid, p0 + 2 * j + 1), 0);
    };
    // With two or more K iterations, a unit that writes its own tile fetches
    // the whole old tile inside the loop: the next-to-last iteration's load
    // slots (which would fetch a stage past the end) take passes 0..7, the
    // last iteration stores them to the free LDS buffer like a stage and
    // takes passes 8..15, so no load is left for the epilogue to wait on.
    // (not in units that also sum dbias: that reduction takes the LDS
    // before the epilogue)
    const bool early = own_write && nk >= 2 && !do_bias;
    // Registers -> LDS buffer `stage`: load j of wave w fills 1 KB block
    // LOADS * w + j of each operand region, lane p at byte 16p.
    auto store_pair = [&](int stage, int j) {
        char* la = smem + stage * STAGE + (LOADS * wave + j) * 1024 + 16 * lane;
        *(u32x4*)la = stg_a[j];
        *(u32x4*)(la + REGION) = stg_b[j];
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
    // forward: the bias values of this lane's accumulator columns
    u32x2 bv[NB][4];

    // Fragments of one 16-deep substep.
    struct Frag {
        bf16x8 a[NB];   // N side (MFMA input A)
        bf16x8 b[MB];   // M side (MFMA input B)
    };
    auto read_sub = [&](int stage, int k, Frag& f) {
        const char* sa = smem + stage * STAGE;
        const char* sb = sa + REGION;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            f.a[nb] = BKC ? frag_kc(sb, wn0 + nb * 32, k, lane) : frag_mn(sb, wn0 + nb * 32, k, lane);
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

    // Ring of two LDS stages plus one stage in registers.  Iteration `it`
    // runs the substeps of stage it (LDS buffer it & 1).  Before substep j it
    // writes load pair j of stage it+1 from registers into the other buffer
    // (free since the previous barrier) and reloads those registers with
    // pair j of stage it+2, so every load has one whole iteration to land
    // and the loads are spread over the iteration.  One barrier, before the
    // last substep, makes stage it+1 visible and retires buffer it & 1.
    // Loads per wave in issue order: pairs 0..3 of each stage; when pair j
    // of stage it+1 is needed, the 6 loads issued after it may still fly.
    if (nk > 0) {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) load_pair(kt0, j);
        wait_loads<0>();
#pragma unroll
        for (int j = 0; j < LOADS; ++j) store_pair(0, j);
#pragma unroll
        for (int j = 0; j < LOADS; ++j) load_pair(kt0 + 1, j);
        __syncthreads();
        Frag f0, f1;
        read_sub(0, 0, f0);
        // One iteration.  In the last one there is no next stage to store:
        // its load slots fetch passes 0..7 of the old tile for the epilogue,
        // or, with `early`, the next-to-last iteration fetches passes 0..7
        // instead of the stage past the end and the last one stores them to
        // the free buffer like a stage and fetches passes 8..15.
        auto iteration = [&](int it, auto mode) {
            // 0: steady state, 1: next to last with `early`, 2: last
            constexpr int MODE = decltype(mode)::value;
            constexpr bool LAST = MODE == 2;
            const int cur = it & 1;
            if (do_bias) bias_add(cur);
            // the forward's bias, fetched while the last stage computes
            if constexpr (LAST && OP == Op::FWD)
                load_bias_frags<NB>((const bf16_t*)p.bias, N, p.ldo, n0, wn0, lane, bv);
            // substeps 0..2: pair j of stage it+1 to LDS, pair j of stage it+2
            // into the registers, fragments of substep j+1, MFMAs of substep j
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                wait_loads<2 * (LOADS - 1)>();
                if constexpr (LAST) {
                    if constexpr (BETA1) {
                        if (early) store_pair(cur ^ 1, j);
                        load_out_pair(j, early ? 2 * LOADS : 0);
                    }
                } else {
                    store_pair(cur ^ 1, j);
                    if constexpr (MODE == 1)
                        load_out_pair(j, 0);
                    else
                        load_pair(kt0 + it + 2, j);
                }
                read_sub(cur, j + 1, (j & 1) ? f0 : f1);
                mma_sub((j & 1) ? f1 : f0);
                interleave_substep<(AK ? MB : 2 * MB) + (BKC ? NB : 2 * NB)>();
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_loads<2 * (LOADS - 1)>();
            if constexpr (LAST) {
                if constexpr (BETA1) {
                    if (early) store_pair(cur ^ 1, 3);
                    load_out_pair(3, early ? 2 * LOADS : 0);
                }
            } else {
                store_pair(cur ^ 1, 3);
                if constexpr (MODE == 1)
                    load_out_pair(3, 0);
                else
                    load_pair(kt0 + it + 2, 3);
            }
            __syncthreads();
            if constexpr (!LAST) read_sub(cur ^ 1, 0, f0);
            mma_sub(f1);
            __builtin_amdgcn_sched_barrier(0);
        };
        const int steady = early ? nk - 2 : nk - 1;
        for (int it = 0; it < steady; ++it) iteration(it, std::integral_constant<int, 0>());
        if constexpr (BETA1)
            if (early) iteration(nk - 2, std::integral_constant<int, 1>());
        iteration(nk - 1, std::integral_constant<int, 2>());
    }
    wait_loads<0>();

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

    if (splits > 1) {
        const int tile = tile_m * g.tiles_n + tile_n;
        float* w0 = p.ws + (long long)slot * (BM * BN);
        publish_partial<MB, NB, NT>(w0 + (long long)split * (BM * BN), acc, tid);
        float* wb = p.ws_bias + (long long)slot * BM + tid;
        if (do_bias && tid < BM) publish_bias(wb + split * BM, bias);
        if (!arrive_last(p.counters + g.tile_base + tile, splits, s_flag)) return;
        sum_partials<MB, NB, NT>(w0, splits, BM * BN, acc, tid);
        if (do_bias && tid < BM) bias = sum_bias(wb, splits, BM);
        if (tid == 0) p.counters[g.tile_base + tile] = 0;
        if constexpr (BETA1)
            write_tile_lds<bf16_t, MB, NB, NT, BM, BN, 0, SR>(D, ldd, M, N, m0, n0, acc, smem, tid,
                                                              lane, wm0, wn0, nullptr, p.seed, 1);
        else
            write_tile_bias<bf16_t, MB, NB, NT, BM, BN>(D, ldd, M, N, m0, n0, acc, smem, tid, lane,
                                                        wm0, wn0, (const bf16_t*)p.bias, p.ldo);
    } else if (!BETA1) {
        if (nk == 0) load_bias_frags<NB>((const bf16_t*)p.bias, N, p.ldo, n0, wn0, lane, bv);
        bias_round_write<MB, NB, NT, BM, BN>(D, ldd, M, N, m0, n0, acc, smem, tid, lane, wm0, wn0,
                                             bv);
    } else if (early) {
        // the whole old tile: passes 0..7 from the free LDS buffer (each
        // thread reads back the vectors it stored there itself), 8..15 staged
        static_assert(LOADS == 4, "the old tile's 16 passes: 8 read back, 8 in the staging pairs");
        const char* e = smem + (((nk - 1) & 1) ^ 1) * STAGE + LOADS * wave * 1024 + 16 * lane;
        u32x4 ev[2 * LOADS];
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            ev[2 * j] = *(const u32x4*)(e + j * 1024);
            ev[2 * j + 1] = *(const u32x4*)(e + j * 1024 + REGION);
        }
        const u32x4 pre[4 * LOADS] = {ev[0],    ev[1],    ev[2],    ev[3],    ev[4],    ev[5],
                                      ev[6],    ev[7],    stg_a[0], stg_b[0], stg_a[1], stg_b[1],
                                      stg_a[2], stg_b[2], stg_a[3], stg_b[3]};
        write_tile_lds<bf16_t, MB, NB, NT, BM, BN, 4 * LOADS, SR>(D, ldd, M, N, m0, n0, acc, smem,
                                                                   tid, lane, wm0, wn0, pre, p.seed, 1);
    } else if (nk > 0) {
        // the last K iteration loaded passes 0..7 of the old tile
        static_assert(LOADS == 4, "the old tile's first 8 passes sit in the 4 staging pairs");
        const u32x4 pre[2 * LOADS] = {stg_a[0], stg_b[0], stg_a[1], stg_b[1],
                                      stg_a[2], stg_b[2], stg_a[3], stg_b[3]};
        write_tile_lds<bf16_t, MB, NB, NT, BM, BN, 2 * LOADS, SR>(D, ldd, M, N, m0, n0, acc, smem,
                                                                   tid, lane, wm0, wn0, pre, p.seed, 1);
    } else {
        write_tile_lds<bf16_t, MB, NB, NT, BM, BN, 0, SR>(D, ldd, M, N, m0, n0, acc, smem, tid, lane,
                                                          wm0, wn0, nullptr, p.seed, 1);
    }
    if (do_bias && tid < BM && m0 + tid < M) {
        if constexpr (SR)
            ((bf16_t*)p.dbias)[m0 + tid] =
                bf16_t{(uint16_t)sr_bf16_element(bias, p.seed, 2, 0, (uint64_t)(m0 + tid))};
        else
            ((bf16_t*)p.dbias)[m0 + tid] = from_f32<bf16_t>(bias);
    }
}

__global__ __launch_bounds__(NT, 1) void mmb_tiles_bf16_kernel(TilesParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
    // the split-K ticket flag lives in the ring, used only after the K loop
    // (the dbias reduction uses the first 8 KB)
    int* s_flag = (int*)(smem + 8192);
    const int4 u = p.units[2 * blockIdx.x], v = p.units[2 * blockIdx.x + 1];
    if (u.x == UNIT_DINP)
        run_unit<Op::DINP>(p, p.g[UNIT_DINP], u, v, smem, s_flag);
    else
        run_unit<Op::DWEIGHT>(p, p.g[UNIT_DWEIGHT], u, v, smem, s_flag);
}

// The same launch with stochastically rounded dweight and dbias (dinp is
// still rounded to nearest).
__global__ __launch_bounds__(NT, 1) void mmb_tiles_bf16_sr_kernel(TilesParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
    int* s_flag = (int*)(smem + 8192);
    const int4 u = p.units[2 * blockIdx.x], v = p.units[2 * blockIdx.x + 1];
    if (u.x == UNIT_DINP)
        run_unit<Op::DINP>(p, p.g[UNIT_DINP], u, v, smem, s_flag);
    else
        run_unit<Op::DWEIGHT, true>(p, p.g[UNIT_DWEIGHT], u, v, smem, s_flag);
}

// The forward product out = inp . W^T + bias over the same tiles (plan slot
// UNIT_FWD).
__global__ __launch_bounds__(NT, 1) void mmb_fwd_bf16_kernel(TilesParams p) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
    int* s_flag = (int*)(smem + 8192);
    const int4 u = p.units[2 * blockIdx.x], v = p.units[2 * blockIdx.x + 1];
    run_unit<Op::FWD>(p, p.g[UNIT_FWD], u, v, smem, s_flag);
}

}  // namespace

int tiles_bf16_bk() { return BK; }
int tiles_bf16_bn() { return BN; }
// one workgroup per CU: the ring and the epilogue tile take most of the 160 KB LDS
int tiles_bf16_resident() { return (160 * 1024) / LDS_BYTES; }

hipError_t launch_tiles_bf16(const TilesParams& p, hipStream_t s) {
    if (p.n_units <= 0) return hipSuccess;
    hipLaunchKernelGGL(mmb_tiles_bf16_kernel, dim3(p.n_units), dim3(NT), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_tiles_bf16_sr(const TilesParams& p, hipStream_t s) {
    if (p.n_units <= 0) return hipSuccess;
    hipLaunchKernelGGL(mmb_tiles_bf16_sr_kernel, dim3(p.n_units), dim3(NT), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_fwd_tiles_bf16(const TilesParams& p, hipStream_t s) {
    if (p.n_units <= 0) return hipSuccess;
    hipLaunchKernelGGL(mmb_fwd_bf16_kernel, dim3(p.n_units), dim3(NT), 0, s, p);
    return hipGetLastError();
}

}  // namespace mmb
