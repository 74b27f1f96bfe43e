// mmb_tiles.hip -- fp32 MFMA tiles of the linear-layer backward pass: both
// GEMMs and the bias reduction in one launch of output-tile work units (the
// bf16 tiles live in mmb_tiles_bf16.hip); and of the forward product
// out = inp . W^T + bias (both operands K-contiguous, beta = 0, the bias
// added in the epilogue), a launch of its own.
//
// Operation (llm.c page "dev/cuda/matmul_backward.cu", launcher
// matmul_backward1 and bias kernels):
//   dinp    [BT,C] += dout[BT,OC] . weight[OC,C]      (unit kind UNIT_DINP)
//   dweight [OC,C] += dout^T[OC,BT] . inp[BT,C]       (unit kind UNIT_DWEIGHT)
//   dbias   [OC]    = column sums of dout             (inside dweight units
//                                                      of output column tile 0)
// The page's check runs its GEMMs in true fp32 (TF32 off); so do these:
// v_mfma_f32_32x32x2_f32 multiplies and accumulates in fp32.
//
// gfx950 design:
//  * One workgroup = 4 wave64s = one 128 x 128 output tile, each wave a
//    64 x 64 quarter (2 x 2 blocks of 32x32 MFMA).  64 KB of LDS, so two
//    workgroups share a CU.
//  * Operands are staged global -> registers -> LDS with a 2-stage ping-pong
//    (the loads of stage k+1 are in flight while the MFMAs of stage k run;
//    one barrier per stage).  LDS holds K-contiguous rows of 128 bytes (32
//    floats); the 16-byte chunk c of row r lives at c ^ (r & 7), so fragment
//    reads (8 rows, one chunk) and staging writes (1 row, 8 chunks) are
//    conflict-free.  Operands that are K-strided in memory (weight, inp, and
//    dout for dweight) are transposed 4 x 4 in registers on the way in.
//  * Each lane reads 4 consecutive K of a row with one ds_read_b128; the
//    four MFMAs of a group of 8 K take element q of both operands (lane half
//    h covers K = 8s + 4h + q), which covers all 8 K exactly once.
//  * The MFMA "A" input is the N-side tile, so each lane's accumulators hold
//    4 consecutive output columns (16-byte epilogue accesses).
//  * Split K (dweight's K = B*T): partial tiles, tickets and the ordered
//    last-arriver sum are the shared helpers of mmb_tile_common.h.
//  * dbias: the dweight units of column tile 0 sum the dout values they
//    stage; a 3-step xor shuffle combines the 8 threads sharing a column.
#include <algorithm>

#include "mmb_tile_common.h"

namespace mmb {
namespace {

constexpr int kRowBytes = 128;  // one LDS row: BK floats of one m or n

template <typename T> struct Cfg;
template <> struct Cfg<float> {
    static constexpr int BM = 128, BN = 128, BK = 32;
    static constexpr int E = 4;
    static constexpr int WM = 64, WN = 64;
};

template <typename T>
struct K {
    static constexpr int BM = Cfg<T>::BM, BN = Cfg<T>::BN, BK = Cfg<T>::BK, E = Cfg<T>::E;
    static constexpr int WM = Cfg<T>::WM, WN = Cfg<T>::WN;
    static constexpr int MB = WM / 32, NB = WN / 32;        // 32x32 blocks per wave
    static constexpr int STAGE_BYTES = (BM + BN) * kRowBytes;
    // the ring, or the whole output tile in the epilogue
    static constexpr int OUT_BYTES = out_lds_bytes<T, BM, BN>();
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES > OUT_BYTES ? 2 * STAGE_BYTES : OUT_BYTES;
    static constexpr int A_KC_PER = BM * 8 / kThreads;      // K-contiguous A: vectors/thread
    static_assert(BK * (int)sizeof(T) == kRowBytes, "row = 8 vectors of 16 bytes");
    static_assert(BM == 2 * WM && BN == 2 * WN, "2 x 2 waves");
    static_assert(BM / E * 8 <= kThreads && BN / E * 8 <= kThreads, "one staging pass");
};

// 16-byte chunk c of LDS row r sits at c ^ ((r >> 1) & 7): a fragment read
// (16 consecutive rows, one chunk, per pass of a wave's ds_read_b128) then
// touches 16 distinct 16-byte bank groups of the 64-bank LDS (group
// 8 (r & 1) + (c ^ ((r >> 1) & 7))), and so does a staging store of two
// consecutive rows' 8 chunks.  (Keyed on r & 7, rows r and r + 8 collided.)
__device__ __forceinline__ int swz(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// ---- E x E transpose of one staged block ---------------------------------
// in[r] holds E consecutive columns of K-row r; out[x] gets E consecutive
// K-rows of column x.
__device__ __forceinline__ void transpose_block(const u32x4 (&in)[4], u32x4 (&out)[4], float) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int p = 0; p < 4; ++p) out[x][p] = in[p][x];
}

// column sums of a staged block (dbias), fp32
__device__ __forceinline__ void add_columns(const u32x4 (&in)[4], float (&s)[4], float) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int x = 0; x < 4; ++x) s[x] += __uint_as_float(in[r][x]);
}

// ---- MFMA steps of one LDS stage ------------------------------------------
// The fragments of one 8-deep substep s (one ds_read_b128 per block and lane).
template <typename T>
struct Frags {
    u32x4 a[K<T>::NB], b[K<T>::MB];
};
template <typename T>
__device__ __forceinline__ void read_frags(const char* sa, const char* sb, int s, int wm0, int wn0,
                                           int lane, Frags<T>& f) {
    using Kt = K<T>;
    const int lr = lane & 31, chunk = 2 * s + (lane >> 5);
#pragma unroll
    for (int nb = 0; nb < Kt::NB; ++nb) f.a[nb] = *(const u32x4*)(sb + swz(wn0 + nb * 32 + lr, chunk));
#pragma unroll
    for (int mb = 0; mb < Kt::MB; ++mb) f.b[mb] = *(const u32x4*)(sa + swz(wm0 + mb * 32 + lr, chunk));
}
// lane half h holds k = 8s + 4h + q in element q: MFMA q reduces over the
// pair {8s + q, 8s + 4 + q}; all four cover the 8 k.
template <typename T>
__device__ __forceinline__ void mma_sub(const Frags<T>& f, f32x16 (&acc)[K<T>::MB][K<T>::NB]) {
    using Kt = K<T>;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int mb = 0; mb < Kt::MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < Kt::NB; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                    __uint_as_float(f.a[nb][q]), __uint_as_float(f.b[mb][q]), acc[mb][nb], 0, 0, 0);
}

// ---- one work unit ---------------------------------------------------------
// The three GEMMs, with the orientation of their operands in memory:
//   DINP     dinp [BT,C]   += dout [BT,OC] . weight [OC,C]  A K-contiguous, B N-contiguous
//   DWEIGHT  dweight [OC,C] += dout^T . inp [BT,C]          A M-contiguous, B N-contiguous
//   FWD      out [BT,OC]    = inp [BT,C] . weight^T + bias  A K-contiguous, B K-contiguous
// (FWD: out = inp . W^T, the forward product whose gradients the other two are.)
enum class Op { DINP, DWEIGHT, FWD };

template <typename T, Op OP>
__device__ __forceinline__ void run_unit(const TilesParams& p, const GemmPlan& g, int4 u, int4 v,
                                         char* smem, int* s_flag) {
    using Kt = K<T>;
    constexpr bool AK = OP != Op::DWEIGHT;   // A rows K-contiguous (dout rows, inp rows)
    constexpr bool BKC = OP == Op::FWD;      // B rows K-contiguous (weight rows)
    constexpr int BM = Kt::BM, BN = Kt::BN, BK = Kt::BK, E = Kt::E;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tile_m = u.y, tile_n = u.z, split = u.w;
    const int M = g.M, N = g.N, Kd = g.K;
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    // K iterations [kt0, kt1) of a tile cut into `splits` units; the tile's
    // partial sums (if any) start at workspace slot `slot`
    const int kt0 = v.x, kt1 = v.y, splits = v.z, slot = v.w;

    const T* A = (const T*)(OP == Op::FWD ? p.inp : p.dout);
    const T* Bop = (const T*)(OP == Op::DWEIGHT ? p.inp : p.weight);   // ld = C
    T* D = (T*)(OP == Op::DINP ? p.dinp : OP == Op::DWEIGHT ? p.dweight : p.out);
    // row pitches: dout (out) rows ldo, the C-wide tensors' rows ldc
    const long long lda = OP == Op::FWD ? p.ldc : p.ldo, ldb = p.ldc, ldd = OP == Op::FWD ? p.ldo : p.ldc;
    const bool do_bias = OP == Op::DWEIGHT && p.dbias != nullptr && tile_n == 0;

    // staging thread roles
    const int kg = tid & 7, xg = tid >> 3;       // E x E block: K-group, column group
    const bool b_active = BKC || xg < BN / E;
    const bool a_active = AK || xg < BM / E;

    constexpr int APER = AK ? Kt::A_KC_PER : E;
    u32x4 ra[APER], rb[E];
    float bsum[E];
#pragma unroll
    for (int x = 0; x < E; ++x) bsum[x] = 0.f;

    static_assert(Kt::BN * 8 / kThreads == E, "K-contiguous B: E vectors per thread");
    static_assert(APER == E, "4 vectors per operand and thread");
    // Buffer-load geometry, fixed per thread: byte offsets from the stage's
    // origin in the operand (the origin moves each stage, so every offset
    // stays below 2^31).  Out-of-range vectors load zeros: columns past N or
    // M through an offset of 2^31, rows past the operand's end because they
    // fall outside the buffer range, K-contiguous vectors at or past K
    // through a per-stage mask.
    //   K-contiguous operand: vector j = row (tid >> 3) + 32 j, K 4 (tid & 7)
    //   M/N-contiguous: vector r = K-row 4 kg + r, columns 4 xg .. 4 xg + 3
    const long long a_elems = (long long)p.BT * lda;
    const long long b_elems = OP == Op::DWEIGHT ? (long long)p.BT * ldb : (long long)p.OC * ldb;
    uint32_t a_off[E], b_off[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const long long kc_row = (long long)((tid >> 3) + 32 * j);
        if constexpr (AK)
            a_off[j] = (uint32_t)((kc_row * lda + (tid & 7) * E) * 4);
        else
            a_off[j] = (uint32_t)((((long long)(kg * E + j)) * lda + m0 + xg * E) * 4) |
                       oob_if_ge(m0 + xg * E, M);
        if constexpr (BKC)
            b_off[j] = (uint32_t)((kc_row * ldb + (tid & 7) * E) * 4);
        else
            b_off[j] = (uint32_t)((((long long)(kg * E + j)) * ldb + n0 + xg * E) * 4) |
                       oob_if_ge(n0 + xg * E, N);
    }
    auto load = [&](int kt) {
        const int k0 = kt * BK;
        const uint32_t kmask = oob_if_ge(k0 + (tid & 7) * E, Kd);
        {
            const long long o = BKC ? (long long)n0 * ldb + k0 : (long long)k0 * ldb;
            const auto r = make_rsrc(Bop + o, (b_elems - o) * 4);
#pragma unroll
            for (int j = 0; j < E; ++j) rb[j] = buffer_load16(r, b_off[j] | (BKC ? kmask : 0u), 0);
        }
        {
            const long long o = AK ? (long long)m0 * lda + k0 : (long long)k0 * lda;
            const auto r = make_rsrc(A + o, (a_elems - o) * 4);
#pragma unroll
            for (int j = 0; j < E; ++j) ra[j] = buffer_load16(r, a_off[j] | (AK ? kmask : 0u), 0);
        }
    };

    auto store = [&](int stage) {
        char* sa = smem + stage * Kt::STAGE_BYTES;
        char* sb = sa + BM * kRowBytes;
        if constexpr (BKC) {
#pragma unroll
            for (int j = 0; j < E; ++j) *(u32x4*)(sb + swz((tid >> 3) + 32 * j, tid & 7)) = rb[j];
        } else if (b_active) {
            u32x4 t[E];
            transpose_block(rb, t, T{});
#pragma unroll
            for (int x = 0; x < E; ++x) *(u32x4*)(sb + swz(xg * E + x, kg)) = t[x];
        }
        if constexpr (AK) {
#pragma unroll
            for (int j = 0; j < APER; ++j)
                *(u32x4*)(sa + swz((tid >> 3) + 32 * j, tid & 7)) = ra[j];
        } else {
            if (a_active) {
                if (do_bias) add_columns(ra, bsum, T{});
                u32x4 t[E];
                transpose_block(ra, t, T{});
#pragma unroll
                for (int x = 0; x < E; ++x) *(u32x4*)(sa + swz(xg * E + x, kg)) = t[x];
            }
        }
    };

    f32x16 acc[Kt::MB][Kt::NB];
#pragma unroll
    for (int i = 0; i < Kt::MB; ++i)
#pragma unroll
        for (int j = 0; j < Kt::NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int wm0 = (wave & 1) * Kt::WM, wn0 = (wave >> 1) * Kt::WN;

    // Fragments are read one substep ahead of the MFMAs that use them, and
    // the stage barrier sits before the last substep's MFMAs, so the next
    // stage's first fragments are read while those run.
    load(kt0);
    store(0);
    __syncthreads();
    Frags<T> f0, f1;
    read_frags<T>(smem, smem + BM * kRowBytes, 0, wm0, wn0, lane, f0);
    for (int kt = kt0; kt < kt1; ++kt) {
        const int cur = (kt - kt0) & 1;
        const bool more = kt + 1 < kt1;
        if (more) load(kt + 1);
        const char* sa = smem + cur * Kt::STAGE_BYTES;
        const char* sb = sa + BM * kRowBytes;
        read_frags<T>(sa, sb, 1, wm0, wn0, lane, f1);
        mma_sub<T>(f0, acc);
        read_frags<T>(sa, sb, 2, wm0, wn0, lane, f0);
        mma_sub<T>(f1, acc);
        read_frags<T>(sa, sb, 3, wm0, wn0, lane, f1);
        mma_sub<T>(f0, acc);
        if (more) store(cur ^ 1);
        __syncthreads();
        if (more) {
            const char* na = smem + (cur ^ 1) * Kt::STAGE_BYTES;
            read_frags<T>(na, na + BM * kRowBytes, 0, wm0, wn0, lane, f0);
        }
        mma_sub<T>(f1, acc);
    }

    // dbias: combine the 8 K-groups of each column (lanes differing in bits 0..2)
    if (do_bias) {
#pragma unroll
        for (int x = 0; x < E; ++x) {
            float v = bsum[x];
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            bsum[x] = v;
        }
    }

    const bool bias_owner = do_bias && kg == 0 && a_active;
    if (splits > 1) {
        const int tile = tile_m * g.tiles_n + tile_n;
        float* w0 = p.ws + (long long)slot * (BM * BN);
        publish_partial<Kt::MB, Kt::NB, kThreads>(w0 + (long long)split * (BM * BN), acc, tid);
        float* wb = p.ws_bias + (long long)slot * BM + xg * E;
        if (bias_owner) {
#pragma unroll
            for (int x = 0; x < E; ++x) publish_bias(wb + split * BM + x, bsum[x]);
        }
        if (!arrive_last(p.counters + g.tile_base + tile, splits, s_flag)) return;
        sum_partials<Kt::MB, Kt::NB, kThreads>(w0, splits, BM * BN, acc, tid);
        if (bias_owner) {
#pragma unroll
            for (int x = 0; x < E; ++x) bsum[x] = sum_bias(wb + x, splits, BM);
        }
        if (tid == 0) p.counters[g.tile_base + tile] = 0;
    }

    if constexpr (OP == Op::FWD)
        write_tile_bias<T, Kt::MB, Kt::NB, kThreads, BM, BN>(D, ldd, M, N, m0, n0, acc, smem, tid,
                                                            lane, wm0, wn0, (const T*)p.bias, p.ldo);
    else
        write_tile_lds<T, Kt::MB, Kt::NB, kThreads, BM, BN>(D, ldd, M, N, m0, n0, acc, smem, tid,
                                                           lane, wm0, wn0);
    if (bias_owner) {
        T* db = (T*)p.dbias;
#pragma unroll
        for (int x = 0; x < E; ++x) {
            const int m = m0 + xg * E + x;
            if (m < M) db[m] = from_f32<T>(bsum[x]);
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void mmb_tiles_kernel(TilesParams p) {
    __shared__ __attribute__((aligned(16))) char smem[K<T>::LDS_BYTES];
    __shared__ int s_flag;
    const int4 u = p.units[2 * blockIdx.x], v = p.units[2 * blockIdx.x + 1];
    if (u.x == UNIT_DINP)
        run_unit<T, Op::DINP>(p, p.g[UNIT_DINP], u, v, smem, &s_flag);
    else
        run_unit<T, Op::DWEIGHT>(p, p.g[UNIT_DWEIGHT], u, v, smem, &s_flag);
}

// The forward product out = inp . W^T + bias over the same tiles (plan slot
// UNIT_FWD).
template <typename T>
__global__ __launch_bounds__(kThreads) void mmb_fwd_kernel(TilesParams p) {
    __shared__ __attribute__((aligned(16))) char smem[K<T>::LDS_BYTES];
    __shared__ int s_flag;
    const int4 u = p.units[2 * blockIdx.x], v = p.units[2 * blockIdx.x + 1];
    run_unit<T, Op::FWD>(p, p.g[UNIT_FWD], u, v, smem, &s_flag);
}

}  // namespace

TileShape tile_shape(int dtype) {
    if (dtype == 1) return TileShape{256, tiles_bf16_bn(), tiles_bf16_bk()};
    return TileShape{K<float>::BM, K<float>::BN, K<float>::BK};
}

// fp32: two workgroups per CU (LDS, and at most 128 registers per lane for
// two waves per SIMD)
int tiles_resident(int dtype) {
    if (dtype == 1) return tiles_bf16_resident();
    return std::min(2, (160 * 1024) / (K<float>::LDS_BYTES + 16));
}

hipError_t launch_tiles(int dtype, const TilesParams& p, hipStream_t s) {
    if (dtype == 1) return launch_tiles_bf16(p, s);
    if (p.n_units <= 0) return hipSuccess;
    hipLaunchKernelGGL(mmb_tiles_kernel<float>, dim3(p.n_units), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_fwd_tiles(int dtype, const TilesParams& p, hipStream_t s) {
    if (dtype == 1) return launch_fwd_tiles_bf16(p, s);
    if (p.n_units <= 0) return hipSuccess;
    hipLaunchKernelGGL(mmb_fwd_kernel<float>, dim3(p.n_units), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace mmb
