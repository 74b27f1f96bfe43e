// mmb_internal.h -- declarations shared by the HIP sources of libmmb.so.
// Not installed; the public interface is include/mmb.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmb {

// One unit of work of the tiled kernel: the K iterations [kt0, kt1) of a
// (tile_m, tile_n) output tile of one GEMM.  A tile is cut into `splits`
// units (its own count: tiles of one GEMM may differ); the units of a split
// tile publish fp32 partial sums to workspace slots slot .. slot+splits-1
// (slot counts whole tiles) and the last to arrive finishes the tile.
// Encoded as two int4: {kind, tile_m, tile_n, split}, {kt0, kt1, splits, slot}.
enum UnitKind : int { UNIT_DWEIGHT = 0, UNIT_DINP = 1 };
// The forward launch (out = inp . W^T + bias) runs one GEMM; it sits in slot
// UNIT_DINP of the plan (its A operand, inp, is K-contiguous like dout in
// the dinp GEMM) and slot UNIT_DWEIGHT is empty.
constexpr int UNIT_FWD = UNIT_DINP;

struct GemmPlan {
    int M, N, K;          // D[M,N] += A[M,K] . B[K,N]
    int tiles_m, tiles_n; // ceil(M/BM), ceil(N/BN)
    int kiters;           // ceil(K/BK)
    int tile_base;        // index of tile (0,0) in the counter array
};

// Everything the tiled kernels need, passed by value (the backward launch
// uses dinp .. weight, the forward launch out, bias, inp and weight).
struct TilesParams {
    void* dinp;
    void* dweight;
    void* dbias;          // may be NULL
    const void* dout;
    const void* inp;
    const void* weight;
    int BT, C, OC;
    // row pitches in elements: ldo of dout (backward) or out (forward), ldc of
    // inp, weight, dinp and dweight; OC and C, or larger for packed copies.
    // The forward's bias holds ldo elements (zero past OC).
    int ldo, ldc;
    GemmPlan g[2];        // [UNIT_DWEIGHT], [UNIT_DINP]
    const int4* units;    // two int4 per unit (see above), in launch order
    int n_units;
    float* ws;            // split-K partial tiles (fp32), one tile per slot
    float* ws_bias;       // split-K partial dbias rows (fp32), BM floats per slot
    int* counters;        // one arrival counter per tile, zero at rest
    void* out;            // forward launch: out [BT,OC]
    const void* bias;     // forward launch: bias [OC], may be NULL
    unsigned long long seed;  // stochastic-rounding launch: Philox key word 0
};

// Tile shapes of the MFMA kernels (rows x cols of the output tile, K depth of
// one pipeline stage).
struct TileShape { int BM, BN, BK; };
TileShape tile_shape(int dtype);

// Launchers (return hipError_t of the launch).
hipError_t launch_tiles(int dtype, const TilesParams& p, hipStream_t s);
hipError_t launch_tiles_bf16(const TilesParams& p, hipStream_t s);
// bf16 backward with stochastically rounded dweight and dbias (seed in p)
hipError_t launch_tiles_bf16_sr(const TilesParams& p, hipStream_t s);
int tiles_bf16_bk();   // K depth of one stage of the bf16 tiles
int tiles_bf16_bn();   // output columns of one bf16 tile
// Workgroups of the MFMA tile kernel for `dtype` that fit on one CU at once
// (LDS and register limits of the kernel as built).
int tiles_resident(int dtype);
int tiles_bf16_resident();
// The forward product out = inp . W^T + bias with the same tiles (one GEMM,
// M = BT, N = OC, K = C, in plan slot UNIT_FWD).
hipError_t launch_fwd_tiles(int dtype, const TilesParams& p, hipStream_t s);
hipError_t launch_fwd_tiles_bf16(const TilesParams& p, hipStream_t s);
hipError_t launch_fwd_generic(int dtype, void* out, const void* inp, const void* weight,
                              const void* bias, int BT, int C, int OC, hipStream_t s);
// LayerNorm backward (one dtype for all tensors; every output accumulates).
struct LNParams {
    void* dinp;            // [BT, C]
    void* dweight;         // [C]
    void* dbias;           // [C]
    const void* dout;      // [BT, C]
    const void* inp;       // [BT, C]
    const void* weight;    // [C]
    const void* mean;      // [BT]
    const void* rstd;      // [BT]
    long long BT;
    int C;
    float* partial;        // [G, 2C] fp32 column sums per workgroup
};
// Row-kernel layout for C: nj 16-byte vectors per lane (1, 2, 4; 8 in fp32)
// and wpr waves per row (1, 2, 4 or 8), or nj = 0 for the generic kernels (C
// not a multiple of the vector width, or too wide).
struct LNLayout {
    int nj, wpr;
};
LNLayout ln_layout(int dtype, int C);
int ln_vectors_per_lane(int dtype, int C);   // ln_layout(dtype, C).nj
// G workgroups for the row kernel (partial holds G * 2C floats), each taking
// 8 / wpr rows at a time.  Two launches on `s` (rows, then the column reduce).
hipError_t launch_layernorm_backward(int dtype, const LNParams& p, int G, LNLayout k,
                                     hipStream_t s);

// Row-pitch copies for shapes whose rows are not whole 16-byte vectors:
// pack: dst[r, c] = src[r, c] for c < cols, 0 for cols <= c < ld_dst;
// unpack: dst[r, c] = src[r, c] for c < cols.  es: element size (2 or 4).
hipError_t launch_pack(void* dst, long long ld_dst, const void* src, long long ld_src,
                       long long rows, int cols, int es, hipStream_t s);
hipError_t launch_unpack(void* dst, long long ld_dst, const void* src, long long ld_src,
                         long long rows, int cols, int es, hipStream_t s);

// sr: bf16 only, dweight and dbias stochastically rounded under `seed`
hipError_t launch_generic(int dtype, void* dinp, void* dweight, void* dbias,
                          const void* dout, const void* inp, const void* weight,
                          int BT, int C, int OC, hipStream_t s, bool sr = false,
                          unsigned long long seed = 0);

}  // namespace mmb
