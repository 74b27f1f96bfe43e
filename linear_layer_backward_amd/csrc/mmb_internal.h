// mmb_internal.h -- declarations shared by the HIP sources of libmmb.so.
// Not installed; the public interface is include/mmb.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmb {

// One unit of work of the tiled kernel: a (tile_m, tile_n) output tile of one
// GEMM over the K-iteration range of split `split`.
enum UnitKind : int { UNIT_DWEIGHT = 0, UNIT_DINP = 1 };

struct GemmPlan {
    int M, N, K;          // D[M,N] += A[M,K] . B[K,N]
    int tiles_m, tiles_n; // ceil(M/BM), ceil(N/BN)
    int splits;           // K split into this many ranges (1 = no split)
    int kiters;           // ceil(K/BK)
    int tile_base;        // index of tile (0,0) in the counter array
    long long ws_base;    // float offset of this GEMM's partial tiles in the workspace
};

// Everything the tiled kernel needs, passed by value.
struct TilesParams {
    void* dinp;
    void* dweight;
    void* dbias;          // may be NULL
    const void* dout;
    const void* inp;
    const void* weight;
    int BT, C, OC;
    GemmPlan g[2];        // [UNIT_DWEIGHT], [UNIT_DINP]
    const int4* units;    // {kind, tile_m, tile_n, split}, in launch order
    int n_units;
    float* ws;            // split-K partial tiles (fp32)
    float* ws_bias;       // split-K partial dbias rows (fp32)
    int* counters;        // one arrival counter per split tile, zero at rest
};

// Tile shapes of the MFMA kernels (rows x cols of the output tile, K depth of
// one pipeline stage).
struct TileShape { int BM, BN, BK; };
TileShape tile_shape(int dtype);

// Launchers (return hipError_t of the launch).
hipError_t launch_tiles(int dtype, const TilesParams& p, hipStream_t s);
hipError_t launch_tiles_bf16(const TilesParams& p, hipStream_t s);
int tiles_bf16_bk();   // K depth of one stage of the bf16 tiles
int tiles_bf16_bn();   // output columns of one bf16 tile
// Workgroups of the MFMA tile kernel for `dtype` that fit on one CU at once
// (LDS and register limits of the kernel as built).
int tiles_resident(int dtype);
int tiles_bf16_resident();
hipError_t launch_generic(int dtype, void* dinp, void* dweight, void* dbias,
                          const void* dout, const void* inp, const void* weight,
                          int BT, int C, int OC, hipStream_t s);

}  // namespace mmb
