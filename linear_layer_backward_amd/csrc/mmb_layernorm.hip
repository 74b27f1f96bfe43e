// mmb_layernorm.hip -- LayerNorm backward, the op next to the linear layer in
// a GPT-2 block (llm.c page "dev/cuda/layernorm_backward.cu", CPU reference
// layernorm_backward_cpu).  For every row r of B*T rows of C channels, with
// the forward's saved mean[r] and rstd[r]:
//   norm_i = (inp[r,i] - mean[r]) * rstd[r],   dnorm_i = weight[i] * dout[r,i]
//   a = mean_i dnorm_i,   b = mean_i dnorm_i * norm_i
//   dinp[r,i] += (dnorm_i - a - norm_i * b) * rstd[r]
//   dweight[i] += sum_r norm_i * dout[r,i],   dbias[i] += sum_r dout[r,i]
//
// The op is bound by HBM: per row it reads dout, inp and the old dinp and
// writes dinp; the flops are a few per element.  gfx950 design:
//  * One wave64 per row, 8 waves per workgroup, one workgroup per CU, rows
//    dealt out wave by wave (the row index is wave-uniform, so every buffer
//    descriptor lives in scalar registers).  Lane l owns the 16-byte column
//    vectors l, l + 64, ... (NJ <= 4 of them in bf16, C <= 2048; NJ <= 8 in
//    fp32, C <= 2048), so each row is read
//    with fully coalesced 16-byte loads; the weight row sits in LDS and the
//    lane's dweight / dbias sums stay in registers for all its rows.
//  * Wider rows (bf16 C <= 8192, fp32 C <= 4096) take 2 or 4 waves per row,
//    and rows up to C = 16384 all 8 waves of the workgroup; the parts' two
//    row sums meet in LDS (see ln_bwd_rows).  Wider still, the generic
//    kernels below.
//  * With up to 4 vectors per lane each wave keeps two rows in flight: the
//    loads of its next row (dout, inp, the old dinp, mean, rstd) are issued
//    before it works on the current one; with 8, one row.
//  * The two row means are wave reductions in a fixed order (DPP lane moves).
//  * dweight / dbias: each wave writes its sums to its own LDS slot, each
//    column is added over the 8 waves in wave order, and the workgroup
//    writes one fp32 partial row of 2C values; a second launch sums
//    the partials of all workgroups in a fixed order (32 interleaved groups
//    per column, then the groups in order), adds the old values and rounds
//    once.  No atomics: results repeat bit for bit.
//  * bf16 storage: values widen exactly to fp32, all arithmetic is fp32, each
//    output is rounded once to nearest-even.
#include "mmb_tile_common.h"

namespace mmb {
namespace {

constexpr int LN_NT = 512, LN_NW = LN_NT / 64;

template <typename T> struct Vec;
template <> struct Vec<float> { static constexpr int N = 4; };
template <> struct Vec<bf16_t> { static constexpr int N = 8; };

// element e of a 16-byte vector, widened to fp32
template <typename T>
__device__ __forceinline__ float elem(const u32x4& v, int e) {
    if constexpr (sizeof(T) == 4) return __uint_as_float(v[e]);
    else return __uint_as_float(e & 1 ? (v[e >> 1] & 0xffff0000u) : (v[e >> 1] << 16));
}

template <typename T>
__device__ __forceinline__ u32x4 pack(const float (&f)[Vec<T>::N]) {
    u32x4 o;
    if constexpr (sizeof(T) == 4) {
        for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(f[e]);
    } else {
        for (int e = 0; e < 4; ++e) o[e] = f32x2_to_bf16x2_bits(f[2 * e], f[2 * e + 1]);
    }
    return o;
}

// Sum over the 64 lanes of a wave, in a fixed order, with DPP lane moves
// (no LDS round trips): row_shr 1, 2, 4, 8 leave each 16-lane row's sum in
// its lane 15; row_bcast15 adds row 0's into row 1 and row 2's into row 3;
// row_bcast31 adds lane 31 into rows 2 and 3, so lane 63 holds the total.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF,
                                              true);
    return v + __builtin_bit_cast(float, t);
}
__device__ __forceinline__ float wave_sum(float v) {
    v = dpp_add<0x111, 0xF>(v);   // row_shr:1
    v = dpp_add<0x112, 0xF>(v);   // row_shr:2
    v = dpp_add<0x114, 0xF>(v);   // row_shr:4
    v = dpp_add<0x118, 0xF>(v);   // row_shr:8
    v = dpp_add<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// WPR waves per row: a row wider than one wave's NJ vectors per lane (bf16
// C > 2048, fp32 C > 2048) is split into WPR contiguous parts, part h of 64 *
// NJ vectors taken by wave h of a group of WPR waves (LN_NW / WPR rows per
// workgroup step).  The two row sums then meet in LDS: each wave writes its
// part's sums, one workgroup barrier, and every wave adds the WPR parts in
// part order.  All waves of the workgroup take the same number of steps (a
// group whose row is past the end works on an empty row), so the barriers
// match; the sums' slots alternate between two buffers, so a wave writing
// the next row's sums cannot overwrite values a slower wave still reads.
template <typename T, int NJ, int WPR>
__global__ __launch_bounds__(LN_NT, 1) void ln_bwd_rows(LNParams p) {
    constexpr int V = Vec<T>::N;
    // Rows in flight per wave: two up to 4 vectors per lane; with 8 (wide
    // rows) one, as two would not fit the registers (an fp32 row of 8
    // vectors per lane is as many bytes as a bf16 row of 4, so the bytes in
    // flight per CU stay the same).
    constexpr bool PIPE2 = NJ <= 4;
    static_assert(NJ <= 4 || sizeof(T) == 4, "8 bf16 vectors per lane would spill registers");
    static_assert(WPR >= 1 && LN_NW % WPR == 0, "whole groups of waves");
    constexpr int GROUPS = LN_NW / WPR;       // rows per workgroup step
    constexpr int COLS = 64 * NJ * V;         // one wave's columns
    constexpr int SLOT = 2 * COLS;            // one wave's [dweight | dbias] sums
    // the groups' column sums meet in LDS; with one group (WPR = 8) every
    // column belongs to one wave, which writes its sums out directly
    __shared__ float red[GROUPS > 1 ? LN_NW * SLOT : 1];
    __shared__ float xch[2][WPR > 1 ? LN_NW : 1][2];   // WPR > 1: the parts' row sums
    const int tid = threadIdx.x, lane = tid & 63;
    // uniform per wave: the row index, and so every buffer descriptor built
    // from it, stays in scalar registers (a per-lane value would make the
    // compiler wrap each buffer access in a readfirstlane loop)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = wave / WPR, part = wave % WPR;
    const int C = p.C;
    const long long rowbytes = (long long)C * (long long)sizeof(T);
    // lane's vector j covers columns V * (64 * (NJ * part + j) + lane) .. + V - 1
    uint32_t off[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int col = WPR == 1 ? V * (lane + 64 * j) : V * (64 * (NJ * part + j) + lane);
        off[j] = (uint32_t)(col * (int)sizeof(T)) | oob_if_ge(col, C);
    }
    // the weight row, shared by the workgroup's waves: vector v at wl[v]
    __shared__ u32x4 wl[64 * NJ * WPR];
    float aw[NJ][V], ab[NJ][V];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < V; ++e) aw[j][e] = ab[j][e] = 0.f;

    const long long ngroups = (long long)gridDim.x * GROUPS;
    long long r = (long long)blockIdx.x * GROUPS + group;
    const T* dout = (const T*)p.dout;
    const T* inp = (const T*)p.inp;
    T* dinp = (T*)p.dinp;
    // Everything a row needs, loaded one row ahead: while a wave works on
    // row r, the loads of its next row (dout, inp, the old dinp, mean, rstd)
    // are in flight.  Rows past the end load zeros from an empty range.
    struct RowSet {
        u32x4 d[NJ], x[NJ], g[NJ];
        float m, s;
    };
    auto load_set = [&](RowSet& S, long long row) {
        const bool live = row < p.BT;
        const long long rr = live ? row : 0;
        const long long n = live ? rowbytes : 0;
        const auto rd = make_rsrc(dout + rr * C, n);
        const auto rx = make_rsrc(inp + rr * C, n);
        const auto rg = make_rsrc(dinp + rr * C, n);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            S.d[j] = buffer_load16(rd, off[j], 0);
            S.x[j] = buffer_load16(rx, off[j], 0);
            S.g[j] = buffer_load16(rg, off[j], 0);
        }
        S.m = to_f32(((const T*)p.mean)[rr]);
        S.s = to_f32(((const T*)p.rstd)[rr]);
    };
    const float invC = 1.0f / (float)C;
    int step = 0;   // WPR > 1: row steps taken (the same in every wave)
    auto process = [&](RowSet& S, long long row) {
        float sa = 0.f, sb = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const u32x4 wj = WPR == 1 ? wl[lane + 64 * j] : wl[64 * (NJ * part + j) + lane];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float dv = elem<T>(S.d[j], e);
                const float nrm = (elem<T>(S.x[j], e) - S.m) * S.s;
                const float dn = elem<T>(wj, e) * dv;
                sa += dn;
                sb += dn * nrm;
                ab[j][e] += dv;
                aw[j][e] += nrm * dv;
            }
        }
        float ta = wave_sum(sa), tb = wave_sum(sb);
        if constexpr (WPR > 1) {
            float (*x)[2] = xch[step & 1];
            if (lane == 0) {
                x[wave][0] = ta;
                x[wave][1] = tb;
            }
            __syncthreads();
            ta = x[group * WPR][0];
            tb = x[group * WPR][1];
#pragma unroll
            for (int h = 1; h < WPR; ++h) {
                ta += x[group * WPR + h][0];
                tb += x[group * WPR + h][1];
            }
            ++step;
        }
        const float a = ta * invC, b = tb * invC;
        // widen dout and inp again below instead of keeping 2 * NJ * V floats
        // live across the reductions (empty register barrier, no instruction)
#pragma unroll
        for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(S.d[j]), "+v"(S.x[j]));
        // (with WPR > 1 a group may step past the last row: an empty range)
        const bool live = WPR == 1 || row < p.BT;
        const auto rg = make_rsrc(dinp + (live ? row : 0) * C, live ? rowbytes : 0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const u32x4 wj = WPR == 1 ? wl[lane + 64 * j] : wl[64 * (NJ * part + j) + lane];
            float o[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float nrm = (elem<T>(S.x[j], e) - S.m) * S.s;
                const float dn = elem<T>(wj, e) * elem<T>(S.d[j], e);
                o[e] = elem<T>(S.g[j], e) + (dn - a - nrm * b) * S.s;
            }
            __builtin_amdgcn_raw_buffer_store_b128(pack<T>(o), rg, off[j], 0, 0);
        }
    };
    RowSet A, B;
    load_set(A, r);
    // staged while the first row's loads fly
    {
        const auto rw = make_rsrc(p.weight, rowbytes);
        for (int v = tid; v < 64 * NJ * WPR; v += LN_NT)
            wl[v] = buffer_load16(rw, (uint32_t)(V * v * (int)sizeof(T)) | oob_if_ge(V * v, C), 0);
        __syncthreads();
    }
    if constexpr (WPR > 1) {
        // every wave of the workgroup takes the same steps: the loop runs
        // while the workgroup's first row of the step is live
        const long long r0 = (long long)blockIdx.x * GROUPS;
        long long base = r0;
        if constexpr (PIPE2) {
            while (base < p.BT) {
                load_set(B, r + ngroups);
                process(A, r);
                r += ngroups;
                base += ngroups;
                if (base >= p.BT) break;
                load_set(A, r + ngroups);
                process(B, r);
                r += ngroups;
                base += ngroups;
            }
        } else {
            while (base < p.BT) {
                process(A, r);
                r += ngroups;
                base += ngroups;
                if (base < p.BT) load_set(A, r);
            }
        }
    } else if constexpr (PIPE2) {
        while (r < p.BT) {
            load_set(B, r + ngroups);
            process(A, r);
            r += ngroups;
            if (r >= p.BT) break;
            load_set(A, r + ngroups);
            process(B, r);
            r += ngroups;
        }
    } else {
        while (r < p.BT) {
            process(A, r);
            r += ngroups;
            if (r < p.BT) load_set(A, r);
        }
    }
    float* part_out = p.partial + (long long)blockIdx.x * 2 * C;
    if constexpr (GROUPS == 1) {
        // one row per step: the wave's sums are the workgroup's for its
        // columns (16-byte aligned: the partial rows are 2C floats, C a
        // multiple of V >= 4)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int col = V * (64 * (NJ * part + j) + lane);
            if (col >= C) continue;
#pragma unroll
            for (int e = 0; e < V; e += 4) {
                *(float4*)(part_out + col + e) =
                    make_float4(aw[j][e], aw[j][e + 1], aw[j][e + 2], aw[j][e + 3]);
                *(float4*)(part_out + C + col + e) =
                    make_float4(ab[j][e], ab[j][e + 1], ab[j][e + 2], ab[j][e + 3]);
            }
        }
        return;
    }
    // the 8 waves' column sums [dweight | dbias], each wave in its own slot,
    // then, per column, the groups' sums of its part added in group order
    float* mine = red + wave * SLOT;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const int i = V * (lane + 64 * j) + e;
            mine[i] = aw[j][e];
            mine[COLS + i] = ab[j][e];
        }
    __syncthreads();
    for (int i = tid; i < C; i += LN_NT) {
        // column i sits in part h at index il (one part with one wave per row)
        const int h = WPR == 1 ? 0 : i / COLS, il = WPR == 1 ? i : i - h * COLS;
        float sw = red[h * SLOT + il], sb = red[h * SLOT + COLS + il];
#pragma unroll
        for (int g = 1; g < GROUPS; ++g) {
            sw += red[(g * WPR + h) * SLOT + il];
            sb += red[(g * WPR + h) * SLOT + COLS + il];
        }
        part_out[i] = sw;
        part_out[C + i] = sb;
    }
}

// dweight[i] += sum_g partial[g][i], dbias[i] += sum_g partial[g][C + i]:
// 32 columns per workgroup; 32 groups of workgroup partials g = q, q + 32, ...
// each summed in order (all of a thread's loads issued before its adds),
// then the 32 group sums in order.
constexpr int RED_COLS = 32, RED_GROUPS = 32, RED_BATCH = 8;

template <typename T>
__global__ __launch_bounds__(RED_COLS * RED_GROUPS) void ln_bwd_reduce(LNParams p, int G) {
    __shared__ float s[RED_GROUPS][RED_COLS];
    const int c = threadIdx.x % RED_COLS, q = threadIdx.x / RED_COLS;
    const int col = blockIdx.x * RED_COLS + c;   // over 2C: dweight then dbias
    const int C2 = 2 * p.C;
    float acc = 0.f;
    for (int g0 = q; g0 < G; g0 += RED_BATCH * RED_GROUPS) {
        float v[RED_BATCH];
#pragma unroll
        for (int k = 0; k < RED_BATCH; ++k) {
            const int g = g0 + k * RED_GROUPS;
            v[k] = (g < G && col < C2) ? p.partial[(long long)g * C2 + col] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < RED_BATCH; ++k) acc += v[k];
    }
    s[q][c] = acc;
    __syncthreads();
    if (q == 0 && col < C2) {
        float t = s[0][c];
#pragma unroll
        for (int k = 1; k < RED_GROUPS; ++k) t += s[k][c];
        T* out = col < p.C ? (T*)p.dweight + col : (T*)p.dbias + (col - p.C);
        *out = from_f32<T>(to_f32(*out) + t);
    }
}

// ---- any shape / alignment --------------------------------------------------
// dinp: one wave per row, two passes over the row with a stride of 64.
template <typename T>
__global__ __launch_bounds__(256) void ln_generic_dinp(LNParams p) {
    const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, C = p.C;
    if (r >= p.BT) return;
    const T* d = (const T*)p.dout + r * C;
    const T* x = (const T*)p.inp + r * C;
    const T* w = (const T*)p.weight;
    const float m = to_f32(((const T*)p.mean)[r]), s = to_f32(((const T*)p.rstd)[r]);
    float sa = 0.f, sb = 0.f;
    for (int i = lane; i < C; i += 64) {
        const float dn = to_f32(w[i]) * to_f32(d[i]);
        sa += dn;
        sb += dn * (to_f32(x[i]) - m) * s;
    }
    const float a = wave_sum(sa) / (float)C, b = wave_sum(sb) / (float)C;
    T* g = (T*)p.dinp + r * C;
    for (int i = lane; i < C; i += 64) {
        const float nrm = (to_f32(x[i]) - m) * s;
        const float dn = to_f32(w[i]) * to_f32(d[i]);
        g[i] = from_f32<T>(to_f32(g[i]) + (dn - a - nrm * b) * s);
    }
}

// dweight / dbias partials: one thread per column over a band of `band`
// consecutive rows (in order), band y writing partial row y [dweight |
// dbias]; ln_bwd_reduce then adds the bands in its fixed order, adds the old
// values and rounds once, as after the row kernel.
template <typename T>
__global__ __launch_bounds__(256) void ln_generic_dwb(LNParams p, long long band) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= p.C) return;
    const long long r0 = (long long)blockIdx.y * band;
    const long long r1 = r0 + band < p.BT ? r0 + band : p.BT;
    float sw = 0.f, sb = 0.f;
    for (long long r = r0; r < r1; ++r) {
        const float dv = to_f32(((const T*)p.dout)[r * p.C + i]);
        const float nrm = (to_f32(((const T*)p.inp)[r * p.C + i]) - to_f32(((const T*)p.mean)[r])) *
                          to_f32(((const T*)p.rstd)[r]);
        sb += dv;
        sw += nrm * dv;
    }
    float* out = p.partial + (long long)blockIdx.y * 2 * p.C;
    out[i] = sw;
    out[p.C + i] = sb;
}

template <typename T, int NJ, int WPR = 1>
hipError_t launch_rows(const LNParams& p, int G, hipStream_t s) {
    hipLaunchKernelGGL((ln_bwd_rows<T, NJ, WPR>), dim3(G), dim3(LN_NT), 0, s, p);
    hipLaunchKernelGGL((ln_bwd_reduce<T>), dim3((2 * p.C + RED_COLS - 1) / RED_COLS),
                       dim3(RED_COLS * RED_GROUPS), 0, s, p, G);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_ln(const LNParams& p, int G, LNLayout k, hipStream_t s) {
    if (k.nj == 0) {
        // G bands of whole rows (the last one shorter), one partial row each
        const long long band = (p.BT + G - 1) / G;
        const int bands = (int)((p.BT + band - 1) / band);
        hipLaunchKernelGGL(ln_generic_dinp<T>, dim3((unsigned)((p.BT + 3) / 4)), dim3(256), 0, s, p);
        hipLaunchKernelGGL(ln_generic_dwb<T>, dim3((p.C + 255) / 256, bands), dim3(256), 0, s, p,
                           band);
        hipLaunchKernelGGL((ln_bwd_reduce<T>), dim3((2 * p.C + RED_COLS - 1) / RED_COLS),
                           dim3(RED_COLS * RED_GROUPS), 0, s, p, bands);
        return hipGetLastError();
    }
    if (k.wpr == 1) {
        if (k.nj == 1) return launch_rows<T, 1>(p, G, s);
        if (k.nj == 2) return launch_rows<T, 2>(p, G, s);
        if (k.nj == 4) return launch_rows<T, 4>(p, G, s);
        if constexpr (sizeof(T) == 4)
            if (k.nj == 8) return launch_rows<T, 8>(p, G, s);
    }
    if constexpr (sizeof(T) == 2) {
        if (k.nj == 4 && k.wpr == 2) return launch_rows<T, 4, 2>(p, G, s);
        if (k.nj == 4 && k.wpr == 4) return launch_rows<T, 4, 4>(p, G, s);
        if (k.nj == 4 && k.wpr == 8) return launch_rows<T, 4, 8>(p, G, s);
    } else {
        if (k.nj == 8 && k.wpr == 2) return launch_rows<T, 8, 2>(p, G, s);
        if (k.nj == 4 && k.wpr == 8) return launch_rows<T, 4, 8>(p, G, s);
        if (k.nj == 8 && k.wpr == 8) return launch_rows<T, 8, 8>(p, G, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

LNLayout ln_layout(int dtype, int C) {
    const int V = dtype == 1 ? 8 : 4;
    // vectors per lane of one wave: 8 fit the registers (one row in flight)
    // for fp32; for bf16 they would spill, so wider bf16 rows take 2 or 4
    // waves of 4.  With several rows per workgroup step the LDS (the waves'
    // column sums plus the weight row) caps that at bf16 C <= 8192, fp32
    // C <= 4096; wider rows take all 8 waves of the workgroup (one row per
    // step, no column sums in LDS) up to C = 16384.
    const int nmax = dtype == 1 ? 4 : 8, wmax = dtype == 1 ? 4 : 2;
    if (C % V != 0) return LNLayout{0, 1};
    const int nv = C / V;
    for (int nj = 1; nj <= nmax; nj *= 2)
        if (nv <= 64 * nj) return LNLayout{nj, 1};
    for (int wpr = 2; wpr <= wmax; wpr *= 2)
        if (nv <= 64 * nmax * wpr) return LNLayout{nmax, wpr};
    for (int nj = 4; nj <= nmax; nj *= 2)
        if (nv <= 64 * nj * LN_NW) return LNLayout{nj, LN_NW};
    return LNLayout{0, 1};
}

int ln_vectors_per_lane(int dtype, int C) { return ln_layout(dtype, C).nj; }

hipError_t launch_layernorm_backward(int dtype, const LNParams& p, int G, LNLayout k,
                                     hipStream_t s) {
    if (dtype == 1) return launch_ln<bf16_t>(p, G, k, s);
    return launch_ln<float>(p, G, k, s);
}

}  // namespace mmb
