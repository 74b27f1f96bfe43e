// mmb_api.hip -- the C ABI of libmmb.so (declared in include/mmb.h):
// argument checks, path choice, the split-K / launch-order planner and the
// per-(device, stream) workspace.
//
// Operation: llm.c page "dev/cuda/matmul_backward.cu", launcher
// matmul_backward1 -- dinp and dweight GEMMs with beta = 1, dbias assigned
// when the pointer is not NULL.  That launcher aborts the process on errors;
// this one returns a status instead.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "../../include/mmb.h"
#include "mmb_internal.h"

namespace mmb {
namespace {

size_t elem_size(int dtype) { return dtype == MMB_BF16 ? 2 : 4; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

int check(const void* dinp, const void* dweight, const void* dbias, const void* dout,
          const void* inp, const void* weight, int B, int T, int C, int OC, int dtype) {
    if (!dinp || !dweight || !dout || !inp || !weight) return MMB_ERR_NULL;
    if (B < 1 || T < 1 || C < 1 || OC < 1) return MMB_ERR_DIM;
    if (dtype != MMB_FP32 && dtype != MMB_BF16) return MMB_ERR_DTYPE;
    const long long BT = (long long)B * T;
    if (BT > 0x7fffffffLL) return MMB_ERR_OVERFLOW;
    const uintptr_t es = elem_size(dtype);
    auto R = [&](const void* p, long long n) {
        return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)n * es};
    };
    const Range outs[3] = {R(dinp, BT * C), R(dweight, (long long)OC * C),
                           dbias ? R(dbias, OC) : Range{0, 0}};
    const Range ins[3] = {R(dout, BT * OC), R(inp, BT * C), R(weight, (long long)OC * C)};
    const int n_out = dbias ? 3 : 2;
    for (int a = 0; a < n_out; ++a) {
        for (int b = a + 1; b < n_out; ++b)
            if (overlap(outs[a], outs[b])) return MMB_ERR_ALIAS;
        for (int b = 0; b < 3; ++b)
            if (overlap(outs[a], ins[b])) return MMB_ERR_ALIAS;
    }
    return MMB_OK;
}

// 1 when the MFMA tiles can take the call: 16-byte vectors never straddle a
// row end (C and OC multiples of the vector width) and every streamed buffer
// is 16-byte aligned.  dbias is written one element at a time.
int choose_path(const void* dinp, const void* dweight, const void* dout, const void* inp,
                const void* weight, int C, int OC, int dtype) {
    const int vec = dtype == MMB_BF16 ? 8 : 4;
    if (C % vec != 0 || OC % vec != 0) return 0;
    // the tiles address one 64-row K slab of an operand with 32-bit offsets
    if (C > (1 << 22) || OC > (1 << 22)) return 0;
    const void* ptrs[5] = {dinp, dweight, dout, inp, weight};
    for (const void* p : ptrs)
        if ((uintptr_t)p % 16 != 0) return 0;
    return 1;
}

// ---------------------------------------------------------------------------
// planner

int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

struct DeviceInfo {
    int cus = 0;
    int xcds = 1;
    int slots = 1;   // resident workgroups of the tile kernel per CU
};

// Dispatch model of a grid with `slots` resident workgroups per CU:
// workgroup i goes to XCD i % xcds, and each XCD starts its workgroups in
// order on whichever of its workgroup slots frees first.  Returns the
// makespan in cost units (one unit: one K iteration of a workgroup that
// shares its CU with slots - 1 others).
double simulate(const std::vector<int4>& units, const std::vector<double>& cost,
                const DeviceInfo& dev) {
    const int per = std::max(1, dev.cus / dev.xcds) * std::max(1, dev.slots);
    double worst = 0;
    std::vector<double> slots(per);
    for (int x = 0; x < dev.xcds; ++x) {
        std::fill(slots.begin(), slots.end(), 0.0);
        for (size_t i = x; i < units.size(); i += dev.xcds) {
            auto it = std::min_element(slots.begin(), slots.end());
            *it += cost[i];
        }
        worst = std::max(worst, *std::max_element(slots.begin(), slots.end()));
    }
    return worst;
}

struct Plan {
    TilesParams proto;            // pointers filled per call
    std::vector<int4> units;      // launch order
    int4* d_units = nullptr;      // device copy (owned by the plan cache)
    long long ws_floats = 0;
    long long ws_bias_floats = 0;
    int n_counters = 0;
    int forced_sw = 0, forced_si = 0;
};

// Order of one GEMM's units for L2 reuse inside an XCD: tiles that share an
// operand slab are adjacent.  dinp units share dout rows along tile_n;
// dweight units share the inp rows of one split and the dout columns of one
// tile_m, so they are ordered (split, tile_m, tile_n).
void gemm_units(int kind, const GemmPlan& g, std::vector<int4>& out) {
    if (kind == UNIT_DINP) {
        for (int m = 0; m < g.tiles_m; ++m)
            for (int s = 0; s < g.splits; ++s)
                for (int n = 0; n < g.tiles_n; ++n) out.push_back(make_int4(kind, m, n, s));
    } else {
        for (int s = 0; s < g.splits; ++s)
            for (int m = 0; m < g.tiles_m; ++m)
                for (int n = 0; n < g.tiles_n; ++n) out.push_back(make_int4(kind, m, n, s));
    }
}

int unit_iters(const GemmPlan& g, int split) {
    const long long k0 = (long long)split * g.kiters / g.splits;
    const long long k1 = (long long)(split + 1) * g.kiters / g.splits;
    return (int)(k1 - k0);
}

// Launch order: each XCD receives a contiguous run of the longer GEMM's units
// followed by a contiguous run of the shorter one's (longest first inside an
// XCD), interleaved so that workgroup i lands on XCD i % xcds.
std::vector<int4> order_units(const GemmPlan g[2], const DeviceInfo& dev) {
    std::vector<int4> a, b;
    const double la = (double)g[UNIT_DWEIGHT].kiters / g[UNIT_DWEIGHT].splits;
    const double lb = (double)g[UNIT_DINP].kiters / g[UNIT_DINP].splits;
    const int first = la >= lb ? UNIT_DWEIGHT : UNIT_DINP;
    gemm_units(first, g[first], a);
    gemm_units(1 - first, g[1 - first], b);
    const int X = dev.xcds;
    const size_t n = a.size() + b.size();
    std::vector<std::vector<int4>> seq(X);
    size_t pa = 0, pb = 0;
    bool ok = true;
    for (int x = 0; x < X; ++x) {
        const long long cnt = (long long)(n / X) + ((size_t)x < n % X ? 1 : 0);
        const long long ca = (long long)(a.size() / X) + ((size_t)x < a.size() % X ? 1 : 0);
        const long long cb = cnt - ca;
        if (cb < 0 || pb + cb > b.size()) { ok = false; break; }
        seq[x].insert(seq[x].end(), a.begin() + pa, a.begin() + pa + ca);
        seq[x].insert(seq[x].end(), b.begin() + pb, b.begin() + pb + cb);
        pa += ca;
        pb += cb;
    }
    std::vector<int4> out;
    out.reserve(n);
    if (!ok || pa != a.size() || pb != b.size()) {
        out = a;
        out.insert(out.end(), b.begin(), b.end());
        return out;
    }
    for (size_t i = 0; i < n; ++i) out.push_back(seq[i % X][i / X]);
    return out;
}

// Cost model, in units of one K-iteration of a full tile on one CU.  A unit
// costs its iterations plus a fixed prologue/epilogue.  Split tiles add
// their partials' traffic: every partial tile is written once and read once
// by the tile's last arriver; that traffic competes for HBM with everything
// else, so it is charged to the makespan at an effective bandwidth.
struct CostModel {
    double unit_overhead = 1.5;
    double hbm_bytes_per_us = 4.0e6;   // effective, below the 8 TB/s peak
    double mfma_efficiency = 0.7;
};

double iter_us(int dtype, const TileShape& ts) {
    // per-CU dense MFMA rate on gfx950 at 2.4 GHz: 4096 (bf16) / 256 (fp32)
    // flops per clock
    const double flops = 2.0 * ts.BM * ts.BN * ts.BK;
    const double per_clk = dtype == MMB_BF16 ? 4096.0 : 256.0;
    return flops / per_clk / 2400.0;
}

Plan build_plan(int dtype, int BT, int C, int OC, bool bias, const DeviceInfo& dev,
                int force_sw, int force_si) {
    const TileShape ts = tile_shape(dtype);
    GemmPlan g[2];
    // dweight[OC,C] += dout^T[OC,BT] . inp[BT,C]
    g[UNIT_DWEIGHT] = GemmPlan{OC, C, BT, cdiv(OC, ts.BM), cdiv(C, ts.BN), 1, cdiv(BT, ts.BK), 0, 0};
    // dinp[BT,C] += dout[BT,OC] . weight[OC,C]
    g[UNIT_DINP] = GemmPlan{BT, C, OC, cdiv(BT, ts.BM), cdiv(C, ts.BN), 1, cdiv(OC, ts.BK), 0, 0};

    const CostModel cm;
    // workgroups sharing a CU share its MFMA rate
    const double t_iter = iter_us(dtype, ts) * std::max(1, dev.slots) / cm.mfma_efficiency;
    int best_sw = 1, best_si = 1;
    double best = 1e300;
    const int max_sw = std::min(16, g[UNIT_DWEIGHT].kiters);
    const int max_si = std::min(8, g[UNIT_DINP].kiters);
    for (int sw = 1; sw <= max_sw; ++sw) {
        for (int si = 1; si <= max_si; ++si) {
            if (force_sw > 0 && sw != force_sw) continue;
            if (force_si > 0 && si != force_si) continue;
            GemmPlan h[2] = {g[0], g[1]};
            h[UNIT_DWEIGHT].splits = sw;
            h[UNIT_DINP].splits = si;
            std::vector<int4> u = order_units(h, dev);
            std::vector<double> cost(u.size());
            for (size_t i = 0; i < u.size(); ++i)
                cost[i] = unit_iters(h[u[i].x], u[i].w) + cm.unit_overhead;
            double t = simulate(u, cost, dev);
            double partial_bytes = 0;
            for (int k = 0; k < 2; ++k)
                if (h[k].splits > 1)
                    partial_bytes += 2.0 * h[k].splits * h[k].tiles_m * h[k].tiles_n * ts.BM *
                                     ts.BN * 4.0;
            t += partial_bytes / cm.hbm_bytes_per_us / t_iter;
            if (t < best - 1e-9) {
                best = t;
                best_sw = sw;
                best_si = si;
            }
        }
    }
    if (force_sw > 0) best_sw = std::min(force_sw, max_sw);
    if (force_si > 0) best_si = std::min(force_si, max_si);
    g[UNIT_DWEIGHT].splits = best_sw;
    g[UNIT_DINP].splits = best_si;

    Plan p;
    std::memset(&p.proto, 0, sizeof(p.proto));
    long long ws = 0;
    int tiles = 0;
    for (int k = 0; k < 2; ++k) {
        g[k].tile_base = tiles;
        g[k].ws_base = ws;
        if (g[k].splits > 1) {
            tiles += g[k].tiles_m * g[k].tiles_n;
            ws += (long long)g[k].tiles_m * g[k].tiles_n * g[k].splits * ts.BM * ts.BN;
        }
    }
    p.ws_floats = ws;
    p.ws_bias_floats = bias && g[UNIT_DWEIGHT].splits > 1
                           ? (long long)g[UNIT_DWEIGHT].tiles_m * g[UNIT_DWEIGHT].splits * ts.BM
                           : 0;
    p.n_counters = tiles;
    p.proto.BT = BT;
    p.proto.C = C;
    p.proto.OC = OC;
    p.proto.g[0] = g[0];
    p.proto.g[1] = g[1];
    p.units = order_units(g, dev);
    p.proto.n_units = (int)p.units.size();
    return p;
}

// ---------------------------------------------------------------------------
// state: plans per (device, shape) and workspaces per (device, stream)

struct Workspace {
    void* counters = nullptr;
    size_t counter_bytes = 0;
    void* partials = nullptr;
    size_t partial_bytes = 0;
};

std::mutex g_mu;
std::map<int, DeviceInfo> g_dev;
std::map<std::tuple<int, int, int, int, int, bool>, Plan> g_plans;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

int env_int(const char* name) {
    const char* v = std::getenv(name);
    return v ? std::atoi(v) : 0;
}

int device_info(int dev, DeviceInfo* out) {
    auto it = g_dev.find(dev);
    if (it != g_dev.end()) {
        *out = it->second;
        return MMB_OK;
    }
    DeviceInfo d;
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return MMB_ERR_HIP;
    // MI355X in its single-partition mode spreads 256 CUs over 8 XCDs, each
    // with its own L2; smaller partitions expose one XCD's CUs.
    d.xcds = d.cus >= 128 ? 8 : 1;
    g_dev[dev] = d;
    *out = d;
    return MMB_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int get_plan(int dev, int dtype, int BT, int C, int OC, bool bias, Plan** out) {
    // MMB_SPLITS_DWEIGHT / MMB_SPLITS_DINP force the split counts (tuning
    // sweeps); 0 or unset lets the planner choose.
    const int fsw = env_int("MMB_SPLITS_DWEIGHT");
    const int fsi = env_int("MMB_SPLITS_DINP");
    const auto key = std::make_tuple(dev, dtype, BT, C, OC, bias);
    auto it = g_plans.find(key);
    if (it != g_plans.end()) {
        if (it->second.forced_sw == fsw && it->second.forced_si == fsi) {
            *out = &it->second;
            return MMB_OK;
        }
        // a kernel of the old plan may still read its unit table
        if (hipDeviceSynchronize() != hipSuccess) return MMB_ERR_HIP;
        (void)hipFree(it->second.d_units);
        g_plans.erase(it);
    }
    DeviceInfo di;
    int st = device_info(dev, &di);
    if (st != MMB_OK) return st;
    di.slots = tiles_resident(dtype);
    Plan p = build_plan(dtype, BT, C, OC, bias, di, fsw, fsi);
    p.forced_sw = fsw;
    p.forced_si = fsi;
    const size_t ub = p.units.size() * sizeof(int4);
    if (hipMalloc(&p.d_units, ub) != hipSuccess) return MMB_ERR_NOMEM;
    if (hipMemcpy(p.d_units, p.units.data(), ub, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(p.d_units);
        return MMB_ERR_HIP;
    }
    p.proto.units = p.d_units;
    auto res = g_plans.emplace(key, std::move(p));
    *out = &res.first->second;
    return MMB_OK;
}

// Workspace: two allocations per (device, stream).  `counters` holds one
// arrival counter per split tile and is only ever used for counters: it is
// zeroed when allocated and every counter is reset by the last arriver of
// its tile, so it is all zero at rest whatever plan ran before.  `partials`
// holds [bias partials fp32][tile partials fp32] (each part 256-byte
// aligned) and needs no initial value.
int grow(void** buf, size_t* cap, size_t need, bool zero, hipStream_t s) {
    if (need <= *cap) return MMB_OK;
    if (*buf) {
        if (hipStreamSynchronize(s) != hipSuccess) return MMB_ERR_HIP;
        (void)hipFree(*buf);
        *buf = nullptr;
        *cap = 0;
    }
    const size_t want = std::max(need, *cap * 2);
    if (hipMalloc(buf, want) != hipSuccess) {
        *buf = nullptr;
        return MMB_ERR_NOMEM;
    }
    *cap = want;
    if (zero && hipMemsetAsync(*buf, 0, want, s) != hipSuccess) return MMB_ERR_HIP;
    return MMB_OK;
}

int get_workspace(int dev, hipStream_t s, const Plan& p, TilesParams* tp) {
    const size_t cb = (size_t)p.n_counters * 4;
    const size_t bb = align_up((size_t)p.ws_bias_floats * 4, 256);
    const size_t wb = align_up((size_t)p.ws_floats * 4, 256);
    Workspace& w = g_ws[{dev, s}];
    int st = grow(&w.counters, &w.counter_bytes, cb, true, s);
    if (st != MMB_OK) return st;
    st = grow(&w.partials, &w.partial_bytes, bb + wb, false, s);
    if (st != MMB_OK) return st;
    char* b = (char*)w.partials;
    tp->counters = (int*)w.counters;
    tp->ws_bias = (float*)b;
    tp->ws = (float*)(b + bb);
    return MMB_OK;
}

int backward_impl(void* dinp, void* dweight, void* dbias, const void* dout, const void* inp,
                  const void* weight, int B, int T, int C, int OC, int dtype, hipStream_t s) {
    int st = check(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype);
    if (st != MMB_OK) return st;
    const int BT = B * T;
    if (!choose_path(dinp, dweight, dout, inp, weight, C, OC, dtype)) {
        return launch_generic(dtype, dinp, dweight, dbias, dout, inp, weight, BT, C, OC, s) ==
                       hipSuccess
                   ? MMB_OK
                   : MMB_ERR_HIP;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MMB_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    Plan* plan = nullptr;
    st = get_plan(dev, dtype, BT, C, OC, dbias != nullptr, &plan);
    if (st != MMB_OK) return st;
    TilesParams tp = plan->proto;
    st = get_workspace(dev, s, *plan, &tp);
    if (st != MMB_OK) return st;
    tp.dinp = dinp;
    tp.dweight = dweight;
    tp.dbias = dbias;
    tp.dout = dout;
    tp.inp = inp;
    tp.weight = weight;
    return launch_tiles(dtype, tp, s) == hipSuccess ? MMB_OK : MMB_ERR_HIP;
}

}  // namespace
}  // namespace mmb

extern "C" {

int mmb_check_args(const void* dinp, const void* dweight, const void* dbias, const void* dout,
                   const void* inp, const void* weight, int B, int T, int C, int OC, int dtype) {
    return mmb::check(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype);
}

int mmb_path(const void* dinp, const void* dweight, const void* dbias, const void* dout,
             const void* inp, const void* weight, int B, int T, int C, int OC, int dtype) {
    const int st = mmb::check(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype);
    if (st != MMB_OK) return st;
    return mmb::choose_path(dinp, dweight, dout, inp, weight, C, OC, dtype);
}

int mmb_backward_stream(void* dinp, void* dweight, void* dbias, const void* dout,
                        const void* inp, const void* weight, int B, int T, int C, int OC,
                        int dtype, void* stream) {
    return mmb::backward_impl(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype,
                              (hipStream_t)stream);
}

int mmb_backward(void* dinp, void* dweight, void* dbias, const void* dout, const void* inp,
                 const void* weight, int B, int T, int C, int OC, int dtype) {
    return mmb::backward_impl(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype,
                              nullptr);
}

const char* mmb_strerror(int status) {
    switch (status) {
        case MMB_OK: return "success";
        case MMB_ERR_NULL: return "a required pointer is NULL (only dbias may be NULL)";
        case MMB_ERR_DIM: return "B, T, C and OC must all be >= 1";
        case MMB_ERR_DTYPE: return "dtype must be MMB_FP32 (0) or MMB_BF16 (1)";
        case MMB_ERR_OVERFLOW: return "B*T must be below 2^31";
        case MMB_ERR_ALIAS: return "an output buffer overlaps another buffer";
        case MMB_ERR_HIP: return "a HIP runtime call or kernel launch failed";
        case MMB_ERR_NOMEM: return "the workspace could not be allocated";
        default: return "unknown mmb status";
    }
}

int mmb_plan_units(int B, int T, int C, int OC, int dtype, int has_bias, int num_cus,
                   int* splits, int* units, int max_units) {
    if (B < 1 || T < 1 || C < 1 || OC < 1 || num_cus < 1) return MMB_ERR_DIM;
    if (dtype != MMB_FP32 && dtype != MMB_BF16) return MMB_ERR_DTYPE;
    if ((long long)B * T > 0x7fffffffLL) return MMB_ERR_OVERFLOW;
    if (!splits) return MMB_ERR_NULL;
    mmb::DeviceInfo di;
    di.cus = num_cus;
    di.xcds = num_cus >= 128 ? 8 : 1;
    di.slots = mmb::tiles_resident(dtype);
    const mmb::Plan p = mmb::build_plan(dtype, B * T, C, OC, has_bias != 0, di,
                                        mmb::env_int("MMB_SPLITS_DWEIGHT"),
                                        mmb::env_int("MMB_SPLITS_DINP"));
    splits[0] = p.proto.g[mmb::UNIT_DWEIGHT].splits;
    splits[1] = p.proto.g[mmb::UNIT_DINP].splits;
    if (units) {
        const int n = std::min<int>(max_units, (int)p.units.size());
        for (int i = 0; i < n; ++i) {
            units[4 * i + 0] = p.units[i].x;
            units[4 * i + 1] = p.units[i].y;
            units[4 * i + 2] = p.units[i].z;
            units[4 * i + 3] = p.units[i].w;
        }
    }
    return (int)p.units.size();
}

int mmb_tile_shape(int dtype, int* shape) {
    if (dtype != MMB_FP32 && dtype != MMB_BF16) return MMB_ERR_DTYPE;
    if (!shape) return MMB_ERR_NULL;
    const mmb::TileShape ts = mmb::tile_shape(dtype);
    shape[0] = ts.BM;
    shape[1] = ts.BN;
    shape[2] = ts.BK;
    return MMB_OK;
}

int mmb_release(void) {
    std::lock_guard<std::mutex> lock(mmb::g_mu);
    int prev = 0;
    (void)hipGetDevice(&prev);
    int st = MMB_OK;
    for (auto& kv : mmb::g_ws) {
        (void)hipSetDevice(kv.first.first);
        if (hipDeviceSynchronize() != hipSuccess) st = MMB_ERR_HIP;
        if (kv.second.counters) (void)hipFree(kv.second.counters);
        if (kv.second.partials) (void)hipFree(kv.second.partials);
    }
    mmb::g_ws.clear();
    for (auto& kv : mmb::g_plans) {
        (void)hipSetDevice(std::get<0>(kv.first));
        if (hipDeviceSynchronize() != hipSuccess) st = MMB_ERR_HIP;
        (void)hipFree(kv.second.d_units);
    }
    mmb::g_plans.clear();
    (void)hipSetDevice(prev);
    return st;
}

}  // extern "C"
