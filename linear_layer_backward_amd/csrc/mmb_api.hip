// mmb_api.hip -- the C ABI of libmmb.so (declared in include/mmb.h):
// argument checks, path choice, the split-K / launch-order planner and the
// per-(device, stream) workspace.
//
// Operation: llm.c page "dev/cuda/matmul_backward.cu", launcher
// matmul_backward1 -- dinp and dweight GEMMs with beta = 1, dbias assigned
// when the pointer is not NULL.  That launcher aborts the process on errors;
// this one returns a status instead.
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <mutex>
#include <queue>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "../../include/mmb.h"
#include "mmb_internal.h"
#include "mmb_plan.h"

// Device memory of the allocation-free entry point (mmb_backward_noalloc):
// split-K counters, the work list and the split partials of one call.  Each
// device the library runs on holds its own copy until the process ends; host
// code reaches it only through the per-device address hipGetSymbolAddress
// returns (noalloc_scratch below), never through this name.
static __device__ __align__(256) char scratch[MMB_NOALLOC_SCRATCH_BYTES];

namespace mmb {
namespace {

size_t elem_size(int dtype) { return dtype == MMB_BF16 ? 2 : 4; }

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }

int check(const void* dinp, const void* dweight, const void* dbias, const void* dout,
          const void* inp, const void* weight, int B, int T, int C, int OC, int dtype) {
    if (!dinp || !dweight || !dout || !inp || !weight) return MMB_ERR_NULL;
    if (B < 1 || T < 1 || C < 1 || OC < 1) return MMB_ERR_DIM;
    if (dtype != MMB_FP32 && dtype != MMB_BF16) return MMB_ERR_DTYPE;
    const long long BT = (long long)B * T;
    if (BT > 0x7fffffffLL) return MMB_ERR_OVERFLOW;
    const uintptr_t es = elem_size(dtype);
    auto R = [&](const void* p, long long n) {
        return Span{(uintptr_t)p, (uintptr_t)p + (uintptr_t)n * es};
    };
    const Span outs[3] = {R(dinp, BT * C), R(dweight, (long long)OC * C),
                          dbias ? R(dbias, OC) : Span{0, 0}};
    const Span ins[3] = {R(dout, BT * OC), R(inp, BT * C), R(weight, (long long)OC * C)};
    const int n_out = dbias ? 3 : 2;
    for (int a = 0; a < n_out; ++a) {
        for (int b = a + 1; b < n_out; ++b)
            if (overlap(outs[a], outs[b])) return MMB_ERR_ALIAS;
        for (int b = 0; b < 3; ++b)
            if (overlap(outs[a], ins[b])) return MMB_ERR_ALIAS;
    }
    return MMB_OK;
}

// Forward: out [BT,OC] = inp [BT,C] . weight^T + bias; out may not overlap
// an input.
int check_fwd(const void* out, const void* inp, const void* weight, const void* bias, int B,
              int T, int C, int OC, int dtype) {
    if (!out || !inp || !weight) return MMB_ERR_NULL;
    if (B < 1 || T < 1 || C < 1 || OC < 1) return MMB_ERR_DIM;
    if (dtype != MMB_FP32 && dtype != MMB_BF16) return MMB_ERR_DTYPE;
    const long long BT = (long long)B * T;
    if (BT > 0x7fffffffLL) return MMB_ERR_OVERFLOW;
    const uintptr_t es = elem_size(dtype);
    auto R = [&](const void* p, long long n) {
        return Span{(uintptr_t)p, (uintptr_t)p + (uintptr_t)n * es};
    };
    const Span o = R(out, BT * OC);
    const Span ins[3] = {R(inp, BT * C), R(weight, (long long)OC * C),
                         bias ? R(bias, OC) : Span{0, 0}};
    for (const Span& r : ins)
        if (overlap(o, r)) return MMB_ERR_ALIAS;
    return MMB_OK;
}

// A tensor the tiles can read or write in place: 16-byte aligned (the tiles
// move 16-byte vectors).  One aligned to its element size but not to 16
// bytes goes through a packed copy; one not even aligned to its element size
// sends the call to the generic path.
bool aligned16(const void* p) { return (uintptr_t)p % 16 == 0; }
bool elem_aligned(const void* p, int dtype) { return (uintptr_t)p % elem_size(dtype) == 0; }

// Path of a call: 0 the generic kernels (C or OC too large for the tiles'
// 32-bit offsets, or a streamed buffer not aligned to its element size), 1
// the MFMA tiles on the caller's buffers, 2 the MFMA tiles with some tensors
// through packed copies (rows that are not whole 16-byte vectors, or a
// buffer off the 16-byte alignment; see Packing).  NULL entries (no bias)
// are skipped; dbias is written one element at a time and never matters.
int choose_path_of(const void* const* ptrs, int n, int C, int OC, int dtype) {
    // the tiles address one 64-row K slab of an operand with 32-bit offsets
    if (C > (1 << 22) || OC > (1 << 22)) return 0;
    const int vec = dtype == MMB_BF16 ? 8 : 4;
    bool direct = C % vec == 0 && OC % vec == 0;
    for (int i = 0; i < n; ++i) {
        if (!ptrs[i]) continue;
        if (!elem_aligned(ptrs[i], dtype)) return 0;
        direct = direct && aligned16(ptrs[i]);
    }
    return direct ? 1 : 2;
}

int choose_path(const void* dinp, const void* dweight, const void* dout, const void* inp,
                const void* weight, int C, int OC, int dtype) {
    const void* ptrs[5] = {dinp, dweight, dout, inp, weight};
    return choose_path_of(ptrs, 5, C, OC, dtype);
}

int choose_path_fwd(const void* out, const void* inp, const void* weight, const void* bias, int C,
                    int OC, int dtype) {
    const void* ptrs[4] = {out, inp, weight, bias};
    return choose_path_of(ptrs, 4, C, OC, dtype);
}

// Packed copies: a tensor whose rows are not whole 16-byte vectors (the
// OC-wide dout, out and bias when OC is ragged; the C-wide inp, weight, dinp
// and dweight when C is) or whose address is not 16-byte aligned is copied
// into a 16-byte aligned, zero-padded row pitch in the workspace (the pads add
// nothing to any sum, and the epilogues write only the logical columns); the
// tiles run on the copies with those pitches, and the outputs among them
// (dinp, dweight, out) are copied back.  out is assigned by the forward, so
// its copy starts with no contents.  Offsets into one buffer, each part
// 256-byte aligned.
enum PackedTensor { P_DOUT, P_INP, P_WEIGHT, P_DINP, P_DWEIGHT, P_OUT, P_BIAS, P_COUNT };
struct Packing {
    bool on[P_COUNT] = {};
    size_t off[P_COUNT] = {};
    long long ldo = 0, ldc = 0;   // row pitches the tiles use (OC-wide, C-wide tensors)
    size_t bytes = 0;
};

// ptrs[t]: the caller's tensor t, or NULL where the call has none (the
// backward has no out or bias to pack, the forward no dout, dinp, dweight).
Packing plan_packing(int dtype, long long BT, int C, int OC, const void* const ptrs[P_COUNT]) {
    const int vec = dtype == MMB_BF16 ? 8 : 4;
    const size_t es = elem_size(dtype);
    Packing k;
    k.ldo = ((long long)OC + vec - 1) / vec * vec;
    k.ldc = ((long long)C + vec - 1) / vec * vec;
    const bool oc_wide[P_COUNT] = {true, false, false, false, false, true, true};
    const long long rows[P_COUNT] = {BT, BT, OC, BT, OC, BT, 1};
    for (int t = 0; t < P_COUNT; ++t) {
        if (!ptrs[t]) continue;
        const bool ragged = oc_wide[t] ? OC % vec != 0 : C % vec != 0;
        if (!ragged && aligned16(ptrs[t])) continue;
        k.on[t] = true;
        k.off[t] = k.bytes;
        k.bytes += (size_t)rows[t] * (size_t)(oc_wide[t] ? k.ldo : k.ldc) * es;
        k.bytes = (k.bytes + 255) / 256 * 256;
    }
    return k;
}

Packing plan_packing_bwd(int dtype, long long BT, int C, int OC, const void* dinp,
                         const void* dweight, const void* dout, const void* inp,
                         const void* weight) {
    const void* ptrs[P_COUNT] = {dout, inp, weight, dinp, dweight, nullptr, nullptr};
    return plan_packing(dtype, BT, C, OC, ptrs);
}

Packing plan_packing_fwd(int dtype, long long BT, int C, int OC, const void* out, const void* inp,
                         const void* weight, const void* bias) {
    const void* ptrs[P_COUNT] = {nullptr, inp, weight, nullptr, nullptr, out, bias};
    return plan_packing(dtype, BT, C, OC, ptrs);
}

// Enqueue the packing copies on `s` and point the tile parameters at them
// (tp holds the caller's pointers on entry).
hipError_t pack_operands(const Packing& k, char* base, TilesParams* tp, int dtype, hipStream_t s) {
    const int es = (int)elem_size(dtype);
    const long long BT = tp->BT;
    const void** fields[P_COUNT] = {&tp->dout, &tp->inp, &tp->weight, (const void**)&tp->dinp,
                                    (const void**)&tp->dweight, (const void**)&tp->out,
                                    &tp->bias};
    const long long rows[P_COUNT] = {BT, BT, tp->OC, BT, tp->OC, BT, 1};
    const bool oc_wide[P_COUNT] = {true, false, false, false, false, true, true};
    for (int t = 0; t < P_COUNT; ++t) {
        if (!k.on[t]) continue;
        const long long pitch = oc_wide[t] ? k.ldo : k.ldc;
        const int width = oc_wide[t] ? tp->OC : tp->C;
        if (t != P_OUT) {   // out is assigned: nothing to copy in
            const hipError_t e = launch_pack(base + k.off[t], pitch, *fields[t], width, rows[t],
                                             width, es, s);
            if (e != hipSuccess) return e;
        }
        *fields[t] = base + k.off[t];
    }
    tp->ldo = (int)k.ldo;
    tp->ldc = (int)k.ldc;
    return hipSuccess;
}

// Copy the packed outputs (dinp, dweight; out) back to the caller's buffers.
hipError_t unpack_outputs(const Packing& k, const char* base, void* dinp, void* dweight, void* out,
                          long long BT, int C, int OC, int dtype, hipStream_t s) {
    const int es = (int)elem_size(dtype);
    hipError_t e = hipSuccess;
    if (k.on[P_DINP]) e = launch_unpack(dinp, C, base + k.off[P_DINP], k.ldc, BT, C, es, s);
    if (e == hipSuccess && k.on[P_DWEIGHT])
        e = launch_unpack(dweight, C, base + k.off[P_DWEIGHT], k.ldc, OC, C, es, s);
    if (e == hipSuccess && k.on[P_OUT])
        e = launch_unpack(out, OC, base + k.off[P_OUT], k.ldo, BT, OC, es, s);
    return e;
}

// ---------------------------------------------------------------------------
// tuning overrides

// The MMB_* tuning variables (split overrides, planner constants, plan trace,
// LayerNorm workgroup count) are read from the environment once, when the
// library is loaded, so that a variable set later in the process cannot
// change production plans; mmb_set_tuning replaces a value explicitly
// (tuning sweeps, tests).  Guarded by g_mu.
enum Tune { T_SPLITS_DWEIGHT, T_SPLITS_DINP, T_SPLITS_FWD, T_PLAN_MODEL, T_PLAN_TRACE,
            T_LN_WORKGROUPS, T_COUNT };
const char* const kTuneNames[T_COUNT] = {"MMB_SPLITS_DWEIGHT", "MMB_SPLITS_DINP",
                                         "MMB_SPLITS_FWD",     "MMB_PLAN_MODEL",
                                         "MMB_PLAN_TRACE",     "MMB_LN_WORKGROUPS"};

struct Tuning {
    bool set[T_COUNT];
    std::string val[T_COUNT];
    const char* get(int k) const { return set[k] ? val[k].c_str() : nullptr; }
};

Tuning load_tuning() {
    Tuning t;
    for (int k = 0; k < T_COUNT; ++k) {
        const char* e = std::getenv(kTuneNames[k]);
        t.set[k] = e != nullptr;
        t.val[k] = e ? e : "";
    }
    return t;
}

std::mutex g_mu;                  // guards the tuning values, plans and workspaces
Tuning g_tune = load_tuning();

PlanOptions plan_options(const Tuning& t, bool fwd) {
    PlanOptions o;
    if (fwd) {
        o.force_i = parse_splits(t.get(T_SPLITS_FWD));
    } else {
        o.force_w = parse_splits(t.get(T_SPLITS_DWEIGHT));
        o.force_i = parse_splits(t.get(T_SPLITS_DINP));
    }
    o.model = t.get(T_PLAN_MODEL);
    o.trace = t.get(T_PLAN_TRACE) != nullptr;
    return o;
}

// A profiler range (roctx) around planning and launching, so that a trace
// shows host cost next to kernel time; free when no profiler is attached.
struct TraceRange {
    explicit TraceRange(const char* what) { roctxRangePushA(what); }
    ~TraceRange() { roctxRangePop(); }
    TraceRange(const TraceRange&) = delete;
    TraceRange& operator=(const TraceRange&) = delete;
};

// ---------------------------------------------------------------------------
// state: plans per (device, shape, overrides) and workspaces per (device,
// stream).  Nothing here waits for the device: a plan is never replaced (a
// change of the overrides makes a new one), workspaces grow with
// stream-ordered allocations, and a plan's work list reaches each stream with
// an asynchronous copy on that stream.  Only mmb_release synchronises.

// Device memory in stream order where the device supports memory pools
// (hipMallocAsync / hipFreeAsync), else plain hipMalloc; buffers of the
// second kind that a kernel may still read are kept until mmb_release.
struct DevAlloc {
    void* ptr = nullptr;
    bool async = false;
};

struct Workspace {
    DevAlloc counters;
    size_t counter_bytes = 0;
    DevAlloc partials;
    size_t partial_bytes = 0;
    DevAlloc packed;              // padded copies of ragged operands
    size_t packed_bytes = 0;
    std::map<const void*, DevAlloc> tables;   // this stream's copy of each plan's work list
};

struct PlanEntry {
    Plan plan;
    int4* host_units = nullptr;   // pinned copy of the work list, source of the uploads
};

// key: device, dtype, BT, C, OC, bias, forward (1) or backward (0), and the
// override string the plan was made with
typedef std::tuple<int, int, int, int, int, bool, int, std::string> PlanKey;
std::map<int, DeviceInfo> g_dev;
std::map<int, bool> g_pools;       // device -> supports hipMallocAsync
std::map<PlanKey, PlanEntry> g_plans;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::vector<std::pair<int, void*>> g_retired;   // (device, buffer) freed at release

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
    set_topology(&d);
    int pools = 0;
    if (hipDeviceGetAttribute(&pools, hipDeviceAttributeMemoryPoolsSupported, dev) != hipSuccess)
        pools = 0;
    g_pools[dev] = pools != 0;
    g_dev[dev] = d;
    *out = d;
    return MMB_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int dev_alloc(int dev, DevAlloc* a, size_t bytes, hipStream_t s) {
    a->ptr = nullptr;
    a->async = g_pools[dev];
    const hipError_t e = a->async ? hipMallocAsync(&a->ptr, bytes, s) : hipMalloc(&a->ptr, bytes);
    if (e != hipSuccess) {
        a->ptr = nullptr;
        return MMB_ERR_NOMEM;
    }
    return MMB_OK;
}

// Free a buffer that work already enqueued on `s` may still use.
void dev_retire(int dev, DevAlloc* a, hipStream_t s) {
    if (!a->ptr) return;
    if (a->async)
        (void)hipFreeAsync(a->ptr, s);
    else
        g_retired.emplace_back(dev, a->ptr);
    a->ptr = nullptr;
}

// The override string a plan is keyed by.
std::string tuning_signature(const Tuning& t, bool fwd) {
    const int keys[4] = {fwd ? T_SPLITS_FWD : T_SPLITS_DWEIGHT, fwd ? -1 : T_SPLITS_DINP,
                         T_PLAN_MODEL, -1};
    std::string sig;
    for (int k : keys) {
        if (k < 0) continue;
        sig += t.set[k] ? "=" + t.val[k] : "-";
        sig += "/";
    }
    return sig;
}

// The plan of a shape (made on first use; planning a new shape takes up to
// about 0.1 s of host time and makes no HIP call).
int find_plan(int dev, int dtype, int BT, int C, int OC, bool bias, bool fwd, PlanEntry** out) {
    const PlanKey key(dev, dtype, BT, C, OC, bias, fwd ? 1 : 0, tuning_signature(g_tune, fwd));
    auto it = g_plans.find(key);
    if (it != g_plans.end()) {
        *out = &it->second;
        return MMB_OK;
    }
    TraceRange range("mmb plan");
    DeviceInfo di;
    int st = device_info(dev, &di);
    if (st != MMB_OK) return st;
    di.slots = tiles_resident(dtype);
    const PlanOptions opt = plan_options(g_tune, fwd);
    PlanEntry e;
    e.plan = fwd ? build_plan_forward(dtype, BT, C, OC, bias, di, opt)
                 : build_plan(dtype, BT, C, OC, bias, di, opt);
    static_assert(sizeof(Unit) == 2 * sizeof(int4), "two int4 per unit");
    auto res = g_plans.emplace(key, std::move(e));
    *out = &res.first->second;
    return MMB_OK;
}

// This stream's device copy of a plan's work list: allocated and uploaded
// (from a pinned host copy, asynchronously, in stream order) on the first
// call of the plan on the stream.
int stream_units(int dev, hipStream_t s, PlanEntry& e, Workspace& w, const int4** out) {
    auto it = w.tables.find(&e);
    if (it != w.tables.end()) {
        *out = (const int4*)it->second.ptr;
        return MMB_OK;
    }
    const size_t ub = e.plan.units.size() * sizeof(Unit);
    if (!e.host_units) {
        if (hipHostMalloc((void**)&e.host_units, ub, hipHostMallocDefault) != hipSuccess) {
            e.host_units = nullptr;
            return MMB_ERR_NOMEM;
        }
        std::memcpy(e.host_units, e.plan.units.data(), ub);
    }
    DevAlloc t;
    int st = dev_alloc(dev, &t, ub, s);
    if (st != MMB_OK) return st;
    if (hipMemcpyAsync(t.ptr, e.host_units, ub, hipMemcpyHostToDevice, s) != hipSuccess) {
        dev_retire(dev, &t, s);
        return MMB_ERR_HIP;
    }
    w.tables[&e] = t;
    *out = (const int4*)t.ptr;
    return MMB_OK;
}

// Workspace: two buffers per (device, stream).  `counters` holds one arrival
// counter per output tile and is only ever used for counters: it is zeroed
// when allocated and every counter is reset by the last arriver of its tile,
// so it is all zero at rest whatever plan ran before.  `partials` holds [bias
// partials fp32][tile partials fp32] (each part 256-byte aligned) and needs
// no initial value.  A buffer that is too small is replaced by one twice as
// large (or as large as needed); the old one is freed in stream order.
int grow(int dev, DevAlloc* buf, size_t* cap, size_t need, bool zero, hipStream_t s) {
    if (need <= *cap) return MMB_OK;
    const size_t want = std::max(need, *cap * 2);
    dev_retire(dev, buf, s);
    *cap = 0;
    int st = dev_alloc(dev, buf, want, s);
    if (st != MMB_OK) return st;
    *cap = want;
    if (zero && hipMemsetAsync(buf->ptr, 0, want, s) != hipSuccess) return MMB_ERR_HIP;
    return MMB_OK;
}

int get_workspace(int dev, hipStream_t s, PlanEntry& e, TilesParams* tp) {
    const Plan& p = e.plan;
    const size_t cb = (size_t)p.n_counters * 4;
    const size_t bb = align_up((size_t)p.ws_bias_floats * 4, 256);
    const size_t wb = align_up((size_t)p.ws_floats * 4, 256);
    Workspace& w = g_ws[{dev, s}];
    int st = grow(dev, &w.counters, &w.counter_bytes, cb, true, s);
    if (st != MMB_OK) return st;
    st = grow(dev, &w.partials, &w.partial_bytes, bb + wb, false, s);
    if (st != MMB_OK) return st;
    st = stream_units(dev, s, e, w, &tp->units);
    if (st != MMB_OK) return st;
    char* b = (char*)w.partials.ptr;
    tp->counters = (int*)w.counters.ptr;
    tp->ws_bias = (float*)b;
    tp->ws = (float*)(b + bb);
    return MMB_OK;
}

// sr: bf16 only; dweight and dbias rounded stochastically under `seed`.
int backward_impl(void* dinp, void* dweight, void* dbias, const void* dout, const void* inp,
                  const void* weight, int B, int T, int C, int OC, int dtype, hipStream_t s,
                  bool sr = false, unsigned long long seed = 0) {
    int st = check(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype);
    if (st != MMB_OK) return st;
    const int BT = B * T;
    const int path = choose_path(dinp, dweight, dout, inp, weight, C, OC, dtype);
    if (path == 0) {
        TraceRange range("mmb launch (generic)");
        return launch_generic(dtype, dinp, dweight, dbias, dout, inp, weight, BT, C, OC, s, sr,
                              seed) == hipSuccess
                   ? MMB_OK
                   : MMB_ERR_HIP;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MMB_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    PlanEntry* plan = nullptr;
    st = find_plan(dev, dtype, BT, C, OC, dbias != nullptr, false, &plan);
    if (st != MMB_OK) return st;
    TraceRange range(path == 2 ? "mmb launch (packed)" : "mmb launch");
    TilesParams tp = plan->plan.proto;
    st = get_workspace(dev, s, *plan, &tp);
    if (st != MMB_OK) return st;
    tp.dinp = dinp;
    tp.dweight = dweight;
    tp.dbias = dbias;
    tp.dout = dout;
    tp.inp = inp;
    tp.weight = weight;
    tp.seed = seed;
    Packing pk;
    char* pbase = nullptr;
    if (path == 2) {
        pk = plan_packing_bwd(dtype, BT, C, OC, dinp, dweight, dout, inp, weight);
        Workspace& w = g_ws[{dev, s}];
        st = grow(dev, &w.packed, &w.packed_bytes, pk.bytes, false, s);
        if (st != MMB_OK) return st;
        pbase = (char*)w.packed.ptr;
        if (pack_operands(pk, pbase, &tp, dtype, s) != hipSuccess) return MMB_ERR_HIP;
    }
    const hipError_t e = sr ? launch_tiles_bf16_sr(tp, s) : launch_tiles(dtype, tp, s);
    if (e != hipSuccess) return MMB_ERR_HIP;
    if (path == 2 &&
        unpack_outputs(pk, pbase, dinp, dweight, nullptr, BT, C, OC, dtype, s) != hipSuccess)
        return MMB_ERR_HIP;
    return MMB_OK;
}

// ---------------------------------------------------------------------------
// the allocation-free backward: the same plans and kernels as backward_impl,
// with the workspace carved out of the static `scratch` array and the work
// list passed through kernel arguments, so that a call makes no allocation
// and no host-to-device copy.

// One launch of mmb_put_units carries up to kChunkUnits units (3.5 KB of
// arguments) to their place in the scratch work list; the first launch of a
// call also clears the call's tile counters.
constexpr int kChunkUnits = 112;
struct UnitChunk {
    int4 u[2 * kChunkUnits];
    int4* dst;      // destination of u[0]
    int n;          // int4s to copy
    int* zero;      // counters to clear (n_zero ints), or NULL
    int n_zero;
};

__global__ __launch_bounds__(256) void mmb_put_units(UnitChunk c) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x, nt = gridDim.x * blockDim.x;
    for (int i = t; i < c.n; i += nt) c.dst[i] = c.u[i];
    for (int i = t; i < c.n_zero; i += nt) c.zero[i] = 0;
}

std::map<int, char*> g_scratch;   // device -> address of its `scratch`

// The device address of `scratch` on the current device `dev` (looked up
// once per device).
int noalloc_scratch(int dev, char** out) {
    auto it = g_scratch.find(dev);
    if (it != g_scratch.end()) {
        *out = it->second;
        return MMB_OK;
    }
    char* ptr = nullptr;
    if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
        return MMB_ERR_HIP;
    g_scratch[dev] = ptr;
    *out = ptr;
    return MMB_OK;
}

int backward_noalloc_impl(void* dinp, void* dweight, void* dbias, const void* dout,
                          const void* inp, const void* weight, int B, int T, int C, int OC,
                          int dtype, hipStream_t s) {
    int st = check(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype);
    if (st != MMB_OK) return st;
    const int BT = B * T;
    const int path = choose_path(dinp, dweight, dout, inp, weight, C, OC, dtype);
    if (path == 0) {
        // the generic kernels use no workspace
        TraceRange range("mmb launch (generic)");
        return launch_generic(dtype, dinp, dweight, dbias, dout, inp, weight, BT, C, OC, s) ==
                       hipSuccess
                   ? MMB_OK
                   : MMB_ERR_HIP;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MMB_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    PlanEntry* entry = nullptr;
    st = find_plan(dev, dtype, BT, C, OC, dbias != nullptr, false, &entry);
    if (st != MMB_OK) return st;
    const Plan& plan = entry->plan;
    // scratch layout: counters, work list, dbias partials, tile partials,
    // packed copies of ragged operands (each part 256-byte aligned), all
    // sizes in 64 bits
    const size_t cb = align_up((size_t)plan.n_counters * 4, 256);
    const size_t ub = align_up(plan.units.size() * sizeof(Unit), 256);
    const size_t bb = align_up((size_t)plan.ws_bias_floats * 4, 256);
    const size_t wb = align_up((size_t)plan.ws_floats * 4, 256);
    Packing pk;
    if (path == 2) pk = plan_packing_bwd(dtype, BT, C, OC, dinp, dweight, dout, inp, weight);
    if (cb + ub + bb + wb + pk.bytes > (size_t)MMB_NOALLOC_SCRATCH_BYTES) return MMB_ERR_SCRATCH;
    char* base = nullptr;
    st = noalloc_scratch(dev, &base);
    if (st != MMB_OK) return st;
    TraceRange range("mmb launch (no allocation)");
    int* counters = (int*)base;
    int4* units = (int4*)(base + cb);
    const int n4 = (int)(2 * plan.units.size());
    const int4* src = (const int4*)plan.units.data();
    UnitChunk c;
    for (int first = 0; first < n4 || first == 0; first += 2 * kChunkUnits) {
        c.n = std::min(2 * kChunkUnits, n4 - first);
        std::memcpy(c.u, src + first, (size_t)c.n * sizeof(int4));
        c.dst = units + first;
        c.zero = first == 0 ? counters : nullptr;
        c.n_zero = first == 0 ? plan.n_counters : 0;
        const int work = std::max(c.n, c.n_zero);
        const int blocks = std::max(1, std::min(1024, (work + 255) / 256));
        hipLaunchKernelGGL(mmb_put_units, dim3(blocks), dim3(256), 0, s, c);
        if (hipGetLastError() != hipSuccess) return MMB_ERR_HIP;
    }
    TilesParams tp = plan.proto;
    tp.units = units;
    tp.counters = counters;
    tp.ws_bias = (float*)(base + cb + ub);
    tp.ws = (float*)(base + cb + ub + bb);
    tp.dinp = dinp;
    tp.dweight = dweight;
    tp.dbias = dbias;
    tp.dout = dout;
    tp.inp = inp;
    tp.weight = weight;
    tp.seed = 0;
    char* pbase = base + cb + ub + bb + wb;
    if (path == 2 && pack_operands(pk, pbase, &tp, dtype, s) != hipSuccess) return MMB_ERR_HIP;
    if (launch_tiles(dtype, tp, s) != hipSuccess) return MMB_ERR_HIP;
    if (path == 2 &&
        unpack_outputs(pk, pbase, dinp, dweight, nullptr, BT, C, OC, dtype, s) != hipSuccess)
        return MMB_ERR_HIP;
    return MMB_OK;
}

// LayerNorm backward: every pointer required; the three outputs may not
// overlap each other or any input.
int check_ln(const void* dinp, const void* dweight, const void* dbias, const void* dout,
             const void* inp, const void* weight, const void* mean, const void* rstd, int B, int T,
             int C, int dtype) {
    if (!dinp || !dweight || !dbias || !dout || !inp || !weight || !mean || !rstd)
        return MMB_ERR_NULL;
    if (B < 1 || T < 1 || C < 1) return MMB_ERR_DIM;
    if (dtype != MMB_FP32 && dtype != MMB_BF16) return MMB_ERR_DTYPE;
    const long long BT = (long long)B * T;
    if (BT > 0x7fffffffLL) return MMB_ERR_OVERFLOW;
    const uintptr_t es = elem_size(dtype);
    auto R = [&](const void* p, long long n) {
        return Span{(uintptr_t)p, (uintptr_t)p + (uintptr_t)n * es};
    };
    const Span outs[3] = {R(dinp, BT * C), R(dweight, C), R(dbias, C)};
    const Span ins[5] = {R(dout, BT * C), R(inp, BT * C), R(weight, C), R(mean, BT), R(rstd, BT)};
    for (int a = 0; a < 3; ++a) {
        for (int b = a + 1; b < 3; ++b)
            if (overlap(outs[a], outs[b])) return MMB_ERR_ALIAS;
        for (const Span& r : ins)
            if (overlap(outs[a], r)) return MMB_ERR_ALIAS;
    }
    return MMB_OK;
}

// Vectors per lane of the LayerNorm row kernel, or 0 for the generic kernels
// (also when a row-streamed buffer is not 16-byte aligned).
LNLayout ln_path(const void* dinp, const void* dout, const void* inp, const void* weight, int C,
                 int dtype) {
    const void* ptrs[4] = {dinp, dout, inp, weight};
    for (const void* p : ptrs)
        if ((uintptr_t)p % 16 != 0) return LNLayout{0, 1};
    return ln_layout(dtype, C);
}

int layernorm_impl(void* dinp, void* dweight, void* dbias, const void* dout, const void* inp,
                   const void* weight, const void* mean, const void* rstd, int B, int T, int C,
                   int dtype, hipStream_t s) {
    int st = check_ln(dinp, dweight, dbias, dout, inp, weight, mean, rstd, B, T, C, dtype);
    if (st != MMB_OK) return st;
    LNParams p;
    p.dinp = dinp;
    p.dweight = dweight;
    p.dbias = dbias;
    p.dout = dout;
    p.inp = inp;
    p.weight = weight;
    p.mean = mean;
    p.rstd = rstd;
    p.BT = (long long)B * T;
    p.C = C;
    p.partial = nullptr;
    const LNLayout lay = ln_path(dinp, dout, inp, weight, C, dtype);
    // held through the launch: another call may not regrow the partials first
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MMB_ERR_HIP;
    DeviceInfo di;
    st = device_info(dev, &di);
    if (st != MMB_OK) return st;
    // G partial rows of [dweight | dbias]: the row kernel runs one workgroup
    // of 8 row-waves per CU (fewer for few rows), the generic kernels one
    // band of rows per CU; MMB_LN_WORKGROUPS overrides the count (tuning aid)
    long long want = di.cus;
    if (const char* e = g_tune.get(T_LN_WORKGROUPS)) {
        const long v = std::strtol(e, nullptr, 10);
        if (v > 0) want = std::min(v, 1L << 16);
    }
    // rows per workgroup step (row kernel) or per band (generic); the
    // generic kernels' bands are a grid dimension, at most 65535
    const long long rows_per_step = lay.nj > 0 ? 8 / lay.wpr : 1;
    if (lay.nj == 0) want = std::min(want, 65535LL);
    const int G =
        (int)std::max(1LL, std::min<long long>(want, (p.BT + rows_per_step - 1) / rows_per_step));
    Workspace& w = g_ws[{dev, s}];
    st = grow(dev, &w.partials, &w.partial_bytes, (size_t)G * 2 * C * sizeof(float), false, s);
    if (st != MMB_OK) return st;
    p.partial = (float*)w.partials.ptr;
    TraceRange range("mmb layernorm launch");
    return launch_layernorm_backward(dtype, p, G, lay, s) == hipSuccess ? MMB_OK : MMB_ERR_HIP;
}

int forward_impl(void* out, const void* inp, const void* weight, const void* bias, int B, int T,
                 int C, int OC, int dtype, hipStream_t s) {
    int st = check_fwd(out, inp, weight, bias, B, T, C, OC, dtype);
    if (st != MMB_OK) return st;
    const int BT = B * T;
    const int path = choose_path_fwd(out, inp, weight, bias, C, OC, dtype);
    if (path == 0) {
        TraceRange range("mmb forward launch (generic)");
        return launch_fwd_generic(dtype, out, inp, weight, bias, BT, C, OC, s) == hipSuccess
                   ? MMB_OK
                   : MMB_ERR_HIP;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MMB_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    PlanEntry* plan = nullptr;
    st = find_plan(dev, dtype, BT, C, OC, bias != nullptr, true, &plan);
    if (st != MMB_OK) return st;
    TraceRange range(path == 2 ? "mmb forward launch (packed)" : "mmb forward launch");
    TilesParams tp = plan->plan.proto;
    st = get_workspace(dev, s, *plan, &tp);
    if (st != MMB_OK) return st;
    tp.out = out;
    tp.bias = bias;
    tp.inp = inp;
    tp.weight = weight;
    Packing pk;
    char* pbase = nullptr;
    if (path == 2) {
        pk = plan_packing_fwd(dtype, BT, C, OC, out, inp, weight, bias);
        Workspace& w = g_ws[{dev, s}];
        st = grow(dev, &w.packed, &w.packed_bytes, pk.bytes, false, s);
        if (st != MMB_OK) return st;
        pbase = (char*)w.packed.ptr;
        if (pack_operands(pk, pbase, &tp, dtype, s) != hipSuccess) return MMB_ERR_HIP;
    }
    if (launch_fwd_tiles(dtype, tp, s) != hipSuccess) return MMB_ERR_HIP;
    if (path == 2 &&
        unpack_outputs(pk, pbase, nullptr, nullptr, out, BT, C, OC, dtype, s) != hipSuccess)
        return MMB_ERR_HIP;
    return MMB_OK;
}

}  // namespace
}  // namespace mmb

extern "C" {

int mmb_layernorm_backward(void* dinp, void* dweight, void* dbias, const void* dout,
                           const void* inp, const void* weight, const void* mean,
                           const void* rstd, int B, int T, int C, int dtype, void* stream) {
    return mmb::layernorm_impl(dinp, dweight, dbias, dout, inp, weight, mean, rstd, B, T, C, dtype,
                               (hipStream_t)stream);
}

int mmb_layernorm_check_args(const void* dinp, const void* dweight, const void* dbias,
                             const void* dout, const void* inp, const void* weight,
                             const void* mean, const void* rstd, int B, int T, int C, int dtype) {
    return mmb::check_ln(dinp, dweight, dbias, dout, inp, weight, mean, rstd, B, T, C, dtype);
}

int mmb_layernorm_path(const void* dinp, const void* dweight, const void* dbias, const void* dout,
                       const void* inp, const void* weight, const void* mean, const void* rstd,
                       int B, int T, int C, int dtype) {
    const int st = mmb::check_ln(dinp, dweight, dbias, dout, inp, weight, mean, rstd, B, T, C,
                                 dtype);
    if (st != MMB_OK) return st;
    return mmb::ln_path(dinp, dout, inp, weight, C, dtype).nj > 0 ? 1 : 0;
}

int mmb_forward_check_args(const void* out, const void* inp, const void* weight, const void* bias,
                           int B, int T, int C, int OC, int dtype) {
    return mmb::check_fwd(out, inp, weight, bias, B, T, C, OC, dtype);
}

int mmb_forward_path(const void* out, const void* inp, const void* weight, const void* bias, int B,
                     int T, int C, int OC, int dtype) {
    const int st = mmb::check_fwd(out, inp, weight, bias, B, T, C, OC, dtype);
    if (st != MMB_OK) return st;
    return mmb::choose_path_fwd(out, inp, weight, bias, C, OC, dtype) > 0 ? 1 : 0;
}

int mmb_forward_stream(void* out, const void* inp, const void* weight, const void* bias, int B,
                       int T, int C, int OC, int dtype, void* stream) {
    return mmb::forward_impl(out, inp, weight, bias, B, T, C, OC, dtype, (hipStream_t)stream);
}

int mmb_forward(void* out, const void* inp, const void* weight, const void* bias, int B, int T,
                int C, int OC, int dtype) {
    return mmb::forward_impl(out, inp, weight, bias, B, T, C, OC, dtype, nullptr);
}

int mmb_check_args(const void* dinp, const void* dweight, const void* dbias, const void* dout,
                   const void* inp, const void* weight, int B, int T, int C, int OC, int dtype) {
    return mmb::check(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype);
}

int mmb_path(const void* dinp, const void* dweight, const void* dbias, const void* dout,
             const void* inp, const void* weight, int B, int T, int C, int OC, int dtype) {
    const int st = mmb::check(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype);
    if (st != MMB_OK) return st;
    return mmb::choose_path(dinp, dweight, dout, inp, weight, C, OC, dtype) > 0 ? 1 : 0;
}

int mmb_backward_stream(void* dinp, void* dweight, void* dbias, const void* dout,
                        const void* inp, const void* weight, int B, int T, int C, int OC,
                        int dtype, void* stream) {
    return mmb::backward_impl(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype,
                              (hipStream_t)stream);
}

int mmb_backward_sr(void* dinp, void* dweight, void* dbias, const void* dout, const void* inp,
                    const void* weight, int B, int T, int C, int OC, unsigned long long seed,
                    void* stream) {
    return mmb::backward_impl(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, MMB_BF16,
                              (hipStream_t)stream, true, seed);
}

int mmb_backward_noalloc(void* dinp, void* dweight, void* dbias, const void* dout,
                         const void* inp, const void* weight, int B, int T, int C, int OC,
                         int dtype, void* stream) {
    return mmb::backward_noalloc_impl(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype,
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
        case MMB_ERR_NAME: return "not a tuning variable of the library";
        case MMB_ERR_SCRATCH:
            return "the call needs more device memory than mmb_backward_noalloc's fixed scratch "
                   "(MMB_NOALLOC_SCRATCH_BYTES) holds";
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
    mmb::set_topology(&di);
    di.slots = mmb::tiles_resident(dtype);
    mmb::PlanOptions opt;
    {
        std::lock_guard<std::mutex> lock(mmb::g_mu);
        opt = mmb::plan_options(mmb::g_tune, false);
    }
    const mmb::Plan p = mmb::build_plan(dtype, B * T, C, OC, has_bias != 0, di, opt);
    splits[0] = p.max_splits[mmb::UNIT_DWEIGHT];
    splits[1] = p.max_splits[mmb::UNIT_DINP];
    if (units) {
        const int n = std::min<int>(max_units, (int)p.units.size());
        for (int i = 0; i < n; ++i) {
            const int4 a = p.units[i].a, b = p.units[i].b;
            const int v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            for (int j = 0; j < 8; ++j) units[8 * i + j] = v[j];
        }
    }
    return (int)p.units.size();
}

int mmb_forward_plan_units(int B, int T, int C, int OC, int dtype, int has_bias, int num_cus,
                           int* splits, int* units, int max_units) {
    if (B < 1 || T < 1 || C < 1 || OC < 1 || num_cus < 1) return MMB_ERR_DIM;
    if (dtype != MMB_FP32 && dtype != MMB_BF16) return MMB_ERR_DTYPE;
    if ((long long)B * T > 0x7fffffffLL) return MMB_ERR_OVERFLOW;
    if (!splits) return MMB_ERR_NULL;
    mmb::DeviceInfo di;
    di.cus = num_cus;
    mmb::set_topology(&di);
    di.slots = mmb::tiles_resident(dtype);
    mmb::PlanOptions opt;
    {
        std::lock_guard<std::mutex> lock(mmb::g_mu);
        opt = mmb::plan_options(mmb::g_tune, true);
    }
    const mmb::Plan p = mmb::build_plan_forward(dtype, B * T, C, OC, has_bias != 0, di, opt);
    splits[0] = p.max_splits[mmb::UNIT_FWD];
    if (units) {
        const int n = std::min<int>(max_units, (int)p.units.size());
        for (int i = 0; i < n; ++i) {
            const int4 a = p.units[i].a, b = p.units[i].b;
            const int v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            for (int j = 0; j < 8; ++j) units[8 * i + j] = v[j];
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
    std::map<int, bool> synced;
    auto sync = [&](int dev) {
        if (synced[dev]) return;
        synced[dev] = true;
        (void)hipSetDevice(dev);
        if (hipDeviceSynchronize() != hipSuccess) st = MMB_ERR_HIP;
    };
    for (auto& kv : mmb::g_ws) sync(kv.first.first);
    for (auto& kv : mmb::g_retired) sync(kv.first);
    for (auto& kv : mmb::g_plans) sync(std::get<0>(kv.first));
    // everything enqueued has finished: free in any order
    auto release = [](mmb::DevAlloc& a) {
        if (a.ptr) (void)hipFree(a.ptr);
        a.ptr = nullptr;
    };
    for (auto& kv : mmb::g_ws) {
        (void)hipSetDevice(kv.first.first);
        release(kv.second.counters);
        release(kv.second.partials);
        release(kv.second.packed);
        for (auto& t : kv.second.tables) release(t.second);
    }
    mmb::g_ws.clear();
    for (auto& kv : mmb::g_retired) {
        (void)hipSetDevice(kv.first);
        (void)hipFree(kv.second);
    }
    mmb::g_retired.clear();
    for (auto& kv : mmb::g_plans)
        if (kv.second.host_units) (void)hipHostFree(kv.second.host_units);
    mmb::g_plans.clear();
    (void)hipSetDevice(prev);
    return st;
}

int mmb_set_tuning(const char* name, const char* value) {
    if (!name) return MMB_ERR_NULL;
    std::lock_guard<std::mutex> lock(mmb::g_mu);
    for (int k = 0; k < mmb::T_COUNT; ++k)
        if (std::strcmp(name, mmb::kTuneNames[k]) == 0) {
            mmb::g_tune.set[k] = value != nullptr;
            mmb::g_tune.val[k] = value ? value : "";
            return MMB_OK;
        }
    return MMB_ERR_NAME;
}

}  // extern "C"
