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

// 1 when the MFMA tiles can take a forward call: as for the backward pass,
// and the bias (read as 16-byte groups in the epilogue) is aligned too.
int choose_path_fwd(const void* out, const void* inp, const void* weight, const void* bias, int C,
                    int OC, int dtype) {
    const int vec = dtype == MMB_BF16 ? 8 : 4;
    if (C % vec != 0 || OC % vec != 0) return 0;
    if (C > (1 << 22) || OC > (1 << 22)) return 0;
    const void* ptrs[4] = {out, inp, weight, bias};
    for (const void* p : ptrs)
        if ((uintptr_t)p % 16 != 0) return 0;   // NULL bias passes
    return 1;
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

// A profiler range (roctx) around planning and launching, so that a trace
// shows host cost next to kernel time; free when no profiler is attached.
struct TraceRange {
    explicit TraceRange(const char* what) { roctxRangePushA(what); }
    ~TraceRange() { roctxRangePop(); }
    TraceRange(const TraceRange&) = delete;
    TraceRange& operator=(const TraceRange&) = delete;
};

// ---------------------------------------------------------------------------
// planner

int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

struct DeviceInfo {
    int cus = 0;
    int xcds = 1;
    int ses = 1;     // shader engines per XCD
    int slots = 1;   // resident workgroups of the tile kernel per CU
};

// MI355X hands workgroup i to XCD i mod 8; inside an XCD, consecutive
// workgroups go to its 4 shader engines (8 CUs each) in turn and start in
// order: one that finds its engine full holds back the ones behind it
// (per-workgroup timestamps and hardware ids on MI355X).
void set_topology(DeviceInfo* d) {
    d->xcds = d->cus >= 128 ? 8 : 1;
    const int per_xcd = d->cus / d->xcds;
    d->ses = per_xcd >= 16 && per_xcd % 4 == 0 ? 4 : 1;
}

struct Unit {
    int4 a;   // {kind, tile_m, tile_n, split}
    int4 b;   // {kt0, kt1, splits of the tile, first workspace slot of the tile}
};

struct Plan {
    TilesParams proto;            // pointers filled per call
    std::vector<Unit> units;      // launch order
    int4* d_units = nullptr;      // device copy (owned by the plan cache)
    int max_splits[2] = {1, 1};   // largest split count of each GEMM's tiles
    long long ws_floats = 0;
    long long ws_bias_floats = 0;
    int n_counters = 0;
    std::string forced;           // the split overrides the plan was made with
};

// Costs of the pieces of a unit for the tile kernels as built, measured on
// MI355X with per-workgroup timestamps.  The K loop runs at a speed set by
// the core clock, which falls as more slots run K loops (the chip is power
// limited: about 2.0 GHz with a few CUs idle, 1.7 GHz with all busy);
// t_iter is the time of one K iteration at full speed, and the loops run at
// `slow` times that speed once a fraction busy_hi of the slots loop (linear
// from busy_lo).  The rest is in microseconds: the first-stage loads, the
// beta = 1 epilogue, publishing a partial tile and taking the ticket, and for
// the last arriver of a split tile the fix-up (fix0 + fix_per_partial per
// partial read) and the write of the tile.
struct CostModel {
    double t_iter[2];              // [UNIT_DWEIGHT], [UNIT_DINP]
    double slow, busy_lo, busy_hi;
    double prologue, epilogue, publish;
    double fix0, fix_per_partial, write;
    double partial_bytes_per_us;   // workspace traffic the whole GPU absorbs
};

// MMB_PLAN_MODEL="t_dweight,t_dinp,slow,busy_lo,busy_hi,prologue,epilogue,
// publish,fix0,fix_per_partial,write,bytes_per_us" replaces the constants
// (tuning aid for other devices or kernels).
CostModel cost_model(int dtype, const char* v) {
    CostModel cm = dtype == MMB_BF16
                       ? CostModel{{1.402, 1.263}, 0.7245, 0.9688, 0.9688, 0.78, 3.82, 8.47, 2.07, 2.51, 4.40, 10.16e6}
                       : CostModel{{3.356, 2.463}, 0.470, 0.130, 0.416, 1.22, 3.31, 3.93, 1.79, 1.68, 0.06, 20.73e6};
    if (v) {
        double x[12];
        if (std::sscanf(v, "%lf,%lf,%lf,%lf,%lf,%lf,%lf,%lf,%lf,%lf,%lf,%lf", &x[0], &x[1], &x[2],
                        &x[3], &x[4], &x[5], &x[6], &x[7], &x[8], &x[9], &x[10], &x[11]) == 12)
            cm = CostModel{{x[0], x[1]}, x[2], x[3], x[4], x[5], x[6], x[7], x[8], x[9], x[10], x[11]};
    }
    return cm;
}

// Per-tile split counts of the two GEMMs (row-major tile index).
struct Layout {
    std::vector<int> splits[2];
};

// Launch order.  Inside one GEMM, tiles with fewer splits (longer units)
// come first; among equal ones, dweight units are ordered (split, tile_m,
// tile_n) so that units running together share the inp rows of one K range
// and the dout columns of one tile_m, and dinp units (tile_m, split, tile_n)
// so that they share dout rows.  Every run of equal split counts, of the GEMM
// with the longer units first, is dealt out evenly in contiguous pieces, one
// per XCD (the remainders rotate over the XCDs), and the XCD sequences are
// interleaved so that workgroup i lands on XCD i % xcds.
std::vector<Unit> make_units(const GemmPlan g[2], const Layout& L, const DeviceInfo& dev) {
    std::vector<Unit> per[2];
    int slot = 0;
    std::vector<int> slot_of[2];
    for (int k = 0; k < 2; ++k) {
        slot_of[k].assign(L.splits[k].size(), 0);
        for (size_t t = 0; t < L.splits[k].size(); ++t) {
            slot_of[k][t] = slot;
            if (L.splits[k][t] > 1) slot += L.splits[k][t];
        }
    }
    for (int k = 0; k < 2; ++k) {
        const GemmPlan& G = g[k];
        std::vector<int> levels(L.splits[k].begin(), L.splits[k].end());
        std::sort(levels.begin(), levels.end());
        levels.erase(std::unique(levels.begin(), levels.end()), levels.end());
        for (int S : levels) {
            auto emit = [&](int m, int n, int s) {
                const int t = m * G.tiles_n + n;
                if (L.splits[k][t] != S) return;
                const int kt0 = (int)((long long)s * G.kiters / S);
                const int kt1 = (int)((long long)(s + 1) * G.kiters / S);
                per[k].push_back(Unit{make_int4(k, m, n, s), make_int4(kt0, kt1, S, slot_of[k][t])});
            };
            if (k == UNIT_DINP) {
                for (int m = 0; m < G.tiles_m; ++m)
                    for (int s = 0; s < S; ++s)
                        for (int n = 0; n < G.tiles_n; ++n) emit(m, n, s);
            } else {
                for (int s = 0; s < S; ++s)
                    for (int m = 0; m < G.tiles_m; ++m)
                        for (int n = 0; n < G.tiles_n; ++n) emit(m, n, s);
            }
        }
    }
    auto longest = [&](int k) {
        int x = 0;
        for (const Unit& u : per[k]) x = std::max(x, u.b.y - u.b.x);
        return x;
    };
    const int first = longest(UNIT_DWEIGHT) >= longest(UNIT_DINP) ? UNIT_DWEIGHT : UNIT_DINP;
    const std::vector<Unit>& a = per[first];
    const std::vector<Unit>& b = per[1 - first];
    const int X = std::max(1, dev.xcds);
    const size_t n = a.size() + b.size();
    std::vector<std::vector<Unit>> seq(X);
    int rot = 0;   // XCD that receives the next remainder unit
    auto deal = [&](const std::vector<Unit>& list) {
        for (size_t i = 0; i < list.size();) {
            size_t j = i;
            while (j < list.size() && list[j].b.z == list[i].b.z) ++j;
            const size_t len = j - i, base = len / X, rem = len % X;
            size_t p = i;
            for (int x = 0; x < X; ++x) {
                const size_t c = base + ((size_t)((x - rot + X) % X) < rem ? 1 : 0);
                seq[x].insert(seq[x].end(), list.begin() + p, list.begin() + p + c);
                p += c;
            }
            rot = (int)((rot + rem) % X);
            i = j;
        }
    };
    deal(a);
    deal(b);
    std::vector<Unit> out;
    out.reserve(n);
    for (int x = 0; x < X; ++x)
        if (seq[x].size() != n / X + ((size_t)x < n % X ? 1 : 0)) {   // cannot happen
            out = a;
            out.insert(out.end(), b.begin(), b.end());
            return out;
        }
    for (size_t i = 0; i < n; ++i) out.push_back(seq[i % X][i / X]);
    return out;
}

// Speed of the K loops, relative to full speed, while `c` of `total` slots loop.
double loop_speed(const CostModel& cm, double c, double total) {
    const double lo = cm.busy_lo * total, hi = cm.busy_hi * total;
    if (c <= lo) return 1.0;
    if (c >= hi) return cm.slow;
    return 1.0 + (cm.slow - 1.0) * (c - lo) / (hi - lo);
}

// Event model of one launch with `slots` resident workgroups per CU: the
// k-th workgroup of an XCD starts when a slot frees on engine k mod ses of
// that XCD, after the workgroup before it.  A unit runs its prologue, its K
// loop (at the speed the number of looping slots allows), then its epilogue
// or, in a split tile, the publish; the last unit of a split tile to publish
// then runs the fix-up and the write.  Returns the makespan (us).
double simulate(const std::vector<Unit>& units, const CostModel& cm, const DeviceInfo& dev) {
    const int X = std::max(1, dev.xcds), E = std::max(1, dev.ses);
    const int per = std::max(1, dev.cus / X / E) * std::max(1, dev.slots);
    const double total = (double)per * E * X;
    const size_t n = units.size();
    std::vector<size_t> next(X);
    std::vector<long long> started(X, 0);
    for (int x = 0; x < X; ++x) next[x] = x;
    std::vector<int> free_slots((size_t)X * E, per), engine(n, 0);
    // split tiles numbered densely; left[t] = units of tile t yet to publish
    std::vector<int> tile_of(n, -1), left;
    {
        std::unordered_map<long long, int> ids;   // tile_m and tile_n are below 2^20 here
        for (size_t i = 0; i < n; ++i) {
            const Unit& u = units[i];
            if (u.b.z <= 1) continue;
            const long long key = ((long long)u.a.x << 40) | ((long long)u.a.y << 20) | u.a.z;
            auto it = ids.emplace(key, (int)left.size());
            if (it.second) left.push_back(0);
            tile_of[i] = it.first->second;
            ++left[tile_of[i]];
        }
    }
    // events (finish, 4 * unit + phase): phases 0 prologue, 2 epilogue or
    // publish, 3 fix-up and write run in real time; phase 1, the K loop, in
    // loop time V, which advances at the current speed
    typedef std::pair<double, long long> Ev;
    std::priority_queue<Ev, std::vector<Ev>, std::greater<Ev>> timed, loops;
    double T = 0, V = 0, span = 0;
    auto dispatch = [&]() {
        for (int x = 0; x < X; ++x)
            while (next[x] < n) {
                const int slot = x * E + (int)(started[x] % E);
                if (free_slots[slot] == 0) break;
                --free_slots[slot];
                engine[next[x]] = slot;
                timed.push(Ev(T + cm.prologue, 4LL * (long long)next[x]));
                next[x] += X;
                ++started[x];
            }
    };
    auto speed = [&](size_t looping) { return loop_speed(cm, (double)looping, total); };
    const double inf = 1e300;
    std::vector<long long> fin;
    dispatch();
    while (!timed.empty() || !loops.empty()) {
        const double sp = speed(loops.size());
        const double tt = timed.empty() ? inf : timed.top().first;
        const double tl = loops.empty() ? inf : T + (loops.top().first - V) / sp;
        const double tn = std::min(tt, tl);
        V += (tn - T) * sp;
        T = tn;
        fin.clear();
        while (!timed.empty() && timed.top().first <= T + 1e-9) {
            fin.push_back(timed.top().second);
            timed.pop();
        }
        while (!loops.empty() && loops.top().first <= V + 1e-9) {
            fin.push_back(loops.top().second);
            loops.pop();
        }
        bool freed = false;
        for (long long ev : fin) {
            const size_t i = (size_t)(ev / 4);
            const int ph = (int)(ev % 4);
            const Unit& u = units[i];
            if (ph == 0) {
                loops.push(Ev(V + (u.b.y - u.b.x) * cm.t_iter[u.a.x], 4LL * (long long)i + 1));
            } else if (ph == 1) {
                timed.push(Ev(T + (u.b.z > 1 ? cm.publish : cm.epilogue), 4LL * (long long)i + 2));
            } else if (ph == 2 && tile_of[i] >= 0 && --left[tile_of[i]] == 0) {
                timed.push(Ev(T + cm.fix0 + cm.fix_per_partial * u.b.z + cm.write,
                              4LL * (long long)i + 3));
            } else {
                ++free_slots[engine[i]];
                freed = true;
                span = T;
            }
        }
        if (freed) dispatch();
    }
    return span;
}

// Makespan of a layout plus the time the whole GPU needs for its workspace
// traffic (each partial tile written once and read once), or a lower bound
// of it that is already >= `bound`.
double plan_cost(const GemmPlan g[2], const Layout& L, const DeviceInfo& dev, const CostModel& cm,
                 double tile_bytes, double bound) {
    std::vector<Unit> u = make_units(g, L, dev);
    double partials = 0;
    for (int k = 0; k < 2; ++k)
        for (int s : L.splits[k])
            if (s > 1) partials += s;
    const double traffic = 2.0 * partials * tile_bytes / cm.partial_bytes_per_us;
    // lower bounds: the work spread evenly over all slots at full speed, and
    // the K-loop work at the largest aggregate rate (looping slots x their
    // speed) the model allows; a layout whose bound reaches `bound` is not
    // simulated
    const int total = dev.cus * std::max(1, dev.slots);
    double work = 0, loop = 0, rate = 0;
    for (const Unit& x : u) {
        const double l = (x.b.y - x.b.x) * cm.t_iter[x.a.x];
        loop += l;
        work += cm.prologue + l + (x.b.z > 1 ? cm.publish : cm.epilogue);
    }
    for (int c = 1; c <= total; ++c) rate = std::max(rate, c * loop_speed(cm, c, total));
    const double lower = std::max(work / total, loop / rate) + traffic;
    if (lower >= bound) return lower;
    return simulate(u, cm, dev) + traffic;
}

// Split overrides: empty = the planner chooses; one value = that count for
// every tile of the GEMM; several values = tile t gets value t mod count
// (clamped to the tile's K iterations; for tests of uneven plans).
std::vector<int> parse_splits(const char* v) {
    std::vector<int> out;
    if (!v) return out;
    const char* p = v;
    while (*p) {
        char* end = nullptr;
        const long x = std::strtol(p, &end, 10);
        if (end == p) break;   // not a number: stop
        if (x > 0) out.push_back((int)std::min(x, 1L << 20));
        if (*end != ',') break;
        p = end + 1;
    }
    return out;
}

// What the planner takes from the tuning overrides.
struct PlanOptions {
    std::vector<int> force_w, force_i;   // split overrides (dweight / dinp, or the forward)
    const char* model = nullptr;         // MMB_PLAN_MODEL constants, or NULL
    bool trace = false;                  // print every modelled candidate to stderr
};

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

Plan build_plan(int dtype, int BT, int C, int OC, bool bias, const DeviceInfo& dev,
                const PlanOptions& opt) {
    const std::vector<int>& force_w = opt.force_w;
    const std::vector<int>& force_i = opt.force_i;
    const TileShape ts = tile_shape(dtype);
    GemmPlan g[2];
    // dweight[OC,C] += dout^T[OC,BT] . inp[BT,C]
    g[UNIT_DWEIGHT] = GemmPlan{OC, C, BT, cdiv(OC, ts.BM), cdiv(C, ts.BN), cdiv(BT, ts.BK), 0};
    // dinp[BT,C] += dout[BT,OC] . weight[OC,C]
    g[UNIT_DINP] = GemmPlan{BT, C, OC, cdiv(BT, ts.BM), cdiv(C, ts.BN), cdiv(OC, ts.BK), 0};
    g[UNIT_DINP].tile_base = g[UNIT_DWEIGHT].tiles_m * g[UNIT_DWEIGHT].tiles_n;
    const int ntiles[2] = {g[0].tiles_m * g[0].tiles_n, g[1].tiles_m * g[1].tiles_n};
    const CostModel cm = cost_model(dtype, opt.model);
    const double tile_bytes = 4.0 * ts.BM * ts.BN;
    const int max_s[2] = {std::min(16, g[UNIT_DWEIGHT].kiters), std::min(8, g[UNIT_DINP].kiters)};
    const bool trace = opt.trace;
    // one split count per GEMM (the unit encoding allows a count per tile)
    Layout best_L;
    double best = 1e300;
    const int force_sw = force_w.size() == 1 ? force_w[0] : 0;
    const int force_si = force_i.size() == 1 ? force_i[0] : 0;
    for (int sw = 1; sw <= max_s[0]; ++sw) {
        for (int si = 1; si <= max_s[1]; ++si) {
            if (force_sw > 0 && sw != std::min(force_sw, max_s[0])) continue;
            if (force_si > 0 && si != std::min(force_si, max_s[1])) continue;
            if (force_w.size() > 1 && sw > 1) continue;
            if (force_i.size() > 1 && si > 1) continue;
            Layout L;
            L.splits[UNIT_DWEIGHT].assign(ntiles[0], sw);
            L.splits[UNIT_DINP].assign(ntiles[1], si);
            const double t = plan_cost(g, L, dev, cm, tile_bytes, trace ? 1e300 : best);
            if (trace)
                std::fprintf(stderr, "mmb plan: dweight splits %d dinp splits %d cost %.2f us\n", sw,
                             si, t);
            if (t < best - 1e-9) {
                best = t;
                best_L = L;
            }
        }
    }
    // Tail splits: with the dinp tiles unsplit, also try splitting only the
    // dinp tiles of the last `rows` tile rows.  The launch order runs those
    // last (more splits, shorter units), so they fill the slots that
    // free up while the last wave of whole units is still running.  The
    // model is optimistic about these layouts (GPT-2 XL fc, 8x1024x1600x6400
    // bf16: 11 % predicted, 1-3 % measured), so one is taken only when it is
    // modelled at least 5 % faster than the best uniform layout, and only for
    // bf16, the kernel on which a tail layout was measured.
    if (dtype == MMB_BF16 && force_w.empty() && force_i.empty() &&
        best_L.splits[UNIT_DINP][0] == 1) {
        const GemmPlan& gi = g[UNIT_DINP];
        const Layout base = best_L;
        const double uniform_best = best;
        best = uniform_best * 0.95;   // the margin a tail layout has to beat
        for (int s2 = 2; s2 <= std::min(4, max_s[1]); ++s2)
            for (int eighths = 1; eighths <= 4; ++eighths) {
                const int rows = gi.tiles_m * eighths / 8;
                if (rows < 1) continue;
                Layout L = base;
                for (int t = 0; t < ntiles[1]; ++t)
                    if (t / gi.tiles_n >= gi.tiles_m - rows) L.splits[UNIT_DINP][t] = s2;
                const double t = plan_cost(g, L, dev, cm, tile_bytes, trace ? 1e300 : best);
                if (trace)
                    std::fprintf(stderr, "mmb plan: dweight splits %d, dinp splits %d on the last %d "
                                 "tile rows: cost %.2f us\n", L.splits[UNIT_DWEIGHT][0], s2, rows, t);
                if (t < best - 1e-9) {
                    best = t;
                    best_L = L;
                }
            }
        if (best >= uniform_best * 0.95) best = uniform_best;   // none cleared the margin
    }
    const std::vector<int>* lists[2] = {&force_w, &force_i};
    for (int k = 0; k < 2; ++k) {
        if (lists[k]->size() <= 1) continue;
        for (int t = 0; t < ntiles[k]; ++t)
            best_L.splits[k][t] = std::min((*lists[k])[t % lists[k]->size()], g[k].kiters);
    }

    Plan p;
    std::memset(&p.proto, 0, sizeof(p.proto));
    p.units = make_units(g, best_L, dev);
    long long slots = 0;
    for (int k = 0; k < 2; ++k)
        for (int s : best_L.splits[k]) {
            p.max_splits[k] = std::max(p.max_splits[k], s);
            if (s > 1) slots += s;
        }
    p.ws_floats = slots * ts.BM * ts.BN;
    p.ws_bias_floats = bias ? slots * ts.BM : 0;
    p.n_counters = ntiles[0] + ntiles[1];
    p.proto.BT = BT;
    p.proto.C = C;
    p.proto.OC = OC;
    p.proto.g[0] = g[0];
    p.proto.g[1] = g[1];
    p.proto.n_units = (int)p.units.size();
    return p;
}

// The forward launch: one GEMM (M = BT, N = OC, K = C) in slot UNIT_FWD, the
// other slot empty, and one split count for all its tiles, chosen by the
// same event model (a split forward tile sums its partials like a dinp tile;
// only its epilogue differs, adding the bias instead of the old output).
// MMB_SPLITS_FWD forces the count as MMB_SPLITS_DINP does for dinp.
Plan build_plan_forward(int dtype, int BT, int C, int OC, bool bias, const DeviceInfo& dev,
                        const PlanOptions& opt) {
    const std::vector<int>& force = opt.force_i;
    const TileShape ts = tile_shape(dtype);
    GemmPlan g[2];
    g[UNIT_DWEIGHT] = GemmPlan{0, 0, 0, 0, 0, 0, 0};
    g[UNIT_FWD] = GemmPlan{BT, OC, C, cdiv(BT, ts.BM), cdiv(OC, ts.BN), cdiv(C, ts.BK), 0};
    const int ntiles = g[UNIT_FWD].tiles_m * g[UNIT_FWD].tiles_n;
    const CostModel cm = cost_model(dtype, opt.model);
    const double tile_bytes = 4.0 * ts.BM * ts.BN;
    const int max_s = std::min(8, g[UNIT_FWD].kiters);
    const bool trace = opt.trace;
    Layout best_L;
    double best = 1e300;
    for (int si = 1; si <= max_s; ++si) {
        if (force.size() == 1 && si != std::min(force[0], max_s)) continue;
        if (force.size() > 1 && si > 1) continue;
        Layout L;
        L.splits[UNIT_FWD].assign(ntiles, si);
        const double t = plan_cost(g, L, dev, cm, tile_bytes, trace ? 1e300 : best);
        if (trace) std::fprintf(stderr, "mmb plan: forward splits %d cost %.2f us\n", si, t);
        if (t < best - 1e-9) {
            best = t;
            best_L = L;
        }
    }
    if (force.size() > 1)
        for (int t = 0; t < ntiles; ++t)
            best_L.splits[UNIT_FWD][t] = std::min(force[t % force.size()], g[UNIT_FWD].kiters);

    Plan p;
    std::memset(&p.proto, 0, sizeof(p.proto));
    p.units = make_units(g, best_L, dev);
    long long slots = 0;
    for (int s : best_L.splits[UNIT_FWD]) {
        p.max_splits[UNIT_FWD] = std::max(p.max_splits[UNIT_FWD], s);
        if (s > 1) slots += s;
    }
    (void)bias;
    p.ws_floats = slots * ts.BM * ts.BN;
    p.ws_bias_floats = 0;
    p.n_counters = ntiles;
    p.proto.BT = BT;
    p.proto.C = C;
    p.proto.OC = OC;
    p.proto.g[0] = g[0];
    p.proto.g[1] = g[1];
    p.proto.n_units = (int)p.units.size();
    return p;
}

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
    if (!choose_path(dinp, dweight, dout, inp, weight, C, OC, dtype)) {
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
    TraceRange range("mmb launch");
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
    const hipError_t e = sr ? launch_tiles_bf16_sr(tp, s) : launch_tiles(dtype, tp, s);
    return e == hipSuccess ? MMB_OK : MMB_ERR_HIP;
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
    if (!choose_path(dinp, dweight, dout, inp, weight, C, OC, dtype)) {
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
    // scratch layout: counters, work list, dbias partials, tile partials
    // (each part 256-byte aligned), all sizes in 64 bits
    const size_t cb = align_up((size_t)plan.n_counters * 4, 256);
    const size_t ub = align_up(plan.units.size() * sizeof(Unit), 256);
    const size_t bb = align_up((size_t)plan.ws_bias_floats * 4, 256);
    const size_t wb = align_up((size_t)plan.ws_floats * 4, 256);
    if (cb + ub + bb + wb > (size_t)MMB_NOALLOC_SCRATCH_BYTES) return MMB_ERR_SCRATCH;
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
    return launch_tiles(dtype, tp, s) == hipSuccess ? MMB_OK : MMB_ERR_HIP;
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
int ln_path(const void* dinp, const void* dout, const void* inp, const void* weight, int C,
            int dtype) {
    const void* ptrs[4] = {dinp, dout, inp, weight};
    for (const void* p : ptrs)
        if ((uintptr_t)p % 16 != 0) return 0;
    return ln_vectors_per_lane(dtype, C);
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
    const int nj = ln_path(dinp, dout, inp, weight, C, dtype);
    int G = 0;
    // held through the launch: another call may not regrow the partials first
    std::unique_lock<std::mutex> lock(g_mu, std::defer_lock);
    if (nj > 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return MMB_ERR_HIP;
        lock.lock();
        DeviceInfo di;
        st = device_info(dev, &di);
        if (st != MMB_OK) return st;
        // one workgroup of 8 row-waves per CU (fewer for few rows);
        // MMB_LN_WORKGROUPS overrides the count (tuning aid)
        long long want = di.cus;
        if (const char* e = g_tune.get(T_LN_WORKGROUPS)) {
            const long v = std::strtol(e, nullptr, 10);
            if (v > 0) want = std::min(v, 1L << 16);
        }
        G = (int)std::max(1LL, std::min<long long>(want, (p.BT + 7) / 8));
        Workspace& w = g_ws[{dev, s}];
        st = grow(dev, &w.partials, &w.partial_bytes, (size_t)G * 2 * C * sizeof(float), false, s);
        if (st != MMB_OK) return st;
        p.partial = (float*)w.partials.ptr;
    }
    TraceRange range("mmb layernorm launch");
    return launch_layernorm_backward(dtype, p, G, nj, s) == hipSuccess ? MMB_OK : MMB_ERR_HIP;
}

int forward_impl(void* out, const void* inp, const void* weight, const void* bias, int B, int T,
                 int C, int OC, int dtype, hipStream_t s) {
    int st = check_fwd(out, inp, weight, bias, B, T, C, OC, dtype);
    if (st != MMB_OK) return st;
    const int BT = B * T;
    if (!choose_path_fwd(out, inp, weight, bias, C, OC, dtype)) {
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
    TraceRange range("mmb forward launch");
    TilesParams tp = plan->plan.proto;
    st = get_workspace(dev, s, *plan, &tp);
    if (st != MMB_OK) return st;
    tp.out = out;
    tp.bias = bias;
    tp.inp = inp;
    tp.weight = weight;
    return launch_fwd_tiles(dtype, tp, s) == hipSuccess ? MMB_OK : MMB_ERR_HIP;
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
    return mmb::ln_path(dinp, dout, inp, weight, C, dtype) > 0 ? 1 : 0;
}

int mmb_forward_check_args(const void* out, const void* inp, const void* weight, const void* bias,
                           int B, int T, int C, int OC, int dtype) {
    return mmb::check_fwd(out, inp, weight, bias, B, T, C, OC, dtype);
}

int mmb_forward_path(const void* out, const void* inp, const void* weight, const void* bias, int B,
                     int T, int C, int OC, int dtype) {
    const int st = mmb::check_fwd(out, inp, weight, bias, B, T, C, OC, dtype);
    if (st != MMB_OK) return st;
    return mmb::choose_path_fwd(out, inp, weight, bias, C, OC, dtype);
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
    return mmb::choose_path(dinp, dweight, dout, inp, weight, C, OC, dtype);
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
