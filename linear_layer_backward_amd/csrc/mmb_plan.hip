// mmb_plan.hip -- the launch planner of the MFMA tile kernels (host code
// only): an event model of one launch picks the split-K counts, and the work
// list is ordered for the XCDs' L2s.  Declared in mmb_plan.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <queue>
#include <unordered_map>
#include <vector>

#include "../../include/mmb.h"
#include "mmb_plan.h"

namespace mmb {

int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

void set_topology(DeviceInfo* d) {
    d->xcds = d->cus >= 128 ? 8 : 1;
    const int per_xcd = d->cus / d->xcds;
    d->ses = per_xcd >= 16 && per_xcd % 4 == 0 ? 4 : 1;
}

namespace {

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
// come first; among equal ones, units are ordered (split, tile_m, tile_n), so
// that the units an XCD runs together share one K range: the tile_n units of
// a tile_m share its A rows (dout) and the tile_m units share the B slab of
// each tile_n (inp for dweight, weight for dinp).  Ordered (tile_m, split,
// tile_n) instead, every XCD ran every K range of the LM head's dinp and
// fetched the whole 77 MB weight.  Every run of equal split counts, of the GEMM
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
            for (int s = 0; s < S; ++s)
                for (int m = 0; m < G.tiles_m; ++m)
                    for (int n = 0; n < G.tiles_n; ++n) emit(m, n, s);
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

}  // namespace

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
    p.proto.ldo = OC;
    p.proto.ldc = C;
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
    p.proto.ldo = OC;
    p.proto.ldc = C;
    p.proto.g[0] = g[0];
    p.proto.g[1] = g[1];
    p.proto.n_units = (int)p.units.size();
    return p;
}

}  // namespace mmb
