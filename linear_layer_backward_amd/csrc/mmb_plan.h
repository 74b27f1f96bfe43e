// mmb_plan.h -- the launch planner of the MFMA tile kernels (host code):
// split-K counts per GEMM from an event model of one launch, and the work
// list in launch order.  Internal to libmmb.so.
#pragma once

#include <string>
#include <vector>

#include "mmb_internal.h"

namespace mmb {

int cdiv(long long a, long long b);

// The device as the planner sees it.
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
void set_topology(DeviceInfo* d);

struct Unit {
    int4 a;   // {kind, tile_m, tile_n, split}
    int4 b;   // {kt0, kt1, splits of the tile, first workspace slot of the tile}
};

struct Plan {
    TilesParams proto;            // pointers filled per call
    std::vector<Unit> units;      // launch order
    int max_splits[2] = {1, 1};   // largest split count of each GEMM's tiles
    long long ws_floats = 0;
    long long ws_bias_floats = 0;
    int n_counters = 0;
};

// What the planner takes from the tuning overrides.
struct PlanOptions {
    std::vector<int> force_w, force_i;   // split overrides (dweight / dinp, or the forward)
    const char* model = nullptr;         // MMB_PLAN_MODEL constants, or NULL
    bool trace = false;                  // print every modelled candidate to stderr
};

// Split overrides: empty = the planner chooses; one value = that count for
// every tile of the GEMM; several values = tile t gets value t mod count
// (clamped to the tile's K iterations; for tests of uneven plans).
std::vector<int> parse_splits(const char* v);

// The backward launch (dweight in plan slot UNIT_DWEIGHT, dinp in UNIT_DINP).
Plan build_plan(int dtype, int BT, int C, int OC, bool bias, const DeviceInfo& dev,
                const PlanOptions& opt);
// The forward launch: one GEMM (M = BT, N = OC, K = C) in slot UNIT_FWD.
Plan build_plan_forward(int dtype, int BT, int C, int OC, bool bias, const DeviceInfo& dev,
                        const PlanOptions& opt);

}  // namespace mmb
