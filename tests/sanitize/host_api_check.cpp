// Host-side checks of libmmb.so under AddressSanitizer / UndefinedBehavior-
// Sanitizer: every entry point that runs on the host only (argument checks,
// path choice, the launch planner with its event model, the tuning
// overrides, status strings), over many shapes, CU counts and override
// strings, malformed ones included.  Pointers are fake, well separated
// addresses that nothing dereferences.  Exit status 0 when every plan is
// consistent; the sanitizers abort on any memory or undefined-behaviour
// error.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/mmb.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int a = 0, int b = 0, int c = 0, int d = 0) {
    if (!ok) {
        std::printf("FAIL %s (%d %d %d %d)\n", what, a, b, c, d);
        ++failures;
    }
}

void* addr(int k) { return (void*)(uintptr_t)((1ull << 40) + (uint64_t)k * (1ull << 44)); }

// A plan's units: every tile of both GEMMs covered, K ranges inside [0, kiters).
void check_plan(int B, int T, int C, int OC, int dtype, int bias, int cus) {
    int splits[2] = {0, 0};
    const int n = mmb_plan_units(B, T, C, OC, dtype, bias, cus, splits, nullptr, 0);
    expect(n > 0, "plan unit count", B * T, C, OC, cus);
    if (n <= 0) return;
    std::vector<int> units((size_t)n * 8);
    const int m = mmb_plan_units(B, T, C, OC, dtype, bias, cus, splits, units.data(), n);
    expect(m == n, "plan unit count repeat", B * T, C, OC, cus);
    int shape[3];
    expect(mmb_tile_shape(dtype, shape) == MMB_OK, "tile shape");
    const long long BT = (long long)B * T;
    const int kit[2] = {(int)((BT + shape[2] - 1) / shape[2]), (OC + shape[2] - 1) / shape[2]};
    for (int i = 0; i < n; ++i) {
        const int* u = &units[(size_t)i * 8];
        const int kind = u[0];
        expect(kind == 0 || kind == 1, "unit kind", kind);
        if (kind != 0 && kind != 1) continue;
        expect(u[4] >= 0 && u[4] < u[5] && u[5] <= kit[kind], "unit K range", u[4], u[5], kit[kind]);
        expect(u[3] >= 0 && u[3] < u[6] && u[6] >= 1, "unit split index", u[3], u[6]);
        expect(u[6] <= splits[kind], "unit splits within the plan's maximum", u[6], splits[kind]);
    }
    int fs[1] = {0};
    const int nf = mmb_forward_plan_units(B, T, C, OC, dtype, bias, cus, fs, nullptr, 0);
    expect(nf > 0, "forward plan", B * T, C, OC, cus);
}

}  // namespace

int main() {
    // status strings
    for (int st = -12; st <= 2; ++st) expect(mmb_strerror(st) != nullptr, "strerror", st);

    // argument checks and path choice
    const int dims[] = {1, 2, 3, 7, 8, 17, 64, 129, 768, 3072};
    for (int dtype = -1; dtype <= 2; ++dtype)
        for (int C : dims)
            for (int OC : dims) {
                const int st = mmb_check_args(addr(0), addr(1), addr(2), addr(3), addr(4), addr(5),
                                              2, 3, C, OC, dtype);
                expect(dtype == 0 || dtype == 1 ? st == MMB_OK : st == MMB_ERR_DTYPE, "check",
                       dtype, C, OC);
                (void)mmb_path(addr(0), addr(1), nullptr, addr(3), addr(4), addr(5), 2, 3, C, OC,
                               dtype);
                (void)mmb_forward_check_args(addr(0), addr(1), addr(2), addr(3), 2, 3, C, OC, dtype);
                (void)mmb_forward_path(addr(0), addr(1), addr(2), nullptr, 2, 3, C, OC, dtype);
                (void)mmb_layernorm_check_args(addr(0), addr(1), addr(2), addr(3), addr(4), addr(5),
                                               addr(6), addr(7), 2, 3, C, dtype);
                (void)mmb_layernorm_path(addr(0), addr(1), addr(2), addr(3), addr(4), addr(5),
                                         addr(6), addr(7), 2, 3, C, dtype);
            }
    expect(mmb_check_args(nullptr, addr(1), nullptr, addr(3), addr(4), addr(5), 1, 1, 1, 1, 0) ==
               MMB_ERR_NULL, "null");
    expect(mmb_check_args(addr(0), addr(1), nullptr, addr(3), addr(4), addr(5), 0, 1, 1, 1, 0) ==
               MMB_ERR_DIM, "dim");
    expect(mmb_check_args(addr(0), addr(1), nullptr, addr(3), addr(4), addr(5), 1 << 16, 1 << 16,
                          1, 1, 0) == MMB_ERR_OVERFLOW, "overflow");
    expect(mmb_check_args(addr(0), addr(0), nullptr, addr(3), addr(4), addr(5), 1, 1, 8, 8, 0) ==
               MMB_ERR_ALIAS, "alias");

    // the planner on the benchmark shapes, GPT-2 layers, ragged and tiny ones
    const int shapes[][4] = {{16, 1024, 768, 3072}, {8, 1024, 768, 50304}, {8, 1024, 768, 50257},
                             {8, 1024, 768, 2304},  {8, 1024, 3072, 768},  {2, 16, 64, 192},
                             {8, 1024, 1600, 6400}, {1, 1, 8, 8},          {3, 100, 200, 328},
                             {1, 513, 200, 136},    {1, 3, 12, 10},        {1, 1, 1, 1}};
    const int cus_list[] = {256, 32, 8, 1, 304};
    for (const auto& s : shapes) {
        // the large shapes (long event simulations) on two CU counts
        const bool large = (long long)s[0] * s[1] * s[3] > (1LL << 24);
        for (int dtype = 0; dtype <= 1; ++dtype)
            for (int cus : cus_list)
                if (!large || cus == 256 || cus == 32)
                    check_plan(s[0], s[1], s[2], s[3], dtype, (s[3] & 1) == 0, cus);
    }

    // tuning overrides, malformed values included; each plan must stay valid
    const char* splits[] = {"", ",", "3,,2", "abc", "-1", "0", "99999999999", "1,2,3,4,5,6,7,8,9,10",
                            "2,3,5", "16,1", nullptr};
    for (const char* w : splits)
        for (const char* i : splits) {
            expect(mmb_set_tuning("MMB_SPLITS_DWEIGHT", w) == MMB_OK, "set dweight splits");
            expect(mmb_set_tuning("MMB_SPLITS_DINP", i) == MMB_OK, "set dinp splits");
            expect(mmb_set_tuning("MMB_SPLITS_FWD", i) == MMB_OK, "set forward splits");
            check_plan(2, 150, 264, 400, 1, 1, 256);
            check_plan(3, 100, 202, 330, 0, 1, 32);
        }
    mmb_set_tuning("MMB_SPLITS_DWEIGHT", nullptr);
    mmb_set_tuning("MMB_SPLITS_DINP", nullptr);
    mmb_set_tuning("MMB_SPLITS_FWD", nullptr);
    const char* models[] = {"1,2,3", "x", "1.4,1.26,0.72,0.97,0.97,0.8,3.8,8.5,2.1,2.5,4.4,1e-3",
                            "1,1,1,0,0,0,0,0,0,0,0,1", nullptr};
    for (const char* m : models) {
        expect(mmb_set_tuning("MMB_PLAN_MODEL", m) == MMB_OK, "set model");
        check_plan(16, 1024, 768, 3072, 1, 1, 256);
    }
    expect(mmb_set_tuning("MMB_NO_SUCH", "1") == MMB_ERR_NAME, "unknown tuning name");
    expect(mmb_set_tuning(nullptr, "1") == MMB_ERR_NULL, "null tuning name");
    std::string long_value(100000, '7');
    expect(mmb_set_tuning("MMB_SPLITS_DWEIGHT", long_value.c_str()) == MMB_OK, "long value");
    check_plan(2, 150, 264, 400, 1, 1, 256);
    mmb_set_tuning("MMB_SPLITS_DWEIGHT", nullptr);

    std::printf("%s: %d failures\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
