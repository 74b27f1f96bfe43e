"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every function include/mmb.h declares, validates arguments and plans work.
Pointers here are fake addresses; nothing dereferences them."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mmb.h")


@pytest.fixture(scope="module")
def mmb():
    lib = os.path.join(ROOT, "linear_layer_backward_amd", "libmmb.so")
    if not os.path.exists(lib):
        from linear_layer_backward_amd import build
        build.build()
    from linear_layer_backward_amd import mmb as m
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mmb_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for f in ("mmb_backward", "mmb_backward_stream", "mmb_check_args", "mmb_strerror",
              "mmb_release", "mmb_path", "mmb_plan_units", "mmb_tile_shape"):
        assert f in names


def test_library_exports_every_declared_symbol(mmb):
    out = subprocess.run(["nm", "-D", "--defined-only", mmb.LIBRARY], check=True,
                         stdout=subprocess.PIPE, text=True).stdout
    exported = set(re.findall(r"\bT (mmb_\w+)$", out, flags=re.M))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    # exported C names only: nothing mangled from the mmb namespace leaks as T
    for f in declared_functions():
        assert hasattr(mmb._lib, f)


# fake, 256-byte aligned, well separated device addresses
BASE = 1 << 40
GAP = 1 << 44


def addrs(n=6):
    return [BASE + k * GAP for k in range(n)]


def args(dtype=1, B=16, T=1024, C=768, OC=3072, bias=True):
    dinp, dweight, dbias, dout, inp, weight = addrs()
    return [dinp, dweight, dbias if bias else None, dout, inp, weight, B, T, C, OC, dtype]


def test_valid_arguments(mmb):
    assert mmb.mmb_check_args(*args()) == 0
    assert mmb.mmb_check_args(*args(bias=False)) == 0
    assert mmb.mmb_check_args(*args(dtype=0, B=1, T=1, C=1, OC=1)) == 0


@pytest.mark.parametrize("idx", [0, 1, 3, 4, 5])
def test_null_pointers(mmb, idx):
    a = args()
    a[idx] = None
    assert mmb.mmb_check_args(*a) == -1


@pytest.mark.parametrize("idx", [6, 7, 8, 9])
@pytest.mark.parametrize("val", [0, -1])
def test_bad_dims(mmb, idx, val):
    a = args()
    a[idx] = val
    assert mmb.mmb_check_args(*a) == -2


@pytest.mark.parametrize("dt", [-1, 2, 7])
def test_bad_dtype(mmb, dt):
    assert mmb.mmb_check_args(*args(dtype=dt)) == -3


def test_overflow(mmb):
    assert mmb.mmb_check_args(*args(B=65536, T=32768, C=8, OC=8)) == -4
    assert mmb.mmb_check_args(*args(B=65535, T=32768, C=8, OC=8)) == 0


def test_alias(mmb):
    a = args(dtype=0, B=2, T=4, C=8, OC=8)  # fp32: dinp holds 64 floats = 256 B
    a[1] = a[0] + 255                         # dweight starts inside dinp
    assert mmb.mmb_check_args(*a) == -5
    a[1] = a[0] + 256                         # adjacent, not overlapping
    assert mmb.mmb_check_args(*a) == 0
    b = args(dtype=1)
    b[2] = b[3] + 2                           # dbias inside dout
    assert mmb.mmb_check_args(*b) == -5
    c = args(dtype=1)
    c[0] = c[4]                               # dinp == inp
    assert mmb.mmb_check_args(*c) == -5
    d = args(dtype=1)
    d[4] = d[5]                               # inputs may share memory
    assert mmb.mmb_check_args(*d) == 0


def test_strerror(mmb):
    for st in range(-7, 1):
        assert mmb.mmb_strerror(st)
    assert "unknown" in mmb.mmb_strerror(-99)


def test_path_choice(mmb):
    assert mmb.mmb_path(*args(dtype=1)) == 1
    # ragged rows take the MFMA tiles on packed copies
    assert mmb.mmb_path(*args(dtype=1, C=764)) == 1          # C % 8 != 0 (bf16)
    assert mmb.mmb_path(*args(dtype=0, C=764)) == 1          # C % 4 == 0 (fp32)
    assert mmb.mmb_path(*args(dtype=0, OC=3070)) == 1
    assert mmb.mmb_path(*args(dtype=1, B=8, C=768, OC=50257, bias=False)) == 1
    assert mmb.mmb_path(*args(dtype=1, C=1 << 23)) == 0      # beyond the tiles' offsets
    assert mmb.mmb_path(*args(dtype=1, OC=(1 << 22) + 8)) == 0
    # buffers off the 16-byte alignment go through packed copies; a buffer
    # not aligned to its element size takes the generic path
    for i, dt, off, want in [(4, 1, 8, 1), (4, 1, 2, 1), (3, 1, 14, 1), (0, 1, 2, 1),
                             (1, 0, 4, 1), (5, 0, 12, 1), (4, 1, 1, 0), (0, 0, 2, 0),
                             (5, 0, 6, 0)]:
        a = args(dtype=dt)
        a[i] += off
        assert mmb.mmb_path(*a) == want, (i, dt, off)
    b = args(dtype=1)
    b[2] += 1                                                  # dbias alignment is free
    assert mmb.mmb_path(*b) == 1
    assert mmb.mmb_path(*args(dtype=5)) == -3


@pytest.mark.parametrize("shape", [
    (16, 1024, 768, 3072, 1, True), (8, 1024, 768, 50304, 1, False),
    (8, 1024, 768, 2304, 0, True), (8, 1024, 3072, 768, 0, True), (2, 16, 64, 192, 0, True),
    (3, 100, 200, 328, 0, True), (1, 1, 8, 8, 1, True), (8, 1024, 1600, 6400, 1, True)])
@pytest.mark.parametrize("cus", [256, 32])
def test_plan_covers_every_tile_and_split_once(mmb, shape, cus):
    B, T, C, OC, dt, bias = shape
    (sw, si), units = mmb.mmb_plan_units(B, T, C, OC, dt, bias, cus)
    BM, BN, BK = mmb.mmb_tile_shape(dt)
    cd = lambda a, b: -(-a // b)
    kiters = {0: cd(B * T, BK), 1: cd(OC, BK)}
    tiles = {0: (cd(OC, BM), cd(C, BN)), 1: (cd(B * T, BM), cd(C, BN))}
    by_tile = {}
    for u in units:
        kind, m, n, s, kt0, kt1, S, slot = u
        assert 0 <= m < tiles[kind][0] and 0 <= n < tiles[kind][1]
        by_tile.setdefault((kind, m, n), []).append(u)
    assert len(by_tile) == sum(a * b for a, b in tiles.values())
    used = []
    for (kind, m, n), us in by_tile.items():
        S = us[0][6]
        assert all(u[6] == S for u in us) and all(u[7] == us[0][7] for u in us)
        assert sorted(u[3] for u in us) == list(range(S))
        # the K ranges of the tile's units partition [0, kiters) in split order
        rng = sorted((u[3], u[4], u[5]) for u in us)
        assert rng[0][1] == 0 and rng[-1][2] == kiters[kind]
        assert all(a[2] == b[1] for a, b in zip(rng, rng[1:]))
        assert all(lo < hi for _, lo, hi in rng)
        if S > 1:
            used.append((us[0][7], S))
    # split tiles own disjoint runs of workspace slots
    used.sort()
    assert all(a + s <= b for (a, s), (b, _) in zip(used, used[1:]))
    assert used == [] or used[0][0] == 0
    maxs = {k: max((u[6] for u in units if u[0] == k), default=1) for k in (0, 1)}
    assert (sw, si) == (maxs[0], maxs[1])
    assert 1 <= sw <= kiters[0] and 1 <= si <= kiters[1]


def test_tile_shape(mmb):
    assert mmb.mmb_tile_shape(0) == (128, 128, 32)
    bm, bn, bk = mmb.mmb_tile_shape(1)
    assert bm % 32 == 0 and bn % 32 == 0 and bk % 16 == 0
    with pytest.raises(mmb.MmbError):
        mmb.mmb_tile_shape(7)


@pytest.mark.parametrize("lists", [("2,3,5", "1,2"), ("16,1", "8")])
def test_plan_per_tile_split_lists(mmb, tune, lists):
    tune.set("MMB_SPLITS_DWEIGHT", lists[0])
    tune.set("MMB_SPLITS_DINP", lists[1])
    test_plan_covers_every_tile_and_split_once(mmb, (1, 700, 520, 600, 1, True), 256)
    B, T, C, OC = 1, 700, 520, 600
    BM, BN, BK = mmb.mmb_tile_shape(1)
    cd = lambda a, b: -(-a // b)
    want = {0: [int(x) for x in lists[0].split(",")], 1: [int(x) for x in lists[1].split(",")]}
    kit = {0: cd(B * T, BK), 1: cd(OC, BK)}
    tn = cd(C, BN)
    _, units = mmb.mmb_plan_units(B, T, C, OC, 1, True, 256)
    for u in units:
        kind, m, n = u[0], u[1], u[2]
        t = m * tn + n
        assert u[6] == min(want[kind][t % len(want[kind])], kit[kind])


def test_plan_split_override(mmb, tune):
    tune.set("MMB_SPLITS_DWEIGHT", "3")
    tune.set("MMB_SPLITS_DINP", "2")
    (sw, si), units = mmb.mmb_plan_units(2, 150, 264, 400, 1, True, 256)
    assert (sw, si) == (3, 2)
    assert all(u[6] == (3 if u[0] == 0 else 2) for u in units)


def test_plan_deals_each_split_level_evenly_over_xcds(mmb, tune):
    """Workgroup i runs on XCD i % 8; every run of equal split counts of a
    GEMM is spread over the 8 XCDs within one unit of each other."""
    tune.set("MMB_SPLITS_DWEIGHT", "4")
    tune.set("MMB_SPLITS_DINP", ",".join(["1"] * 5 + ["2", "3"]))
    _, units = mmb.mmb_plan_units(16, 1024, 768, 3072, 1, True, 256)
    levels = {}
    for i, u in enumerate(units):
        levels.setdefault((u[0], u[6]), [0] * 8)[i % 8] += 1
    assert sorted(levels) == [(0, 4), (1, 1), (1, 2), (1, 3)]
    for counts in levels.values():
        assert max(counts) - min(counts) <= 1


@pytest.mark.parametrize("shape,want", [
    ((16, 1024, 768, 3072, 1, True), (4, 1)),     # GPT-2 fc, bf16
    ((8, 1024, 768, 50304, 1, False), (1, 2)),    # GPT-2 LM head, bf16
    ((8, 1024, 768, 2304, 0, True), (13, 1)),     # GPT-2 qkv, fp32
    ((8, 1024, 768, 3072, 0, True), (2, 4)),      # GPT-2 fc, fp32
    ((8, 1024, 3072, 768, 0, True), (2, 1)),      # GPT-2 fc_proj, fp32
], ids=["fc_bf16", "lm_head_bf16", "qkv_f32", "fc_f32", "fc_proj_f32"])
def test_plan_picks_the_measured_best_splits(mmb, tune, shape, want):
    """On a 256-CU MI355X the planner's model picks the split counts that
    timed fastest in forced-split sweeps of these shapes."""
    tune.clear("MMB_SPLITS_DWEIGHT")
    tune.clear("MMB_SPLITS_DINP")
    tune.clear("MMB_PLAN_MODEL")
    B, T, C, OC, dt, bias = shape
    (sw, si), _ = mmb.mmb_plan_units(B, T, C, OC, dt, bias, 256)
    assert (sw, si) == want


def test_plan_tail_layout_on_gpt2_xl_fc(mmb, tune):
    """GPT-2 XL fc (bf16, 256 CUs): the planner splits only the dinp tiles of
    the last 12 of 32 tile rows, 2 ways, and those units launch after every
    unsplit dinp unit, so they fill the slots that free up at the end."""
    for k in ("MMB_SPLITS_DWEIGHT", "MMB_SPLITS_DINP", "MMB_PLAN_MODEL"):
        tune.clear(k)
    (sw, si), units = mmb.mmb_plan_units(8, 1024, 1600, 6400, 1, True, 256)
    assert (sw, si) == (1, 2)
    dinp = [(i, u) for i, u in enumerate(units) if u[0] == 1]
    split = {(u[1], u[2]) for _, u in dinp if u[6] == 2}
    assert split == {(m, n) for m in range(20, 32) for n in range(7)}
    assert all(u[6] == 1 for u in units if u[0] == 0)
    last_whole = max(i for i, u in dinp if u[6] == 1)
    assert all(i > last_whole for i, u in dinp if u[6] == 2)


# The planner's choices (largest dweight and dinp split counts, and whether
# the dinp tiles take a tail layout) on the bf16 linear layers of the four
# GPT-2 sizes at B=8, T=1024, for the 256 CUs of an MI355X and a 32-CU
# partition.  Only the 1558M fc layer on 256 CUs takes a tail layout.
GPT2_WIDTHS = {"124M": 768, "350M": 1024, "774M": 1280, "1558M": 1600}
GPT2_PLANS = {
    ("124M", 256): {"qkv": (5, 1), "attn_proj": (8, 1), "fc": (4, 1), "fc_proj": (4, 1)},
    ("124M", 32): {"qkv": (1, 1), "attn_proj": (3, 1), "fc": (1, 1), "fc_proj": (1, 1)},
    ("350M", 256): {"qkv": (2, 1), "attn_proj": (7, 1), "fc": (2, 1), "fc_proj": (2, 1)},
    ("350M", 32): {"qkv": (1, 1), "attn_proj": (1, 1), "fc": (1, 1), "fc_proj": (1, 1)},
    ("774M", 256): {"qkv": (1, 1), "attn_proj": (6, 1), "fc": (1, 3), "fc_proj": (1, 1)},
    ("774M", 32): {"qkv": (1, 1), "attn_proj": (1, 1), "fc": (1, 1), "fc_proj": (1, 1)},
    ("1558M", 256): {"qkv": (2, 1), "attn_proj": (3, 1), "fc": (1, 2), "fc_proj": (1, 1)},
    ("1558M", 32): {"qkv": (1, 1), "attn_proj": (1, 1), "fc": (1, 1), "fc_proj": (1, 1)},
}


@pytest.mark.parametrize("model,cus", sorted(GPT2_PLANS))
def test_plan_choices_on_gpt2_layers(mmb, tune, model, cus):
    for k in ("MMB_SPLITS_DWEIGHT", "MMB_SPLITS_DINP", "MMB_PLAN_MODEL"):
        tune.clear(k)
    C = GPT2_WIDTHS[model]
    shapes = {"qkv": (C, 3 * C), "attn_proj": (C, C), "fc": (C, 4 * C), "fc_proj": (4 * C, C)}
    for layer, (c, oc) in shapes.items():
        (sw, si), units = mmb.mmb_plan_units(8, 1024, c, oc, 1, True, cus)
        assert (sw, si) == GPT2_PLANS[(model, cus)][layer], (model, cus, layer)
        counts = {k: {u[6] for u in units if u[0] == k} for k in (0, 1)}
        tail = (model, cus, layer) == ("1558M", 256, "fc")
        assert len(counts[0]) == 1
        assert len(counts[1]) == (2 if tail else 1), (model, cus, layer)


def test_plan_tail_layouts_are_bf16_only(mmb, tune):
    """fp32 takes one split count per GEMM on the same shapes (no tail layout
    was measured on the fp32 kernel)."""
    for k in ("MMB_SPLITS_DWEIGHT", "MMB_SPLITS_DINP", "MMB_PLAN_MODEL"):
        tune.clear(k)
    for C in GPT2_WIDTHS.values():
        for c, oc in ((C, 3 * C), (C, C), (C, 4 * C), (4 * C, C)):
            for cus in (256, 32):
                _, units = mmb.mmb_plan_units(8, 1024, c, oc, 0, True, cus)
                for k in (0, 1):
                    assert len({u[6] for u in units if u[0] == k}) <= 1


def test_tuning_is_read_once_at_load(mmb, tune, monkeypatch):
    """The environment is read when the library loads: a variable set later
    changes nothing; mmb_set_tuning does."""
    tune.clear("MMB_SPLITS_DWEIGHT")
    tune.clear("MMB_SPLITS_DINP")
    tune.clear("MMB_PLAN_MODEL")
    shape = (16, 1024, 768, 3072, 1, True)
    base = mmb.mmb_plan_units(*shape, 256)[0]
    monkeypatch.setenv("MMB_SPLITS_DWEIGHT", "7")
    assert mmb.mmb_plan_units(*shape, 256)[0] == base
    tune.set("MMB_SPLITS_DWEIGHT", "7")
    assert mmb.mmb_plan_units(*shape, 256)[0][0] == 7
    tune.clear("MMB_SPLITS_DWEIGHT")
    assert mmb.mmb_plan_units(*shape, 256)[0] == base


def test_set_tuning_rejects_unknown_names(mmb):
    assert mmb._lib.mmb_set_tuning(b"MMB_NOT_A_VARIABLE", b"1") == -8
    assert mmb._lib.mmb_set_tuning(None, b"1") == -1
    with pytest.raises(mmb.MmbError):
        mmb.mmb_set_tuning("MMB_SPLITS", "2")
    assert "tuning" in mmb.mmb_strerror(-8)


def test_plan_model_override(mmb, tune):
    """MMB_PLAN_MODEL replaces the cost constants; a malformed value is
    ignored."""
    tune.clear("MMB_SPLITS_DWEIGHT")
    tune.clear("MMB_SPLITS_DINP")
    shape = (16, 1024, 768, 3072, 1, True)
    base = mmb.mmb_plan_units(*shape, 256)[0]
    tune.set("MMB_PLAN_MODEL", "1,2,3")
    assert mmb.mmb_plan_units(*shape, 256)[0] == base
    # splitting made ruinous: every partial costs a millisecond of traffic
    tune.set("MMB_PLAN_MODEL", "1.4,1.26,0.72,0.97,0.97,0.8,3.8,8.5,2.1,2.5,4.4,1e-3")
    assert mmb.mmb_plan_units(*shape, 256)[0] == (1, 1)


# ---------------------------------------------------------------------------
# the forward product: out = inp . W^T + bias

def fargs(dtype=1, B=16, T=1024, C=768, OC=3072, bias=True):
    out, inp, weight, b = addrs(4)
    return [out, inp, weight, b if bias else None, B, T, C, OC, dtype]


def test_header_declares_the_forward_entry_points():
    names = declared_functions()
    for f in ("mmb_forward", "mmb_forward_stream", "mmb_forward_check_args", "mmb_forward_path",
              "mmb_forward_plan_units"):
        assert f in names


def test_forward_valid_arguments(mmb):
    assert mmb.mmb_forward_check_args(*fargs()) == 0
    assert mmb.mmb_forward_check_args(*fargs(bias=False)) == 0
    assert mmb.mmb_forward_check_args(*fargs(dtype=0, B=1, T=1, C=1, OC=1)) == 0


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_forward_null_pointers(mmb, idx):
    a = fargs()
    a[idx] = None
    assert mmb.mmb_forward_check_args(*a) == -1


@pytest.mark.parametrize("idx", [4, 5, 6, 7])
@pytest.mark.parametrize("val", [0, -3])
def test_forward_bad_dims(mmb, idx, val):
    a = fargs()
    a[idx] = val
    assert mmb.mmb_forward_check_args(*a) == -2


def test_forward_bad_dtype_and_overflow(mmb):
    assert mmb.mmb_forward_check_args(*fargs(dtype=2)) == -3
    assert mmb.mmb_forward_check_args(*fargs(B=65536, T=32768, C=8, OC=8)) == -4
    assert mmb.mmb_forward_check_args(*fargs(B=65535, T=32768, C=8, OC=8)) == 0


def test_forward_alias(mmb):
    a = fargs(dtype=0, B=2, T=4, C=8, OC=8)   # fp32: out holds 64 floats = 256 B
    a[1] = a[0] + 252                          # inp starts inside out
    assert mmb.mmb_forward_check_args(*a) == -5
    a[1] = a[0] + 256                          # adjacent
    assert mmb.mmb_forward_check_args(*a) == 0
    b = fargs(dtype=1)
    b[3] = b[0] + 2                            # bias inside out
    assert mmb.mmb_forward_check_args(*b) == -5
    c = fargs(dtype=1)
    c[2] = c[1]                                # inputs may share memory
    assert mmb.mmb_forward_check_args(*c) == 0


def test_forward_path_choice(mmb):
    assert mmb.mmb_forward_path(*fargs(dtype=1)) == 1
    assert mmb.mmb_forward_path(*fargs(dtype=1, bias=False)) == 1
    # ragged rows and buffers off the 16-byte alignment: MFMA tiles on packed
    # copies; a buffer not aligned to its element size: the generic path
    assert mmb.mmb_forward_path(*fargs(dtype=1, C=764)) == 1
    assert mmb.mmb_forward_path(*fargs(dtype=0, C=764)) == 1
    assert mmb.mmb_forward_path(*fargs(dtype=0, OC=3070)) == 1
    assert mmb.mmb_forward_path(*fargs(dtype=1, B=8, C=768, OC=50257)) == 1
    assert mmb.mmb_forward_path(*fargs(dtype=1, OC=1 << 23)) == 0
    for i, dt, off, want in [(3, 1, 2, 1), (0, 1, 8, 1), (1, 0, 4, 1), (2, 1, 6, 1),
                             (3, 1, 1, 0), (0, 0, 2, 0), (1, 1, 3, 0)]:
        a = fargs(dtype=dt)
        a[i] += off
        assert mmb.mmb_forward_path(*a) == want, (i, dt, off)
    assert mmb.mmb_forward_path(*fargs(dtype=4)) == -3


@pytest.mark.parametrize("shape", [
    (16, 1024, 768, 3072, 1), (8, 1024, 768, 50304, 1), (16, 1024, 3072, 768, 1),
    (8, 1024, 768, 2304, 0), (8, 1024, 3072, 768, 0), (2, 16, 64, 192, 0), (1, 1, 8, 8, 1)])
@pytest.mark.parametrize("cus", [256, 32])
def test_forward_plan_covers_every_tile_once(mmb, shape, cus):
    """M = B*T rows, N = OC columns, K = C; every output tile appears with K
    ranges that partition [0, kiters) in split order."""
    B, T, C, OC, dt = shape
    smax, units = mmb.mmb_forward_plan_units(B, T, C, OC, dt, True, cus)
    BM, BN, BK = mmb.mmb_tile_shape(dt)
    cd = lambda a, b: -(-a // b)
    tm, tn, kiters = cd(B * T, BM), cd(OC, BN), cd(C, BK)
    by_tile = {}
    for u in units:
        kind, m, n, s, kt0, kt1, S, slot = u
        assert kind == 1 and 0 <= m < tm and 0 <= n < tn
        by_tile.setdefault((m, n), []).append(u)
    assert len(by_tile) == tm * tn
    for us in by_tile.values():
        S = us[0][6]
        rng = sorted((u[3], u[4], u[5]) for u in us)
        assert [r[0] for r in rng] == list(range(S))
        assert rng[0][1] == 0 and rng[-1][2] == kiters
        assert all(a[2] == b[1] for a, b in zip(rng, rng[1:]))
    assert smax == max(u[6] for u in units)


def test_forward_plan_split_override(mmb, tune):
    tune.set("MMB_SPLITS_FWD", "3")
    smax, units = mmb.mmb_forward_plan_units(2, 150, 264, 400, 1, True, 256)
    assert smax == 3 and all(u[6] == 3 for u in units)
    tune.set("MMB_SPLITS_FWD", "2,1,3")
    smax, units = mmb.mmb_forward_plan_units(2, 150, 264, 400, 1, True, 256)
    assert smax == 3 and {u[6] for u in units} == {1, 2, 3}


# ---------------------------------------------------------------------------
# LayerNorm backward

def largs(dtype=1, B=8, T=1024, C=1600):
    return addrs(8) + [B, T, C, dtype]


def test_layernorm_entry_points_declared():
    for f in ("mmb_layernorm_backward", "mmb_layernorm_check_args", "mmb_layernorm_path"):
        assert f in declared_functions()


def test_layernorm_check_args(mmb):
    assert mmb.mmb_layernorm_check_args(*largs()) == 0
    for idx in range(8):
        a = largs()
        a[idx] = None
        assert mmb.mmb_layernorm_check_args(*a) == -1
    for idx in (8, 9, 10):
        a = largs()
        a[idx] = 0
        assert mmb.mmb_layernorm_check_args(*a) == -2
    assert mmb.mmb_layernorm_check_args(*largs(dtype=3)) == -3
    assert mmb.mmb_layernorm_check_args(*largs(B=65536, T=32768, C=8)) == -4


def test_layernorm_alias(mmb):
    a = largs(dtype=0, B=1, T=2, C=8)          # fp32 dweight: 32 bytes
    a[2] = a[1] + 16                           # dbias inside dweight
    assert mmb.mmb_layernorm_check_args(*a) == -5
    b = largs(dtype=0, B=1, T=2, C=8)
    b[0] = b[7] + 4                            # dinp starting inside rstd
    assert mmb.mmb_layernorm_check_args(*b) == -5
    c = largs(dtype=0, B=1, T=2, C=8)
    c[6] = c[7]                                # inputs may share memory
    assert mmb.mmb_layernorm_check_args(*c) == 0


def test_layernorm_path(mmb):
    assert mmb.mmb_layernorm_path(*largs(dtype=1, C=1600)) == 1
    assert mmb.mmb_layernorm_path(*largs(dtype=1, C=2048)) == 1
    assert mmb.mmb_layernorm_path(*largs(dtype=1, C=2056)) == 1    # two waves per row
    assert mmb.mmb_layernorm_path(*largs(dtype=1, C=8192)) == 1    # four waves per row
    assert mmb.mmb_layernorm_path(*largs(dtype=1, C=8200)) == 1    # eight waves per row
    assert mmb.mmb_layernorm_path(*largs(dtype=1, C=16384)) == 1
    assert mmb.mmb_layernorm_path(*largs(dtype=1, C=16392)) == 0   # wider than the row kernel
    assert mmb.mmb_layernorm_path(*largs(dtype=0, C=1024)) == 1
    assert mmb.mmb_layernorm_path(*largs(dtype=0, C=1600)) == 1    # the page's shape, fp32
    assert mmb.mmb_layernorm_path(*largs(dtype=0, C=2048)) == 1
    assert mmb.mmb_layernorm_path(*largs(dtype=0, C=2052)) == 1    # two waves per row
    assert mmb.mmb_layernorm_path(*largs(dtype=0, C=4096)) == 1
    assert mmb.mmb_layernorm_path(*largs(dtype=0, C=4100)) == 1    # eight waves per row
    assert mmb.mmb_layernorm_path(*largs(dtype=0, C=16384)) == 1
    assert mmb.mmb_layernorm_path(*largs(dtype=0, C=16388)) == 0
    assert mmb.mmb_layernorm_path(*largs(dtype=1, C=1604)) == 0    # not a multiple of 8
    a = largs(dtype=1, C=768)
    a[3] += 8                                  # dout 8-byte aligned only
    assert mmb.mmb_layernorm_path(*a) == 0
    b = largs(dtype=1, C=768)
    b[6] += 2                                  # mean is read element by element
    assert mmb.mmb_layernorm_path(*b) == 1
