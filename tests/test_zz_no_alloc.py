"""The allocation-free entry point (mmb_backward_noalloc) against the
allocating one (mmb_backward_stream), through the C ABI.

Both take the same plan and kernels, so their outputs must be bit-identical;
the smaller cases are also checked against the CPU oracle (max |g - r| /
max |r| <= 1e-4 fp32, 2e-2 bf16).  Calls come in pairs, the second on a
smaller input than the first, so that the fixed scratch (tile counters, work
list, split partials) is reused with different contents: the counters must
be cleared and the work list replaced on every call.
"""
import numpy as np
import pytest

import oracle
from linear_layer_backward_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from linear_layer_backward_amd import mmb  # noqa: F401  (fails loudly if unbuilt)
    return torch.device("cuda:0")


def up(x, dtype, dev):
    import torch
    raw = wl.storage(np.asarray(x, np.float32).ravel(), dtype)
    if dtype == "bf16":
        return torch.from_numpy(raw.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    return torch.from_numpy(raw.copy()).to(dev)


def down(t, dtype):
    import torch
    if dtype == "bf16":
        return wl.from_storage(t.view(torch.int16).cpu().numpy().view(np.uint16), dtype)
    return wl.from_storage(t.cpu().numpy(), dtype)


def both(case, dev):
    """Run the case through mmb_backward_stream and mmb_backward_noalloc on
    separate, identically prefilled outputs; return both results (raw bits)."""
    import torch
    from linear_layer_backward_amd import mmb
    dt = case.dtype
    code = mmb.MMB_BF16 if dt == "bf16" else mmb.MMB_FP32
    dout, inp, w = (up(a, dt, dev) for a in (case.dout, case.inp, case.weight))
    s = torch.cuda.current_stream(dev)
    outs = []
    for fn in (mmb.mmb_backward_stream, mmb.mmb_backward_noalloc):
        gi, gw = up(case.dinp0, dt, dev), up(case.dweight0, dt, dev)
        gb = up(np.full(case.OC, np.nan, np.float32), dt, dev) if case.with_bias else None
        print(f"[noalloc] {fn.__name__} {dt} B={case.B} T={case.T} C={case.C} OC={case.OC}",
              flush=True)
        fn(gi, gw, gb, dout, inp, w, case.B, case.T, case.C, case.OC, code, s)
        torch.cuda.synchronize(dev)
        outs.append((down(gi, dt), down(gw, dt), None if gb is None else down(gb, dt)))
    return outs


def check(case, dev, with_oracle):
    ref, got = both(case, dev)
    for name, a, b in zip(("dinp", "dweight", "dbias"), ref, got):
        if a is None:
            continue
        np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                      b.view(np.uint32) if b.dtype == np.float32 else b,
                                      err_msg=name)
    if with_oracle:
        ri, rw, rb = oracle.case_backward(case)
        for name, g, r in (("dinp", got[0], ri), ("dweight", got[1], rw), ("dbias", got[2], rb)):
            if r is None:
                continue
            g = np.asarray(g, np.float64).reshape(r.shape)
            err = np.max(np.abs(g - r)) / np.max(np.abs(r))
            assert err <= TOL[case.dtype], f"{name}: {err:.3e}"


# pairs (larger, then smaller); the fp32 pair's first plan has 732 units, so
# its work list takes several argument-passing launches
PAIRS = [
    ((4, 512, 768, 1024, "bf16"), (2, 150, 264, 400, "bf16")),
    ((2, 512, 768, 2304, "f32"), (1, 300, 132, 260, "f32")),
    ((16, 1024, 768, 3072, "bf16"), (1, 513, 200, 136, "bf16")),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: "_then_".join(
    "x".join(map(str, s)) for s in p))
def test_noalloc_matches_the_allocating_call(dev, pair):
    for i, (B, T, C, OC, dt) in enumerate(pair):
        case = wl.random_case(B, T, C, OC, dt, seed=40 + i,
                              with_bias=(i == 0 or dt == "f32"))
        check(case, dev, with_oracle=B * T * C * OC <= 1 << 27)


def test_noalloc_with_split_partials(dev, tune):
    """Forced split counts put partial tiles and dbias partials in the scratch."""
    tune.set("MMB_SPLITS_DWEIGHT", "3")
    tune.set("MMB_SPLITS_DINP", "2")
    check(wl.random_case(2, 300, 520, 600, "bf16", seed=44), dev, with_oracle=True)
    tune.set("MMB_SPLITS_DWEIGHT", "2,5")
    check(wl.random_case(1, 200, 264, 136, "bf16", seed=45), dev, with_oracle=True)


def test_noalloc_ragged_rows(dev):
    """C or OC not a multiple of the 16-byte vector: the packed copies live in
    the scratch too (larger shape first, then a smaller one)."""
    check(wl.random_case(2, 64, 770, 1027, "bf16", seed=46), dev, with_oracle=True)
    check(wl.random_case(3, 5, 33, 17, "bf16", seed=47), dev, with_oracle=True)
    check(wl.random_case(3, 100, 202, 330, "f32", seed=48), dev, with_oracle=True)


def test_noalloc_unaligned_input(dev):
    """An input 8 bytes off the 16-byte alignment: a packed copy in the
    scratch; same result as the allocating call."""
    import torch
    from linear_layer_backward_amd import mmb
    case = wl.random_case(2, 20, 64, 96, "bf16", seed=49)
    outs = []
    for fn in (mmb.mmb_backward_stream, mmb.mmb_backward_noalloc):
        raw = torch.empty(case.BT * case.C + 8, dtype=torch.bfloat16, device=dev)
        inp = raw[4:4 + case.BT * case.C]
        inp.copy_(up(case.inp, "bf16", dev))
        gi, gw = up(case.dinp0, "bf16", dev), up(case.dweight0, "bf16", dev)
        gb = up(np.zeros(case.OC, np.float32), "bf16", dev)
        assert mmb.mmb_path(gi, gw, gb, up(case.dout, "bf16", dev), inp,
                            up(case.weight, "bf16", dev), case.B, case.T, case.C, case.OC,
                            mmb.MMB_BF16) == 1
        fn(gi, gw, gb, up(case.dout, "bf16", dev), inp, up(case.weight, "bf16", dev), case.B,
           case.T, case.C, case.OC, mmb.MMB_BF16, torch.cuda.current_stream(dev))
        torch.cuda.synchronize(dev)
        outs.append([down(t, "bf16") for t in (gi, gw, gb)])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def test_noalloc_generic_path(dev):
    """C above 2^22: the generic kernels, which use no scratch; same result
    as the allocating call."""
    check(wl.random_case(1, 1, (1 << 22) + 16, 8, "bf16", seed=50), dev, with_oracle=False)


@pytest.mark.parametrize("shape", [(2, 300, 520, 600, "bf16"), (1, 200, 130, 261, "bf16"),
                                   (2, 100, 200, 328, "f32")],
                         ids=["split_partials", "ragged_packed", "f32"])
def test_noalloc_graph_replays(dev, tune, shape):
    """A HIP graph captured around one mmb_backward_noalloc call (the call
    makes no allocation and no host-to-device copy, so it can be captured):
    every replay, with eager work and synchronisations between replays and
    the outputs reset to the prefill, gives the eager call's bits."""
    import torch
    from linear_layer_backward_amd import mmb
    if shape[0] == 2 and shape[4] == "bf16":
        tune.set("MMB_SPLITS_DWEIGHT", "3")
        tune.set("MMB_SPLITS_DINP", "2")
    B, T, C, OC, dt = shape
    case = wl.random_case(B, T, C, OC, dt, seed=51)
    code = mmb.MMB_BF16 if dt == "bf16" else mmb.MMB_FP32
    dout, inp, w = (up(a, dt, dev) for a in (case.dout, case.inp, case.weight))
    gi0, gw0 = up(case.dinp0, dt, dev), up(case.dweight0, dt, dev)
    gi, gw = gi0.clone(), gw0.clone()
    gb = up(np.zeros(case.OC, np.float32), dt, dev)
    args = (gi, gw, gb, dout, inp, w, B, T, C, OC, code)
    # eager reference (also plans the shape and looks up the scratch address)
    mmb.mmb_backward_noalloc(*args, torch.cuda.current_stream(dev))
    torch.cuda.synchronize(dev)
    ref = [down(t, dt) for t in (gi, gw, gb)]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mmb.mmb_backward_noalloc(*args, s)
    torch.cuda.synchronize(dev)
    for rep in range(3):
        gi.copy_(gi0)
        gw.copy_(gw0)
        gb.fill_(float("nan"))
        x = dout.float().sum()   # eager work between replays
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        assert torch.isfinite(x)
        for name, a, b in zip(("dinp", "dweight", "dbias"), ref, (gi, gw, gb)):
            np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                          down(b, dt).view(np.uint32) if a.dtype == np.float32
                                          else down(b, dt), err_msg=f"replay {rep}: {name}")


def test_noalloc_rejects_plans_larger_than_the_scratch(dev, tune):
    """16 dweight splits of the GPT-2 fc shape need 144 MiB of partials: the
    call returns MMB_ERR_SCRATCH and enqueues nothing (the outputs keep their
    contents)."""
    import torch
    from linear_layer_backward_amd import mmb
    tune.set("MMB_SPLITS_DWEIGHT", "16")
    B, T, C, OC = 16, 1024, 768, 3072
    bf = torch.bfloat16
    dout = torch.zeros(B * T * OC, dtype=bf, device=dev)
    inp = torch.zeros(B * T * C, dtype=bf, device=dev)
    w = torch.zeros(OC * C, dtype=bf, device=dev)
    gi = torch.full((B * T * C,), 3.0, dtype=bf, device=dev)
    gw = torch.full((OC * C,), 3.0, dtype=bf, device=dev)
    gb = torch.full((OC,), 3.0, dtype=bf, device=dev)
    st = mmb._lib.mmb_backward_noalloc(gi.data_ptr(), gw.data_ptr(), gb.data_ptr(),
                                       dout.data_ptr(), inp.data_ptr(), w.data_ptr(),
                                       B, T, C, OC, mmb.MMB_BF16, None)
    assert st == -9 and "scratch" in mmb.mmb_strerror(st)
    torch.cuda.synchronize(dev)
    for t in (gi, gw, gb):
        assert bool((t == 3.0).all())
