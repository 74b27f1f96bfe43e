"""GPU parity over seeded random calls: shapes (ragged and aligned, one to
several tiles), element offsets of every buffer (direct tiles, packed
copies), dtypes, forced split counts and the three entry points (backward,
allocation-free backward, forward), each against the CPU oracle.

Integer inputs in [-2, 2], so every sum is exact in any order: fp32 results
must equal the oracle bit for bit, bf16 results its exact value rounded once
to nearest-even.  Each call's outputs sit between canaries that must survive.
"""
import os

import numpy as np
import pytest

import oracle
from linear_layer_backward_amd import workloads as wl
from test_parity import from_dev, round_bf16

pytestmark = pytest.mark.gpu

# more calls for a longer sweep: MMB_RANDOM_CALLS=1000 python -m pytest ...
CASES = int(os.environ.get("MMB_RANDOM_CALLS", "120"))
CANARY = 12288.0


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from linear_layer_backward_amd import mmb  # noqa: F401  (fails loudly if unbuilt)
    return torch.device("cuda:0")


def draw_call(i):
    """The i-th random call: (entry, dtype, B, T, C, OC, bias, offsets, splits)."""
    g = np.random.default_rng(9000 + i)
    entry = ["backward", "noalloc", "forward"][i % 3]
    dt = ["bf16", "f32"][(i // 3) % 2]
    B = int(g.integers(1, 4))
    T = int(g.integers(1, 400))
    C = int(g.choice([int(g.integers(1, 600)), 8 * int(g.integers(1, 80))]))
    OC = int(g.choice([int(g.integers(1, 700)), 8 * int(g.integers(1, 90))]))
    bias = bool(g.integers(0, 2))
    # element offsets of the buffers past a 256-byte boundary (0 = aligned)
    offs = [int(g.choice([0, 0, 1, 2, 3, 5])) for _ in range(6)]
    splits = (None if g.integers(0, 2) == 0 else
              (str(int(g.integers(1, 6))), str(int(g.integers(1, 4)))))
    return entry, dt, B, T, C, OC, bias, offs, splits


def place(x, dt, dev, off, guard=64):
    """x in a fresh buffer, `off` elements past its start plus `guard`
    canaries on each side; returns (full buffer, view of x)."""
    import torch
    x = np.asarray(x, np.float32).ravel()
    full = np.full(x.size + 2 * guard + off, CANARY, np.float32)
    full[guard + off:guard + off + x.size] = x
    raw = wl.storage(full, dt)
    if dt == "bf16":
        t = torch.from_numpy(raw.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    else:
        t = torch.from_numpy(raw.copy()).to(dev)
    return t, t[guard + off:guard + off + x.size]


def canaries_intact(full, view_len, off, dt, guard=64):
    h = from_dev(full, dt)
    return np.all(h[:guard + off] == CANARY) and np.all(h[guard + off + view_len:] == CANARY)


@pytest.mark.parametrize("i", range(CASES))
def test_random_call(dev, tune, i):
    import torch
    from linear_layer_backward_amd import mmb
    entry, dt, B, T, C, OC, bias, offs, splits = draw_call(i)
    print(f"[random] {i}: {entry} {dt} B={B} T={T} C={C} OC={OC} bias={bias} offsets={offs} "
          f"splits={splits}", flush=True)
    code = mmb.MMB_BF16 if dt == "bf16" else mmb.MMB_FP32
    s = torch.cuda.current_stream(dev)
    if entry == "forward":
        if splits:
            tune.set("MMB_SPLITS_FWD", splits[0])
        case = wl.integer_case(B, T, C, OC, dt, seed=i, with_bias=False, prefill=False)
        b = np.random.default_rng(i).integers(-2, 3, size=OC).astype(np.float32) if bias else None
        _, x = place(case.inp, dt, dev, offs[0])
        _, w = place(case.weight, dt, dev, offs[1])
        bt = place(b, dt, dev, offs[2])[1] if bias else None
        out_full, out = place(np.full(case.BT * OC, np.nan, np.float32), dt, dev, offs[3])
        assert mmb.mmb_forward_path(out, x, w, bt, B, T, C, OC, code) == 1
        mmb.mmb_forward_stream(out, x, w, bt, B, T, C, OC, code, s)
        torch.cuda.synchronize(dev)
        ref = oracle.forward(case.inp, case.weight, b, B=B, T=T, C=C, OC=OC)
        got = from_dev(out, dt).reshape(case.BT, OC)
        np.testing.assert_array_equal(got, round_bf16(ref) if dt == "bf16" else ref)
        assert canaries_intact(out_full, case.BT * OC, offs[3], dt)
        return
    if splits:
        tune.set("MMB_SPLITS_DWEIGHT", splits[0])
        tune.set("MMB_SPLITS_DINP", splits[1])
    case = wl.integer_case(B, T, C, OC, dt, seed=i, with_bias=bias, prefill=True)
    _, dout = place(case.dout, dt, dev, offs[0])
    _, inp = place(case.inp, dt, dev, offs[1])
    _, w = place(case.weight, dt, dev, offs[2])
    gi_full, gi = place(case.dinp0, dt, dev, offs[3])
    gw_full, gw = place(case.dweight0, dt, dev, offs[4])
    gb_full, gb = place(np.full(OC, np.nan, np.float32), dt, dev, offs[5]) if bias else (None, None)
    args = (gi, gw, gb, dout, inp, w, B, T, C, OC, code)
    assert mmb.mmb_path(*args) == 1
    fn = mmb.mmb_backward_noalloc if entry == "noalloc" else mmb.mmb_backward_stream
    fn(*args, s)
    torch.cuda.synchronize(dev)
    ri, rw, rb = oracle.case_backward(case)
    fix = round_bf16 if dt == "bf16" else (lambda v: v)
    np.testing.assert_array_equal(from_dev(gi, dt).reshape(case.BT, C), fix(ri))
    np.testing.assert_array_equal(from_dev(gw, dt).reshape(OC, C), fix(rw))
    assert canaries_intact(gi_full, case.BT * C, offs[3], dt)
    assert canaries_intact(gw_full, OC * C, offs[4], dt)
    if bias:
        np.testing.assert_array_equal(from_dev(gb, dt), fix(rb))
        assert canaries_intact(gb_full, OC, offs[5], dt)
