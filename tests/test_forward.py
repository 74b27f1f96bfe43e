"""GPU parity of the forward product out = inp . W^T + bias (the step before
the backward pass) through the C ABI, against the CPU oracle's forward.

Same bar as the backward pass: max|gpu - oracle| / max|oracle| <= 1e-4 for
fp32 and <= 2e-2 for bf16; with integer inputs fp32 results equal the oracle
bit for bit and bf16 results equal the oracle's exact value rounded once to
nearest-even bf16.  out is filled with NaN before each call: the forward
assigns it, so no NaN may survive.
"""
import numpy as np
import pytest

import oracle
from linear_layer_backward_amd import workloads as wl
from test_parity import TOL, assert_close, from_dev, round_bf16, sample, tile_edges, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from linear_layer_backward_amd import mmb  # noqa: F401  (fails loudly if unbuilt)
    return torch.device("cuda:0")


def make_bias(OC, seed, integer=False):
    if integer:
        return np.random.default_rng(seed).integers(-2, 3, size=OC).astype(np.float32)
    return wl.normal(seed, (OC,), 0.02, "f32")


def run_fwd(case, bias, dev, guard=0, stream=None):
    """out for a workloads.Case's inp and weight (and bias or None); returns
    [BT, OC] float64 and, with guard > 0, the guarded buffer."""
    import torch
    from linear_layer_backward_amd import mmb
    dt = case.dtype
    _, x = to_dev(case.inp, dt, dev)
    _, w = to_dev(case.weight, dt, dev)
    _, b = (None, None) if bias is None else to_dev(bias, dt, dev)
    full, out = to_dev(np.full(case.BT * case.OC, np.nan, np.float32), dt, dev, guard)
    mmb.mmb_forward_stream(out, x, w, b, case.B, case.T, case.C, case.OC,
                           mmb.MMB_BF16 if dt == "bf16" else mmb.MMB_FP32,
                           stream if stream is not None else torch.cuda.current_stream(dev))
    torch.cuda.synchronize(dev)
    got = from_dev(out, dt).reshape(case.BT, case.OC)
    return (got, full) if guard else got


def oracle_fwd(case, bias, rows=None):
    x = case.inp if rows is None else case.inp[rows]
    n = case.BT if rows is None else len(rows)
    return oracle.forward(x, case.weight, bias, B=1, T=n, C=case.C, OC=case.OC)


def check(case, bias, got, exact=False, rows=None):
    ref = oracle_fwd(case, bias, rows)
    g = got if rows is None else got[rows]
    assert not np.any(np.isnan(got)), "out not fully written"
    if exact:
        np.testing.assert_array_equal(g, round_bf16(ref) if case.dtype == "bf16" else ref)
    else:
        assert_close(g, ref, case.dtype, "out")



def assert_same_nonfinite(g, r, dt, what):
    """nan and inf at the same positions, infs of the same sign, finite
    values within tolerance."""
    np.testing.assert_array_equal(np.isnan(g), np.isnan(r), err_msg=what)
    np.testing.assert_array_equal(np.isinf(g), np.isinf(r), err_msg=what)
    inf = np.isinf(r)
    np.testing.assert_array_equal(np.sign(g[inf]), np.sign(r[inf]), err_msg=what)
    fin = np.isfinite(r)
    assert_close(g[fin], r[fin], dt, what)


@pytest.mark.parametrize("dt,C,OC", [("bf16", 264, 400), ("f32", 132, 260), ("bf16", 130, 258)])
def test_forward_nonfinite_inputs_propagate(dev, dt, C, OC):
    """nan in inp[r1, c1] makes out row r1 nan; +inf in weight[o0, c0] makes
    out column o0 +-inf (nan where inp is 0); +inf in the bias makes its
    column +inf: positions and signs as the oracle gives them."""
    case = wl.random_case(2, 40, C, OC, dt, seed=43)
    bias = make_bias(OC, 44)
    r1, c1, o0, c0, ob = 7, 11, 9, 5, 20
    case.inp[r1, c1] = np.nan
    case.weight[o0, c0] = np.inf
    case.inp[3, c0] = 0.0
    bias[ob] = np.inf
    got = run_fwd(case, bias, dev)
    ref = oracle_fwd(case, bias)
    assert_same_nonfinite(got, ref, dt, "out")
    assert np.isnan(got[r1]).all() and np.isnan(got[3, o0])

SMALL = [
    (2, 16, 64, 192, "f32"), (3, 100, 200, 328, "f32"), (1, 300, 132, 260, "f32"),
    (2, 150, 264, 400, "bf16"), (1, 513, 200, 136, "bf16"), (1, 1, 8, 8, "bf16"),
    (1, 1, 4, 4, "f32"),
    # C or OC not a multiple of the vector width: MFMA tiles on packed copies
    (2, 7, 65, 129, "f32"), (3, 5, 33, 17, "bf16"), (1, 3, 12, 10, "bf16"),
    (2, 40, 130, 258, "bf16"), (1, 70, 68, 300, "f32"),
]


@pytest.mark.parametrize("bias", [True, False])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_forward_small_random(dev, shape, bias):
    B, T, C, OC, dt = shape
    case = wl.random_case(B, T, C, OC, dt, seed=C + OC)
    b = make_bias(OC, 7) if bias else None
    if b is not None:
        b = wl.from_storage(wl.storage(b, dt), dt)
    check(case, b, run_fwd(case, b, dev))


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_forward_small_integer_exact(dev, shape):
    B, T, C, OC, dt = shape
    case = wl.integer_case(B, T, C, OC, dt, seed=3 + C)
    b = make_bias(OC, 11, integer=True)
    check(case, b, run_fwd(case, b, dev), exact=True)


@pytest.mark.parametrize("splits", ["2", "3", "5", "2,1,3", "4,2"])
@pytest.mark.parametrize("shape", [(3, 100, 200, 328, "f32"), (2, 150, 264, 400, "bf16"),
                                   (1, 300, 520, 264, "bf16")], ids=lambda s: "x".join(map(str, s)))
def test_forward_forced_splits(dev, tune, shape, splits):
    """Split-K forward tiles: partials summed by the last arriver, then the
    bias epilogue; exact with integer inputs."""
    tune.set("MMB_SPLITS_FWD", splits)
    B, T, C, OC, dt = shape
    case = wl.integer_case(B, T, C, OC, dt, seed=17)
    b = make_bias(OC, 5, integer=True)
    check(case, b, run_fwd(case, b, dev), exact=True)
    check(case, None, run_fwd(case, None, dev), exact=True)


@pytest.mark.parametrize("shape", [(2, 150, 264, 400, "bf16"), (3, 100, 200, 328, "f32"),
                                   (3, 5, 33, 17, "bf16")], ids=lambda s: "x".join(map(str, s)))
def test_forward_guard_bands(dev, shape):
    """Nothing outside out is written (canaries on both sides)."""
    B, T, C, OC, dt = shape
    case = wl.random_case(B, T, C, OC, dt, seed=2)
    g = 4096
    got, full = run_fwd(case, None, dev, guard=g)
    check(case, None, got)
    host = from_dev(full, dt)
    assert np.all(host[:g] == 12288.0) and np.all(host[-g:] == 12288.0)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_forward_ragged_split_k_with_bias(dev, tune, dt):
    """Ragged C and OC with split K: the last arriver adds the packed bias
    (its final group straddles OC) to the summed partials."""
    tune.set("MMB_SPLITS_FWD", "3")
    case = wl.integer_case(2, 150, 263, 397, dt, seed=5)
    b = make_bias(397, 6, integer=True)
    check(case, b, run_fwd(case, b, dev), exact=True)
    case = wl.random_case(1, 300, 130, 258, dt, seed=7)
    b = wl.from_storage(wl.storage(make_bias(258, 8), dt), dt)
    check(case, b, run_fwd(case, b, dev))


def test_forward_deterministic(dev, tune):
    tune.set("MMB_SPLITS_FWD", "3")
    case = wl.random_case(2, 150, 264, 400, "bf16", seed=4)
    b = make_bias(400, 3)
    a = run_fwd(case, b, dev)
    c = run_fwd(case, b, dev)
    assert a.tobytes() == c.tobytes()


FULL = [  # (B, T, C, OC, dtype, bias): GPT-2 124M layer shapes
    (16, 1024, 768, 3072, "bf16", True),    # MLP fc
    (16, 1024, 3072, 768, "bf16", True),    # MLP fc_proj (few tiles: split K)
    (8, 1024, 768, 50304, "bf16", False),   # LM head
    (8, 1024, 768, 2304, "f32", True),      # qkv
    (8, 1024, 3072, 768, "f32", True),      # fc_proj
]


@pytest.mark.parametrize("shape", FULL, ids=lambda s: "x".join(map(str, s[:5])))
def test_forward_full_shapes_sampled(dev, shape):
    """Full layer shapes, inputs drawn like the backward workloads
    (inp N(0,1), weight N(0,0.02), bias N(0,0.02)); sampled rows (tile
    edges and random ones) against the oracle row by row."""
    B, T, C, OC, dt, bias = shape
    BT = B * T
    inp = wl.normal(500 + C, (BT, C), 1.0, dt)
    weight = wl.normal(501 + OC, (OC, C), 0.02, dt)
    b = wl.normal(502, (OC,), 0.02, dt) if bias else None
    case = wl.Case(name=f"forward {B}x{T}x{C}x{OC} {dt}", B=B, T=T, C=C, OC=OC, dtype=dt,
                   inp=inp, weight=weight, dout=None, dinp0=None, dweight0=None,
                   dbias0=None)
    print(f"[parity] {case.name}", flush=True)
    got = run_fwd(case, b, dev)
    rows = sample(BT, tile_edges(BT, 256), 48, seed=OC)
    check(case, b, got, rows=rows)


@pytest.mark.parametrize("shape", [(16, 1024, 768, 3072, "bf16"), (8, 1024, 3072, 768, "f32"),
                                   (8, 1024, 768, 50304, "bf16")], ids=["fc", "fc_proj", "lm_head"])
def test_forward_full_shapes_integer_exact(dev, shape):
    B, T, C, OC, dt = shape
    case = wl.integer_case(B, T, C, OC, dt, seed=C, prefill=False)
    b = make_bias(OC, 9, integer=True)
    print(f"[parity] forward integer {case.name}", flush=True)
    got = run_fwd(case, b, dev)
    rows = sample(case.BT, tile_edges(case.BT, 256), 32, seed=1)
    check(case, b, got, exact=True, rows=rows)


def test_forward_backward_adjoint(dev):
    """The backward pass is the adjoint of the forward product: with integer
    inputs (fp32, every sum exact) sum(dout * inp.W^T) == sum(inp * ddinp)
    == sum(W * ddweight), each side computed by the GPU."""
    import torch
    from linear_layer_backward_amd import mmb
    B, T, C, OC = 2, 300, 264, 392
    case = wl.integer_case(B, T, C, OC, "f32", seed=77, prefill=False)
    out = run_fwd(case, None, dev)
    _, dout = to_dev(case.dout, "f32", dev)
    _, x = to_dev(case.inp, "f32", dev)
    _, w = to_dev(case.weight, "f32", dev)
    gi = torch.zeros(case.BT * C, device=dev)
    gw = torch.zeros(OC * C, device=dev)
    mmb.mmb_backward_stream(gi, gw, None, dout, x, w, B, T, C, OC, mmb.MMB_FP32,
                            torch.cuda.current_stream(dev))
    torch.cuda.synchronize(dev)
    lhs = int(np.sum(case.dout.astype(np.int64) * out.astype(np.int64)))
    assert lhs == int(np.sum(case.inp.astype(np.int64).ravel() * gi.cpu().numpy().astype(np.int64)))
    assert lhs == int(np.sum(case.weight.astype(np.int64).ravel() *
                             gw.cpu().numpy().astype(np.int64)))


def test_forward_tensor_binding(dev):
    import torch
    from linear_layer_backward_amd import mmb
    B, T, C, OC = 2, 64, 128, 256
    case = wl.random_case(B, T, C, OC, "bf16", seed=6)
    x = torch.from_numpy(case.inp.reshape(B, T, C)).to(dev).to(torch.bfloat16)
    w = torch.from_numpy(case.weight).to(dev).to(torch.bfloat16)
    b = torch.linspace(-1, 1, OC, device=dev).to(torch.bfloat16)
    out = torch.full((B, T, OC), float("nan"), device=dev, dtype=torch.bfloat16)
    mmb.forward(out, x, w, b)
    torch.cuda.synchronize(dev)
    ref = oracle.forward(x.float().cpu().numpy().reshape(B * T, C), w.float().cpu().numpy(),
                         b.float().cpu().numpy(), B=B, T=T, C=C, OC=OC)
    assert_close(out.float().cpu().numpy().reshape(B * T, OC).astype(np.float64), ref, "bf16",
                 "out")
    with pytest.raises(ValueError):
        mmb.forward(out, x, w.float(), b)


def test_forward_and_backward_share_the_workspace(dev, tune):
    """Split forward and split backward calls alternate on one stream: the
    shared tile counters and partial buffers stay consistent."""
    from test_parity import check_exact, run
    for n in range(3):
        tune.set("MMB_SPLITS_FWD", str(2 + n))
        tune.set("MMB_SPLITS_DWEIGHT", str(3 + n))
        case = wl.integer_case(2, 150, 264, 400, "bf16", seed=90 + n)
        b = make_bias(400, n, integer=True)
        check(case, b, run_fwd(case, b, dev), exact=True)
        check_exact(case, run(case, dev))
    assert TOL["f32"] == 1e-4


def test_forward_unaligned_pointers_take_packed_tiles(dev):
    """Shapes the tiles accept, but out, inp and the bias start some elements
    past a 16-byte boundary: packed copies on the MFMA tiles, out copied back."""
    import torch
    from linear_layer_backward_amd import mmb
    B, T, C, OC = 2, 40, 64, 96
    case = wl.random_case(B, T, C, OC, "bf16", seed=31)
    bias = wl.normal(32, (OC,), 0.02, "bf16")
    _, xs = to_dev(np.concatenate([[0.0], case.inp.ravel()]), "bf16", dev)
    _, w = to_dev(case.weight, "bf16", dev)
    _, bs = to_dev(np.concatenate([[0.0] * 3, bias]), "bf16", dev)
    _, outs = to_dev(np.full(B * T * OC + 1, np.nan, np.float32), "bf16", dev)
    x, out, b = xs[1:], outs[1:], bs[3:]
    assert mmb.mmb_forward_path(out, x, w, b, B, T, C, OC, mmb.MMB_BF16) == 1
    mmb.mmb_forward_stream(out, x, w, b, B, T, C, OC, mmb.MMB_BF16, torch.cuda.current_stream(dev))
    torch.cuda.synchronize(dev)
    got = from_dev(out, "bf16").reshape(B * T, OC)
    check(case, bias, got)
    assert np.isnan(from_dev(outs[:1], "bf16")).all()   # nothing written before out


def test_forward_generic_path_beyond_tile_offsets(dev):
    """OC above 2^22: the generic forward kernel (B*T = 2, C = 8)."""
    from linear_layer_backward_amd import mmb
    for dt in ("bf16", "f32"):
        case = wl.random_case(1, 2, 8, (1 << 22) + 40, dt, seed=33)
        bias = wl.from_storage(wl.storage(make_bias(case.OC, 34), dt), dt)
        _, x = to_dev(case.inp, dt, dev)
        _, w = to_dev(case.weight, dt, dev)
        _, b = to_dev(bias, dt, dev)
        _, out = to_dev(np.full(case.BT * case.OC, np.nan, np.float32), dt, dev)
        code = mmb.MMB_BF16 if dt == "bf16" else mmb.MMB_FP32
        assert mmb.mmb_forward_path(out, x, w, b, case.B, case.T, case.C, case.OC, code) == 0
        check(case, bias, run_fwd(case, bias, dev))


def test_forward_unpadded_vocabulary(dev):
    """The GPT-2 LM-head forward at the real vocabulary (OC = 50257): out and
    the bias on packed copies; sampled rows exact with integer inputs."""
    case = wl.integer_case(8, 1024, 768, 50257, "bf16", seed=35, with_bias=False, prefill=False)
    bias = make_bias(case.OC, 36, integer=True)
    print(f"[forward] {case.name}", flush=True)
    got = run_fwd(case, bias, dev)
    rows = sample(case.BT, tile_edges(case.BT, 256), 16, 37)
    check(case, bias, got, rows=rows, exact=True)