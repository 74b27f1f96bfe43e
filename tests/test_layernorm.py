"""GPU parity of the LayerNorm backward (mmb_layernorm_backward, the op next
to the linear layer in a GPT-2 block) through the C ABI against the CPU
oracle: max|gpu - oracle| / max|oracle| per output <= 1e-4 (fp32) and
<= 2e-2 (bf16), the same rule as the linear layer."""
import numpy as np
import pytest

import oracle
from linear_layer_backward_amd import workloads as wl
from test_parity import assert_close, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from linear_layer_backward_amd import mmb  # noqa: F401  (fails loudly if unbuilt)
    return torch.device("cuda:0")


def run_ln(c, dev, guard=0):
    import torch
    from linear_layer_backward_amd import mmb
    dt = c.dtype
    ins = [to_dev(a, dt, dev)[1] for a in (c.dout, c.inp, c.weight, c.mean, c.rstd)]
    outs = [to_dev(a, dt, dev, guard) for a in (c.dinp0, c.dweight0, c.dbias0)]
    views = [o[1] for o in outs]
    mmb.mmb_layernorm_backward(*views, *ins, c.B, c.T, c.C,
                               mmb.MMB_BF16 if dt == "bf16" else mmb.MMB_FP32,
                               torch.cuda.current_stream(dev))
    torch.cuda.synchronize(dev)
    got = (from_dev(views[0], dt).reshape(c.BT, c.C), from_dev(views[1], dt), from_dev(views[2], dt))
    if guard:
        return got, [from_dev(o[0], dt) for o in outs]
    return got


def check(c, got):
    ref = oracle.layernorm_backward(c.dout, c.inp, c.weight, c.mean, c.rstd, c.dinp0, c.dweight0,
                                    c.dbias0, B=c.B, T=c.T, C=c.C)
    for name, g, r in zip(("dinp", "dweight", "dbias"), got, ref):
        assert_close(g, r, c.dtype, name)


SHAPES = [  # (B, T, C, dtype): row kernel with 1, 2, 4 (and fp32 8) vectors per lane
    (2, 37, 1600, "bf16"), (1, 300, 768, "bf16"), (3, 20, 256, "bf16"), (1, 5, 2048, "bf16"),
    (2, 33, 1000, "bf16"), (2, 50, 768, "f32"), (1, 70, 1024, "f32"), (3, 9, 100, "f32"),
    (2, 13, 1600, "f32"), (1, 40, 2048, "f32"), (3, 17, 1028, "f32"),
    # wide rows, 2 or 4 waves per row (row counts not a multiple of the rows
    # a workgroup takes per step, so the last step has groups past the end)
    (1, 9, 2056, "bf16"), (2, 21, 3000, "bf16"), (1, 37, 4096, "bf16"), (3, 7, 5000, "bf16"),
    (1, 13, 8192, "bf16"), (1, 6, 2052, "f32"), (2, 19, 3000, "f32"), (1, 11, 4096, "f32"),
    # eight waves per row, one row per workgroup step (parts past C idle)
    (1, 5, 8200, "bf16"), (2, 3, 12288, "bf16"), (1, 4, 16384, "bf16"), (1, 4, 4100, "f32"),
    (3, 3, 8192, "f32"), (1, 5, 12300, "f32"), (1, 3, 16384, "f32"),
    # generic kernels: C not a multiple of the vector width, or wider than the row kernel
    (2, 11, 1603, "bf16"), (1, 3, 16392, "bf16"), (1, 2, 16388, "f32"), (1, 4, 7, "f32"),
    # degenerate: one row (one busy wave), one channel
    (1, 1, 768, "bf16"), (1, 1, 8, "f32"), (3, 1, 1, "f32"), (1, 2, 1, "bf16"),
]


@pytest.mark.parametrize("prefill", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_layernorm_small(dev, shape, prefill):
    B, T, C, dt = shape
    c = wl.layernorm_case(B, T, C, dt, seed=C + T, prefill=prefill)
    check(c, run_ln(c, dev))


@pytest.mark.parametrize("shape", [(8, 1024, 4096, "bf16"), (4, 1024, 8192, "bf16"),
                                   (8, 1024, 4096, "f32"), (2, 1024, 12288, "bf16"),
                                   (2, 1024, 8192, "f32")], ids=lambda s: "x".join(map(str, s)))
def test_layernorm_wide_rows(dev, shape):
    """Rows of 4096 to 12288 channels (several waves per row) at full row
    counts, against the oracle."""
    from linear_layer_backward_amd import mmb
    B, T, C, dt = shape
    c = wl.layernorm_case(B, T, C, dt, seed=C, prefill=True)
    code = mmb.MMB_BF16 if dt == "bf16" else mmb.MMB_FP32
    fake = [256 * (i + 1) << 20 for i in range(8)]
    assert mmb.mmb_layernorm_path(*fake, B, T, C, code) == 1
    print(f"[layernorm] wide B={B} T={T} C={C} {dt}", flush=True)
    check(c, run_ln(c, dev))


@pytest.mark.parametrize("shape", [(4, 777, 1603, "bf16"), (2, 1000, 770, "f32"),
                                   (1, 600, 16392, "bf16")], ids=lambda s: "x".join(map(str, s)))
def test_layernorm_generic_bands(dev, shape):
    """The generic kernels with many rows: dweight/dbias summed over bands of
    rows (several rows per band, the last band shorter), then reduced."""
    from linear_layer_backward_amd import mmb
    B, T, C, dt = shape
    c = wl.layernorm_case(B, T, C, dt, seed=C + 1, prefill=True)
    code = mmb.MMB_BF16 if dt == "bf16" else mmb.MMB_FP32
    fake = [256 * (i + 1) << 20 for i in range(8)]
    assert mmb.mmb_layernorm_path(*fake, B, T, C, code) == 0
    print(f"[layernorm] generic B={B} T={T} C={C} {dt}", flush=True)
    a = run_ln(c, dev)
    check(c, a)
    b = run_ln(c, dev)
    for x, y in zip(a, b):
        assert x.tobytes() == y.tobytes()


@pytest.mark.parametrize("dt,C", [("bf16", 1600), ("f32", 1600), ("bf16", 4096), ("bf16", 1603)])
def test_layernorm_nonfinite_inputs_propagate(dev, dt, C):
    """nan in inp[r, i] makes dinp row r nan (both row means see it) and
    dweight[i] nan; +inf in dout[r2, j] makes dinp row r2 nan or inf,
    dweight[j] and dbias[j] inf: positions and signs as the oracle gives
    them (row kernel, several waves per row, generic kernels)."""
    c = wl.layernorm_case(2, 37, C, dt, seed=C + 5, prefill=True)
    r, i, r2, j = 4, 10, 20, 33
    c.inp[r, i] = np.nan
    c.dout[r2, j] = np.inf
    got = run_ln(c, dev)
    ref = oracle.layernorm_backward(c.dout, c.inp, c.weight, c.mean, c.rstd, c.dinp0, c.dweight0,
                                    c.dbias0, B=c.B, T=c.T, C=c.C)
    for name, g, rr in zip(("dinp", "dweight", "dbias"), got, ref):
        np.testing.assert_array_equal(np.isnan(g), np.isnan(rr), err_msg=name)
        np.testing.assert_array_equal(np.isinf(g), np.isinf(rr), err_msg=name)
        inf = np.isinf(rr)
        np.testing.assert_array_equal(np.sign(g[inf]), np.sign(rr[inf]), err_msg=name)
        fin = np.isfinite(rr)
        assert_close(g[fin], rr[fin], dt, name)
    assert np.isnan(got[0][r]).all() and np.isnan(got[1][i])


LN_RANDOM = 60


@pytest.mark.parametrize("i", range(LN_RANDOM))
def test_layernorm_random_call(dev, i):
    """Seeded random calls: row counts, widths from a few channels to past
    the row kernel's limit (every layout: one to eight waves per row, ragged
    and generic), both dtypes, prefilled or zero outputs."""
    g = np.random.default_rng(7000 + i)
    dt = ["bf16", "f32"][i % 2]
    vec = 8 if dt == "bf16" else 4
    kind = i % 3
    if kind == 0:
        C = int(g.integers(1, 2200))                       # often ragged
    elif kind == 1:
        C = vec * int(g.integers(1, 2100))                 # row kernel, up to 16800
    else:
        C = vec * int(g.integers(256, 2100)) + int(g.integers(0, 2))
    B, T = int(g.integers(1, 4)), int(g.integers(1, 120))
    c = wl.layernorm_case(B, T, C, dt, seed=i, prefill=bool(i % 4 < 2))
    print(f"[layernorm] random {i}: B={B} T={T} C={C} {dt}", flush=True)
    check(c, run_ln(c, dev))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_layernorm_page_shape(dev, dt):
    """The page's benchmark shape B=8, T=1024, C=1600 (fp32 takes the row
    kernel with 8 vectors per lane and one row in flight per wave)."""
    c = wl.layernorm_case(8, 1024, 1600, dt, seed=1)
    print(f"[parity] {c.name}", flush=True)
    check(c, run_ln(c, dev))


def test_layernorm_gpt2_shape(dev):
    c = wl.layernorm_case(16, 1024, 768, "bf16", seed=2, prefill=True)
    print(f"[parity] {c.name}", flush=True)
    check(c, run_ln(c, dev))


def test_layernorm_guard_bands(dev):
    c = wl.layernorm_case(2, 37, 1600, "bf16", seed=5)
    got, full = run_ln(c, dev, guard=4096)
    check(c, got)
    for f in full:
        assert np.all(f[:4096] == 12288.0) and np.all(f[-4096:] == 12288.0)


def test_layernorm_deterministic(dev):
    c = wl.layernorm_case(4, 256, 1600, "bf16", seed=6)
    a = run_ln(c, dev)
    b = run_ln(c, dev)
    for x, y in zip(a, b):
        assert x.tobytes() == y.tobytes()


def test_layernorm_unaligned_pointers_take_generic_path(dev):
    """C fits the row kernel, but dinp and dout start 2 bytes into their
    buffers: the call takes the generic kernels and still matches."""
    import torch
    from linear_layer_backward_amd import mmb
    c = wl.layernorm_case(2, 30, 768, "bf16", seed=8, prefill=True)
    _, gis = to_dev(np.concatenate([[0.0], c.dinp0.ravel()]), "bf16", dev)
    _, ds = to_dev(np.concatenate([[0.0], c.dout.ravel()]), "bf16", dev)
    gi, d = gis[1:], ds[1:]
    ins = [to_dev(a, "bf16", dev)[1] for a in (c.inp, c.weight, c.mean, c.rstd)]
    gw, gb = to_dev(c.dweight0, "bf16", dev)[1], to_dev(c.dbias0, "bf16", dev)[1]
    args = (gi, gw, gb, d, *ins, c.B, c.T, c.C, mmb.MMB_BF16)
    assert mmb.mmb_layernorm_path(*args) == 0
    mmb.mmb_layernorm_backward(*args, torch.cuda.current_stream(dev))
    torch.cuda.synchronize(dev)
    check(c, (from_dev(gi, "bf16").reshape(c.BT, c.C), from_dev(gw, "bf16"), from_dev(gb, "bf16")))


def test_layernorm_tensor_binding(dev):
    import torch
    from linear_layer_backward_amd import mmb
    c = wl.layernorm_case(2, 40, 768, "bf16", seed=9, prefill=True)

    def t(a, shape=None):
        x = torch.from_numpy(np.asarray(a, np.float32)).to(dev).to(torch.bfloat16)
        return x.reshape(shape) if shape else x
    gi = t(c.dinp0, (c.B, c.T, c.C))
    gw, gb = t(c.dweight0), t(c.dbias0)
    mmb.layernorm_backward(gi, gw, gb, t(c.dout, (c.B, c.T, c.C)), t(c.inp, (c.B, c.T, c.C)),
                           t(c.weight), t(c.mean), t(c.rstd))
    torch.cuda.synchronize(dev)
    check(c, (gi.float().cpu().numpy().reshape(c.BT, c.C).astype(np.float64),
              gw.float().cpu().numpy().astype(np.float64), gb.float().cpu().numpy().astype(np.float64)))
    with pytest.raises(ValueError):
        mmb.layernorm_backward(gi, gw.float(), gb, gi, gi, gw, t(c.mean), t(c.rstd))
