"""GPU parity of the stochastically rounded bf16 backward pass
(mmb_backward_sr) through the C ABI against the CPU oracle.

With integer inputs every fp32 sum on the GPU is exact, so the GPU's dweight
and dbias bits must equal the oracle's stochastic rounding of the exact
values bit for bit (same Philox-4x64-10 bits per element), and dinp must
equal the exact value rounded to nearest.  With random inputs the results
stay within the bf16 tolerance and are unbiased.
"""
import numpy as np
import pytest

import oracle
from linear_layer_backward_amd import workloads as wl
from test_parity import assert_close, from_dev, round_bf16, run, sample, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from linear_layer_backward_amd import mmb  # noqa: F401  (fails loudly if unbuilt)
    return torch.device("cuda:0")


def run_sr(case, dev, seed):
    """(dinp float64, dweight bf16 bits, dbias bf16 bits or None)."""
    import torch
    from linear_layer_backward_amd import mmb
    assert case.dtype == "bf16"
    _, dout = to_dev(case.dout, "bf16", dev)
    _, inp = to_dev(case.inp, "bf16", dev)
    _, w = to_dev(case.weight, "bf16", dev)
    _, gi = to_dev(case.dinp0, "bf16", dev)
    _, gw = to_dev(case.dweight0, "bf16", dev)
    gb = to_dev(np.full(case.OC, np.nan, np.float32), "bf16", dev)[1] if case.with_bias else None
    mmb.mmb_backward_sr(gi, gw, gb, dout, inp, w, case.B, case.T, case.C, case.OC, seed,
                        torch.cuda.current_stream(dev))
    torch.cuda.synchronize(dev)

    def bits(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16).copy()

    return (from_dev(gi, "bf16").reshape(case.BT, case.C), bits(gw).reshape(case.OC, case.C),
            bits(gb) if gb is not None else None)


def expected_rows(exact, row_ids, seed, tag):
    """Oracle stochastic rounding of rows `row_ids` of a gradient, element by
    element with each element's own (row, col) bits."""
    out = np.zeros(exact.shape, np.uint16)
    for k, r in enumerate(row_ids):
        for c in range(exact.shape[1]):
            out[k, c] = oracle.sr_bf16(np.float32(exact[k, c]), oracle.sr_bits(seed, tag, int(r), c))
    return out


def bits_to_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


SHAPES = [(2, 150, 264, 400), (1, 513, 200, 136), (1, 1, 8, 8), (4, 300, 64, 96),
          (3, 5, 33, 17), (1, 3, 12, 10)]   # the last two through packed copies


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_sr_integer_exact(dev, shape):
    B, T, C, OC = shape
    case = wl.integer_case(B, T, C, OC, "bf16", seed=C, lo=-4, hi=4)
    seed = 0x1234_5678_9ABC_DEF0 + C
    gi, gw, gb = run_sr(case, dev, seed)
    ri, rw, rb = oracle.backward_sr(case.dout, case.inp, case.weight, case.dinp0,
                                    case.dweight0, True, seed=seed, B=B, T=T, C=C, OC=OC)
    np.testing.assert_array_equal(gi, round_bf16(ri))
    np.testing.assert_array_equal(gw, rw)
    np.testing.assert_array_equal(gb, rb)


@pytest.mark.parametrize("splits", ["2", "3", "5", "2,3,1,4"])
def test_sr_split_k(dev, tune, splits):
    """The split-K fix-up rounds once, with the element's bits, whatever the
    plan: bits equal the oracle's for every split count."""
    tune.set("MMB_SPLITS_DWEIGHT", splits)
    B, T, C, OC = 4, 300, 264, 520
    case = wl.integer_case(B, T, C, OC, "bf16", seed=7, lo=-4, hi=4)
    gi, gw, gb = run_sr(case, dev, 99)
    ri, rw, rb = oracle.backward_sr(case.dout, case.inp, case.weight, case.dinp0,
                                    case.dweight0, True, seed=99, B=B, T=T, C=C, OC=OC)
    assert np.mean(np.abs(bits_to_f64(rw)) > 256) > 0.2   # many values need rounding
    np.testing.assert_array_equal(gw, rw)
    np.testing.assert_array_equal(gb, rb)
    np.testing.assert_array_equal(gi, round_bf16(ri))


def test_sr_full_shape_integer_exact(dev):
    """GPT-2 fc shape (B=16, T=1024, C=768, OC=3072): sampled dweight rows and
    all of dbias bit-exact against the oracle's rounding."""
    B, T, C, OC = 16, 1024, 768, 3072
    case = wl.integer_case(B, T, C, OC, "bf16", seed=3, lo=-2, hi=2)
    print(f"[parity] sr {case.name}", flush=True)
    seed = 2024
    gi, gw, gb = run_sr(case, dev, seed)
    chans = sample(OC, [0, 1, 255, 256, OC - 1], 12, seed=4)
    rw = oracle.dweight(case.dout[:, chans], case.inp, case.dweight0[chans], B=B, T=T, C=C,
                        OC=len(chans))
    np.testing.assert_array_equal(gw[chans], expected_rows(rw, chans, seed, 1))
    rb = oracle.dbias(case.dout, B=B, T=T, OC=OC)
    np.testing.assert_array_equal(gb, oracle.round_sr(rb, seed, 2).ravel())
    rows = sample(case.BT, [0, 255, 256, case.BT - 1], 8, seed=5)
    ri = oracle.dinp(case.dout[rows], case.weight, case.dinp0[rows], B=1, T=len(rows), C=C,
                     OC=OC)
    np.testing.assert_array_equal(gi[rows], round_bf16(ri))


def test_sr_random_inputs(dev):
    """Random inputs (the fc distributions at a smaller B*T): within the bf16
    tolerance; every dweight value is one of the two bf16 neighbours of the
    GPU's own round-to-nearest result or equal to it; dinp identical to the
    round-to-nearest call; unbiased: the mean signed error in units of the
    bf16 spacing is near zero."""
    B, T, C, OC = 4, 1024, 768, 1024
    case = wl.random_case(B, T, C, OC, "bf16", seed=8, prefill=True, dout_std=1e-3,
                          prefill_std=0.02)
    gi, gw, gb = run_sr(case, dev, 5)
    ni, nw, nb = run(case, dev)
    ri, rw, rb = oracle.case_backward(case)
    np.testing.assert_array_equal(gi, ni)
    v = bits_to_f64(gw)
    assert_close(v, rw, "bf16", "dweight (sr)")
    assert_close(bits_to_f64(gb), rb, "bf16", "dbias (sr)")
    step = np.abs(nw) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(v - nw) <= step * 1.01)
    z = (v - rw) / (2.0 ** (np.floor(np.log2(np.abs(rw) + 1e-30)) - 7))
    assert abs(np.mean(z)) < 0.01, np.mean(z)
    assert np.any(v != nw)


def test_sr_deterministic_and_seeded(dev):
    case = wl.random_case(2, 150, 264, 400, "bf16", seed=9)
    a = run_sr(case, dev, 11)
    b = run_sr(case, dev, 11)
    c = run_sr(case, dev, 12)
    assert a[1].tobytes() == b[1].tobytes() and a[2].tobytes() == b[2].tobytes()
    assert a[1].tobytes() != c[1].tobytes()


def test_sr_rejects_bad_arguments(dev):
    from linear_layer_backward_amd import mmb
    with pytest.raises(mmb.MmbError):
        mmb.mmb_backward_sr(0, 0, 0, 0, 0, 0, 1, 1, 8, 8, 1, None)


def test_sr_without_bias(dev):
    """dbias = NULL (the LM-head form): dweight bits still equal the oracle's,
    on a shape with ragged tiles in every dimension."""
    B, T, C, OC = 2, 300, 200, 392
    case = wl.integer_case(B, T, C, OC, "bf16", seed=12, lo=-4, hi=4, with_bias=False)
    gi, gw, gb = run_sr(case, dev, 77)
    assert gb is None
    ri, rw, _ = oracle.backward_sr(case.dout, case.inp, case.weight, case.dinp0, case.dweight0,
                                   False, seed=77, B=B, T=T, C=C, OC=OC)
    np.testing.assert_array_equal(gw, rw)
    np.testing.assert_array_equal(gi, round_bf16(ri))


def test_sr_tensor_binding(dev):
    """The tensor-level call gives the same bits as the C entry point."""
    import torch
    from linear_layer_backward_amd import mmb
    B, T, C, OC = 2, 64, 128, 256
    case = wl.integer_case(B, T, C, OC, "bf16", seed=13, lo=-4, hi=4)
    gi_ref, gw_ref, gb_ref = run_sr(case, dev, 21)

    def t(a, shape=None):
        x = torch.from_numpy(np.asarray(a, np.float32)).to(dev).to(torch.bfloat16)
        return x.reshape(shape) if shape else x
    gi, gw, gb = t(case.dinp0, (B, T, C)), t(case.dweight0), torch.zeros(OC, device=dev,
                                                                            dtype=torch.bfloat16)
    mmb.backward_sr(gi, gw, gb, t(case.dout, (B, T, OC)), t(case.inp), t(case.weight), 21)
    torch.cuda.synchronize(dev)
    bits = lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16).ravel()
    np.testing.assert_array_equal(bits(gw), gw_ref.ravel())
    np.testing.assert_array_equal(bits(gb), gb_ref)
    with pytest.raises(ValueError):
        mmb.backward_sr(gi.float(), gw, gb, t(case.dout, (B, T, OC)), t(case.inp), t(case.weight), 1)
