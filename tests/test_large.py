"""GPU parity at the largest tensors: more than 2^31 elements (over 4 GiB of
bf16) in one operand, so that element and byte offsets pass 2^31 and 2^32.

The tile kernels address memory through 32-bit buffer offsets from a 64-bit
origin that moves with every stage and output tile; these cases reach the
rows past those limits:

* tall: B*T = 2^21 rows, C = 1040, OC = 264 -- inp, dinp (read-modify-write)
  and the forward's A operand hold 2.18e9 elements; dweight's K = B*T runs
  over all of them (split K); the forward product reads the same inp.
* wide: the padded GPT-2 LM head at B*T = 43008 rows -- dout holds 2.16e9
  elements, read row-wise by dinp and column-wise by dweight.

Inputs are integers in [-2, 2] (one byte per element on the host), so every
sum is an exact integer below 2^24 and the bf16 results must equal the
oracle's exact value rounded once to nearest-even.  The oracle computes
sampled rows and columns: the first and last rows, the rows around element
2^31 and random ones.
"""
import numpy as np
import pytest

import oracle
from linear_layer_backward_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from linear_layer_backward_amd import mmb  # noqa: F401  (fails loudly if unbuilt)
    return torch.device("cuda:0")


def upload(vals, dev):
    """int8 host values -> a bf16 device tensor of the same shape (the
    widening runs on the device; integers of this size are exact in bf16)."""
    import torch
    return torch.from_numpy(vals).to(dev).to(torch.bfloat16)


def fetch(t):
    """bf16 device tensor -> float64 host values."""
    import torch
    return wl.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


def rne_bf16(x):
    """Exact integer values (|x| < 2^24) -> nearest-even bf16, as float64."""
    return wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


def pick(n, fixed, k, seed):
    rng = np.random.default_rng(seed)
    s = {i for i in fixed if 0 <= i < n} | set(rng.integers(0, n, size=k).tolist())
    return np.array(sorted(s))


def f64(a):
    return np.asarray(a, dtype=np.float64)


def test_tall_rows_past_2_31_elements(dev):
    import torch
    from linear_layer_backward_amd import mmb
    B, T, C, OC = 2048, 1024, 1040, 264
    BT = B * T
    assert BT * C > 2 ** 31
    print(f"[large] tall B={B} T={T} C={C} OC={OC} bf16: drawing", flush=True)
    inp = wl.small_integers(1, (BT, C))
    weight = wl.small_integers(2, (OC, C))
    dout = wl.small_integers(3, (BT, OC))
    dinp0 = wl.small_integers(4, (BT, C))
    dweight0 = wl.small_integers(5, (OC, C))
    bias = wl.small_integers(6, (OC,))
    d_inp, d_w, d_dout = upload(inp, dev), upload(weight, dev), upload(dout, dev)
    d_dinp, d_dw = upload(dinp0, dev), upload(dweight0, dev)
    d_db = torch.zeros(OC, dtype=torch.bfloat16, device=dev)
    d_bias = upload(bias, dev)
    d_out = torch.full((BT, OC), float("nan"), dtype=torch.bfloat16, device=dev)
    args = (d_dinp, d_dw, d_db, d_dout, d_inp, d_w, B, T, C, OC, mmb.MMB_BF16)
    assert mmb.mmb_path(*args) == 1
    print("[large] tall: backward and forward", flush=True)
    mmb.mmb_backward(*args)
    mmb.mmb_forward(d_out, d_inp, d_w, d_bias, B, T, C, OC, mmb.MMB_BF16)
    torch.cuda.synchronize()

    edge = 2 ** 31 // C   # the row holding element 2^31 of inp and dinp
    rows = pick(BT, [0, 1, 255, 256, edge - 1, edge, edge + 1, BT - 257, BT - 256, BT - 2,
                     BT - 1], 24, 7)
    chans = pick(OC, [0, 1, 255, 256, OC - 2, OC - 1], 10, 8)
    cols = pick(C, [0, 1, 255, 256, 1023, 1024, C - 2, C - 1], 16, 9)
    print(f"[large] tall: oracle on {len(rows)} rows, {len(chans)}x{len(cols)} dweight "
          "entries, all of dbias", flush=True)
    ri = oracle.dinp(f64(dout[rows]), f64(weight), f64(dinp0[rows]), B=1, T=len(rows), C=C, OC=OC)
    rw = oracle.dweight(f64(dout[:, chans]), f64(inp[:, cols]), f64(dweight0[chans][:, cols]),
                        B=1, T=BT, C=len(cols), OC=len(chans))
    rb = oracle.dbias(f64(dout), B=1, T=BT, OC=OC)
    ro = oracle.forward(f64(inp[rows]), f64(weight), f64(bias), B=1, T=len(rows), C=C, OC=OC)
    rows_t = torch.from_numpy(rows).to(dev)
    np.testing.assert_array_equal(fetch(d_dinp.index_select(0, rows_t)), rne_bf16(ri))
    got_w = fetch(d_dw)[chans][:, cols]
    np.testing.assert_array_equal(got_w, rne_bf16(rw))
    np.testing.assert_array_equal(fetch(d_db), rne_bf16(rb))
    np.testing.assert_array_equal(fetch(d_out.index_select(0, rows_t)), rne_bf16(ro))


def test_wide_lm_head_past_2_31_elements(dev):
    import torch
    from linear_layer_backward_amd import mmb
    B, T, C, OC = 42, 1024, 768, 50304
    BT = B * T
    assert BT * OC > 2 ** 31
    print(f"[large] wide B={B} T={T} C={C} OC={OC} bf16: drawing", flush=True)
    inp = wl.small_integers(11, (BT, C))
    weight = wl.small_integers(12, (OC, C))
    dout = wl.small_integers(13, (BT, OC))
    dinp0 = wl.small_integers(14, (BT, C))
    dweight0 = wl.small_integers(15, (OC, C))
    d_inp, d_w, d_dout = upload(inp, dev), upload(weight, dev), upload(dout, dev)
    d_dinp, d_dw = upload(dinp0, dev), upload(dweight0, dev)
    args = (d_dinp, d_dw, None, d_dout, d_inp, d_w, B, T, C, OC, mmb.MMB_BF16)
    assert mmb.mmb_path(*args) == 1
    print("[large] wide: backward", flush=True)
    mmb.mmb_backward(*args)
    torch.cuda.synchronize()

    edge = 2 ** 31 // OC   # the row holding element 2^31 of dout
    rows = pick(BT, [0, 1, 255, 256, edge - 1, edge, edge + 1, BT - 257, BT - 256, BT - 2,
                     BT - 1], 16, 17)
    chans = pick(OC, [0, 1, 255, 256, 50047, 50048, OC - 2, OC - 1], 16, 18)
    print(f"[large] wide: oracle on {len(rows)} rows and {len(chans)} channels", flush=True)
    ri = oracle.dinp(f64(dout[rows]), f64(weight), f64(dinp0[rows]), B=1, T=len(rows), C=C, OC=OC)
    rw = oracle.dweight(f64(dout[:, chans]), f64(inp), f64(dweight0[chans]),
                        B=1, T=BT, C=C, OC=len(chans))
    np.testing.assert_array_equal(fetch(d_dinp[torch.from_numpy(rows).to(dev)]), rne_bf16(ri))
    np.testing.assert_array_equal(fetch(d_dw[torch.from_numpy(chans).to(dev)]), rne_bf16(rw))
