"""Python binding of libmmb.so (C ABI in include/mmb.h).

Argument marshalling only: every step of the backward pass (and of the
forward product) runs in the HIP kernels of the library.  Importing this
module loads ``libmmb.so`` from this package directory and raises
ImportError if it has not been built
(``python -m linear_layer_backward_amd.build``); there is no fallback.

The functions named like the C entry points take raw device addresses
(ints) or torch tensors (their ``data_ptr()`` is passed) and raise
``MmbError`` on a non-zero status, except ``mmb_check_args`` and
``mmb_path`` (and their forward twins), which return the status like their
C counterparts.
``backward`` and ``forward`` are the tensor-level conveniences: they infer
B, T, C, OC and the dtype from the tensors and enqueue on torch's current
stream.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libmmb.so")

MMB_FP32 = 0
MMB_BF16 = 1

STATUS = {
    0: "MMB_OK", -1: "MMB_ERR_NULL", -2: "MMB_ERR_DIM", -3: "MMB_ERR_DTYPE",
    -4: "MMB_ERR_OVERFLOW", -5: "MMB_ERR_ALIAS", -6: "MMB_ERR_HIP", -7: "MMB_ERR_NOMEM",
    -8: "MMB_ERR_NAME", -9: "MMB_ERR_SCRATCH",
}
MMB_NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024

if not os.path.exists(LIBRARY):
    raise ImportError(f"{LIBRARY} is not built; run `python -m linear_layer_backward_amd.build`")

_lib = ctypes.CDLL(LIBRARY)
_vp = ctypes.c_void_p
_i = ctypes.c_int
_ARGS = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i]
_lib.mmb_backward.argtypes = _ARGS
_lib.mmb_backward.restype = _i
_lib.mmb_backward_stream.argtypes = _ARGS + [_vp]
_lib.mmb_backward_stream.restype = _i
_lib.mmb_backward_noalloc.argtypes = _ARGS + [_vp]
_lib.mmb_backward_noalloc.restype = _i
_lib.mmb_check_args.argtypes = _ARGS
_lib.mmb_check_args.restype = _i
_lib.mmb_path.argtypes = _ARGS
_lib.mmb_path.restype = _i
_lib.mmb_strerror.argtypes = [_i]
_lib.mmb_strerror.restype = ctypes.c_char_p
_lib.mmb_plan_units.argtypes = [_i] * 7 + [ctypes.POINTER(_i), ctypes.POINTER(_i), _i]
_lib.mmb_plan_units.restype = _i
_lib.mmb_tile_shape.argtypes = [_i, ctypes.POINTER(_i)]
_lib.mmb_tile_shape.restype = _i
_lib.mmb_release.argtypes = []
_lib.mmb_release.restype = _i
_lib.mmb_backward_sr.argtypes = [_vp] * 6 + [_i] * 4 + [ctypes.c_ulonglong, _vp]
_lib.mmb_backward_sr.restype = _i
_LN_ARGS = [_vp] * 8 + [_i] * 4
_lib.mmb_layernorm_backward.argtypes = _LN_ARGS + [_vp]
_lib.mmb_layernorm_backward.restype = _i
_lib.mmb_layernorm_check_args.argtypes = _LN_ARGS
_lib.mmb_layernorm_check_args.restype = _i
_lib.mmb_layernorm_path.argtypes = _LN_ARGS
_lib.mmb_layernorm_path.restype = _i
_FWD_ARGS = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i]
for _f in ("mmb_forward", "mmb_forward_check_args", "mmb_forward_path"):
    getattr(_lib, _f).argtypes = _FWD_ARGS
    getattr(_lib, _f).restype = _i
_lib.mmb_forward_stream.argtypes = _FWD_ARGS + [_vp]
_lib.mmb_forward_stream.restype = _i
_lib.mmb_forward_plan_units.argtypes = [_i] * 7 + [ctypes.POINTER(_i), ctypes.POINTER(_i), _i]
_lib.mmb_forward_plan_units.restype = _i
_lib.mmb_set_tuning.argtypes = [ctypes.c_char_p, ctypes.c_char_p]
_lib.mmb_set_tuning.restype = _i

# The library reads its MMB_* tuning variables from the environment once, at
# load; this mirror of the values set through mmb_set_tuning lets `tuning`
# restore them.
_TUNING_NAMES = ("MMB_SPLITS_DWEIGHT", "MMB_SPLITS_DINP", "MMB_SPLITS_FWD", "MMB_PLAN_MODEL",
                 "MMB_PLAN_TRACE", "MMB_LN_WORKGROUPS")
_tuning_now = {k: os.environ.get(k) for k in _TUNING_NAMES}


class MmbError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {mmb_strerror(status)}")


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    return x.data_ptr() or None


def _args(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype):
    return (_addr(dinp), _addr(dweight), _addr(dbias), _addr(dout), _addr(inp),
            _addr(weight), int(B), int(T), int(C), int(OC), int(dtype))


def mmb_strerror(status: int) -> str:
    return _lib.mmb_strerror(int(status)).decode()


def mmb_set_tuning(name: str, value) -> None:
    """Set one tuning variable of the library (None clears it)."""
    st = _lib.mmb_set_tuning(name.encode(), None if value is None else str(value).encode())
    if st != 0:
        raise MmbError(st)
    _tuning_now[name] = None if value is None else str(value)


class tuning:
    """Context manager: ``with mmb.tuning(MMB_SPLITS_DWEIGHT="4"):`` sets the
    given tuning variables (None clears one) and restores the previous values
    on exit."""

    def __init__(self, **values):
        self.values = values
        self.saved = {}

    def __enter__(self):
        for k, v in self.values.items():
            self.saved[k] = _tuning_now.get(k)
            mmb_set_tuning(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self.saved.items():
            mmb_set_tuning(k, v)
        return False


def mmb_check_args(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype) -> int:
    return _lib.mmb_check_args(*_args(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype))


def mmb_path(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype) -> int:
    return _lib.mmb_path(*_args(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype))


def mmb_backward(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype) -> None:
    st = _lib.mmb_backward(*_args(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype))
    if st != 0:
        raise MmbError(st)


def mmb_backward_stream(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype,
                        stream) -> None:
    s = stream if isinstance(stream, int) or stream is None else stream.cuda_stream
    st = _lib.mmb_backward_stream(*_args(dinp, dweight, dbias, dout, inp, weight,
                                         B, T, C, OC, dtype), s or None)
    if st != 0:
        raise MmbError(st)


def mmb_backward_noalloc(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, dtype,
                         stream) -> None:
    """mmb_backward_stream with the library's fixed per-device scratch instead
    of allocated workspace (no allocation, no host-to-device copy)."""
    s = stream if isinstance(stream, int) or stream is None else stream.cuda_stream
    st = _lib.mmb_backward_noalloc(*_args(dinp, dweight, dbias, dout, inp, weight,
                                          B, T, C, OC, dtype), s or None)
    if st != 0:
        raise MmbError(st)


def mmb_backward_sr(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, seed,
                    stream) -> None:
    """bf16 backward with stochastically rounded dweight and dbias."""
    s = stream if isinstance(stream, int) or stream is None else stream.cuda_stream
    a = _args(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, MMB_BF16)[:10]
    st = _lib.mmb_backward_sr(*a, int(seed) & ((1 << 64) - 1), s or None)
    if st != 0:
        raise MmbError(st)


def _ln_args(dinp, dweight, dbias, dout, inp, weight, mean, rstd, B, T, C, dtype):
    return tuple(_addr(t) for t in (dinp, dweight, dbias, dout, inp, weight, mean, rstd)) + (
        int(B), int(T), int(C), int(dtype))


def mmb_layernorm_backward(dinp, dweight, dbias, dout, inp, weight, mean, rstd, B, T, C, dtype,
                           stream) -> None:
    """LayerNorm backward (all three outputs accumulate)."""
    s = stream if isinstance(stream, int) or stream is None else stream.cuda_stream
    st = _lib.mmb_layernorm_backward(*_ln_args(dinp, dweight, dbias, dout, inp, weight, mean,
                                               rstd, B, T, C, dtype), s or None)
    if st != 0:
        raise MmbError(st)


def mmb_layernorm_check_args(*a) -> int:
    return _lib.mmb_layernorm_check_args(*_ln_args(*a))


def mmb_layernorm_path(*a) -> int:
    return _lib.mmb_layernorm_path(*_ln_args(*a))


def _fwd_args(out, inp, weight, bias, B, T, C, OC, dtype):
    return (_addr(out), _addr(inp), _addr(weight), _addr(bias), int(B), int(T), int(C),
            int(OC), int(dtype))


def mmb_forward_check_args(out, inp, weight, bias, B, T, C, OC, dtype) -> int:
    return _lib.mmb_forward_check_args(*_fwd_args(out, inp, weight, bias, B, T, C, OC, dtype))


def mmb_forward_path(out, inp, weight, bias, B, T, C, OC, dtype) -> int:
    return _lib.mmb_forward_path(*_fwd_args(out, inp, weight, bias, B, T, C, OC, dtype))


def mmb_forward(out, inp, weight, bias, B, T, C, OC, dtype) -> None:
    st = _lib.mmb_forward(*_fwd_args(out, inp, weight, bias, B, T, C, OC, dtype))
    if st != 0:
        raise MmbError(st)


def mmb_forward_stream(out, inp, weight, bias, B, T, C, OC, dtype, stream) -> None:
    s = stream if isinstance(stream, int) or stream is None else stream.cuda_stream
    st = _lib.mmb_forward_stream(*_fwd_args(out, inp, weight, bias, B, T, C, OC, dtype),
                                 s or None)
    if st != 0:
        raise MmbError(st)


def mmb_forward_plan_units(B, T, C, OC, dtype, has_bias, num_cus):
    """(largest split count, list of units) of the forward plan, as
    mmb_plan_units.  Host only."""
    sp = (_i * 1)()
    n = _lib.mmb_forward_plan_units(B, T, C, OC, dtype, int(has_bias), num_cus, sp, None, 0)
    if n < 0:
        raise MmbError(n)
    buf = (_i * (8 * n))()
    _lib.mmb_forward_plan_units(B, T, C, OC, dtype, int(has_bias), num_cus, sp, buf, n)
    return sp[0], [tuple(buf[8 * k:8 * k + 8]) for k in range(n)]


def mmb_release() -> None:
    st = _lib.mmb_release()
    if st != 0:
        raise MmbError(st)


def mmb_plan_units(B, T, C, OC, dtype, has_bias, num_cus):
    """(largest split counts {dweight, dinp}, list of units (kind, tile_m,
    tile_n, split, kt0, kt1, splits of the tile, first workspace slot)) of the
    plan for a device with num_cus compute units.  Host only."""
    sp = (_i * 2)()
    n = _lib.mmb_plan_units(B, T, C, OC, dtype, int(has_bias), num_cus, sp, None, 0)
    if n < 0:
        raise MmbError(n)
    buf = (_i * (8 * n))()
    _lib.mmb_plan_units(B, T, C, OC, dtype, int(has_bias), num_cus, sp, buf, n)
    return (sp[0], sp[1]), [tuple(buf[8 * k:8 * k + 8]) for k in range(n)]


def mmb_tile_shape(dtype):
    """(BM, BN, BK) of the MFMA tiles for dtype.  Host only."""
    sh = (_i * 3)()
    st = _lib.mmb_tile_shape(int(dtype), sh)
    if st != 0:
        raise MmbError(st)
    return sh[0], sh[1], sh[2]


def torch_dtype_code(dt) -> int:
    import torch
    if dt == torch.float32:
        return MMB_FP32
    if dt == torch.bfloat16:
        return MMB_BF16
    raise TypeError(f"unsupported dtype {dt}")


def backward(dinp, dweight, dbias, dout, inp, weight, B=None, T=None, stream=None) -> None:
    """dinp += dout.weight, dweight += dout^T.inp, dbias = sum of dout rows.

    Tensors: contiguous, on one GPU, all float32 or all bfloat16.  dout is
    [B, T, OC] (or [B*T, OC] with B and T given), inp/dinp hold B*T*C
    elements, weight/dweight OC*C, dbias OC or None.  Enqueued on `stream`
    (default: torch's current stream of dout's device)."""
    import torch
    ts = [dinp, dweight, dout, inp, weight] + ([dbias] if dbias is not None else [])
    dt = dout.dtype
    for t in ts:
        if not t.is_cuda or not t.is_contiguous() or t.dtype != dt or t.device != dout.device:
            raise ValueError("tensors must be contiguous, on one GPU, and share one dtype")
    OC = dout.shape[-1]
    if B is None or T is None:
        if dout.dim() != 3:
            raise ValueError("give B and T for a 2-D dout")
        B, T = dout.shape[0], dout.shape[1]
    if dout.numel() != B * T * OC or weight.numel() % OC != 0:
        raise ValueError("inconsistent shapes")
    C = weight.numel() // OC
    if inp.numel() != B * T * C or dinp.numel() != B * T * C or dweight.numel() != OC * C:
        raise ValueError("inconsistent shapes")
    if dbias is not None and dbias.numel() != OC:
        raise ValueError("dbias must hold OC elements")
    if stream is None:
        stream = torch.cuda.current_stream(dout.device)
    with torch.cuda.device(dout.device):
        mmb_backward_stream(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC,
                            torch_dtype_code(dt), stream)


def forward(out, inp, weight, bias=None, B=None, T=None, stream=None) -> None:
    """out = inp . weight^T + bias (assigned).

    Tensors: contiguous, on one GPU, all float32 or all bfloat16.  inp is
    [B, T, C] (or [B*T, C] with B and T given), weight [OC, C], out B*T*OC
    elements, bias OC or None.  Enqueued on `stream` (default: torch's
    current stream of inp's device)."""
    import torch
    ts = [out, inp, weight] + ([bias] if bias is not None else [])
    dt = inp.dtype
    for t in ts:
        if not t.is_cuda or not t.is_contiguous() or t.dtype != dt or t.device != inp.device:
            raise ValueError("tensors must be contiguous, on one GPU, and share one dtype")
    if weight.dim() != 2:
        raise ValueError("weight must be [OC, C]")
    OC, C = weight.shape
    if B is None or T is None:
        if inp.dim() != 3:
            raise ValueError("give B and T for a 2-D inp")
        B, T = inp.shape[0], inp.shape[1]
    if inp.numel() != B * T * C or out.numel() != B * T * OC:
        raise ValueError("inconsistent shapes")
    if bias is not None and bias.numel() != OC:
        raise ValueError("bias must hold OC elements")
    if stream is None:
        stream = torch.cuda.current_stream(inp.device)
    with torch.cuda.device(inp.device):
        mmb_forward_stream(out, inp, weight, bias, B, T, C, OC, torch_dtype_code(dt), stream)


def backward_sr(dinp, dweight, dbias, dout, inp, weight, seed, B=None, T=None,
                stream=None) -> None:
    """As backward() for bfloat16 tensors, with dweight and dbias rounded
    stochastically under `seed` (see mmb_backward_sr in include/mmb.h)."""
    import torch
    ts = [dinp, dweight, dout, inp, weight] + ([dbias] if dbias is not None else [])
    for t in ts:
        if (not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16
                or t.device != dout.device):
            raise ValueError("tensors must be contiguous bfloat16 on one GPU")
    OC = dout.shape[-1]
    if B is None or T is None:
        if dout.dim() != 3:
            raise ValueError("give B and T for a 2-D dout")
        B, T = dout.shape[0], dout.shape[1]
    if dout.numel() != B * T * OC or weight.numel() % OC != 0:
        raise ValueError("inconsistent shapes")
    C = weight.numel() // OC
    if inp.numel() != B * T * C or dinp.numel() != B * T * C or dweight.numel() != OC * C:
        raise ValueError("inconsistent shapes")
    if dbias is not None and dbias.numel() != OC:
        raise ValueError("dbias must hold OC elements")
    if stream is None:
        stream = torch.cuda.current_stream(dout.device)
    with torch.cuda.device(dout.device):
        mmb_backward_sr(dinp, dweight, dbias, dout, inp, weight, B, T, C, OC, seed, stream)


def layernorm_backward(dinp, dweight, dbias, dout, inp, weight, mean, rstd, B=None, T=None,
                       stream=None) -> None:
    """LayerNorm backward, every output accumulating (see
    mmb_layernorm_backward in include/mmb.h).  Tensors contiguous on one GPU,
    all float32 or all bfloat16: dout, inp, dinp [B, T, C] (or B*T*C elements
    with B and T given), weight, dweight, dbias [C], mean, rstd [B*T]."""
    import torch
    ts = [dinp, dweight, dbias, dout, inp, weight, mean, rstd]
    dt = dout.dtype
    for t in ts:
        if not t.is_cuda or not t.is_contiguous() or t.dtype != dt or t.device != dout.device:
            raise ValueError("tensors must be contiguous, on one GPU, and share one dtype")
    C = weight.numel()
    if B is None or T is None:
        if dout.dim() != 3:
            raise ValueError("give B and T for a 2-D dout")
        B, T = dout.shape[0], dout.shape[1]
    if dout.numel() != B * T * C or inp.numel() != B * T * C or dinp.numel() != B * T * C:
        raise ValueError("inconsistent shapes")
    if dweight.numel() != C or dbias.numel() != C or mean.numel() != B * T or rstd.numel() != B * T:
        raise ValueError("inconsistent shapes")
    if stream is None:
        stream = torch.cuda.current_stream(dout.device)
    with torch.cuda.device(dout.device):
        mmb_layernorm_backward(dinp, dweight, dbias, dout, inp, weight, mean, rstd, B, T, C,
                               torch_dtype_code(dt), stream)
