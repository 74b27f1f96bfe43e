"""CPU oracle for the GPT-2 linear-layer backward pass and its forward
(test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does; the two share no code.

The arithmetic lives in ``mmb_oracle.c`` (plain C, IEEE double, OpenMP over
independent output elements).  This module only compiles it with gcc and
marshals numpy arrays through ctypes.  Method source: the llm.c page
"dev/cuda/matmul_backward.cu", CPU reference ``matmul_backward_cpu`` and the
cuBLAS launcher ``matmul_backward1``.

Every function returns new float64 arrays and never modifies its inputs.
The dbias and forward output buffers are filled with NaN before the C code
runs, so a result that added onto the buffer instead of assigning it would
show.  ``forward`` is the layer's forward product (out = inp . W^T + bias),
the step before the backward pass.  ``backward_sr`` rounds the bf16
parameter gradients stochastically (Philox-4x64-10 random bits, see
mmb_oracle.c).  ``layernorm_backward`` is the adjacent LayerNorm backward
of the same model (its own page, dev/cuda/layernorm_backward.cu).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "mmb_oracle.c")
LIBRARY = os.path.join(_HERE, "libmmb_oracle.so")


def compile_library(source: str, out: str, verbose: bool = False) -> str:
    """gcc -O2 -fopenmp: compile an oracle source file into a shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-Wall", "-Werror", source, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile mmb_oracle.c into libmmb_oracle.so next to it."""
    return compile_library(SOURCE, LIBRARY, verbose)


def _f64(a, shape):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if a.shape != tuple(shape):
        a = a.reshape(shape)
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        L = ctypes.c_long
        lib.mmb_oracle_dinp.argtypes = [dp, dp, dp, L, L, L, L]
        lib.mmb_oracle_dweight.argtypes = [dp, dp, dp, L, L, L, L]
        lib.mmb_oracle_dbias.argtypes = [dp, dp, L, L, L]
        lib.mmb_oracle_backward.argtypes = [dp, dp, dp, dp, dp, dp, L, L, L, L]
        lib.mmb_oracle_forward.argtypes = [dp, dp, dp, dp, L, L, L, L]
        for f in ("mmb_oracle_dinp", "mmb_oracle_dweight", "mmb_oracle_dbias",
                  "mmb_oracle_backward", "mmb_oracle_forward"):
            getattr(lib, f).restype = None
        lib.mmb_oracle_layernorm_backward.argtypes = [dp] * 8 + [L, L, L]
        lib.mmb_oracle_layernorm_backward.restype = None
        u64 = ctypes.c_uint64
        lib.mmb_oracle_philox4x64_10.argtypes = [ctypes.POINTER(u64), ctypes.POINTER(u64),
                                                 ctypes.POINTER(u64)]
        lib.mmb_oracle_philox4x64_10.restype = None
        lib.mmb_oracle_sr_bits.argtypes = [u64, u64, u64, u64]
        lib.mmb_oracle_sr_bits.restype = ctypes.c_uint32
        lib.mmb_oracle_sr_bf16.argtypes = [ctypes.c_float, ctypes.c_uint32]
        lib.mmb_oracle_sr_bf16.restype = ctypes.c_uint16
        lib.mmb_oracle_round_sr.argtypes = [ctypes.POINTER(ctypes.c_uint16), dp, L, L, u64, u64]
        lib.mmb_oracle_round_sr.restype = None
        lib.mmb_oracle_threads.argtypes = []
        lib.mmb_oracle_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def dinp(self, dout, weight, dinp_prefill=None, *, B, T, C, OC):
        """dinp_prefill + dout @ weight, shape [B*T, C]."""
        d = _f64(dout, (B * T, OC))
        w = _f64(weight, (OC, C))
        out = (np.zeros((B * T, C)) if dinp_prefill is None
               else _f64(dinp_prefill, (B * T, C)).copy())
        self.lib.mmb_oracle_dinp(_ptr(out), _ptr(d), _ptr(w), B, T, C, OC)
        return out

    def dweight(self, dout, inp, dweight_prefill=None, *, B, T, C, OC):
        """dweight_prefill + dout^T @ inp, shape [OC, C]."""
        d = _f64(dout, (B * T, OC))
        x = _f64(inp, (B * T, C))
        out = (np.zeros((OC, C)) if dweight_prefill is None
               else _f64(dweight_prefill, (OC, C)).copy())
        self.lib.mmb_oracle_dweight(_ptr(out), _ptr(d), _ptr(x), B, T, C, OC)
        return out

    def dbias(self, dout, *, B, T, OC):
        """Column sums of dout over all B*T rows, shape [OC]."""
        d = _f64(dout, (B * T, OC))
        out = np.full(OC, np.nan)
        self.lib.mmb_oracle_dbias(_ptr(out), _ptr(d), B, T, OC)
        return out

    def backward(self, dout, inp, weight, dinp_prefill=None, dweight_prefill=None,
                 with_bias=True, *, B, T, C, OC):
        """The whole pass in one call: (dinp, dweight, dbias or None)."""
        d = _f64(dout, (B * T, OC))
        x = _f64(inp, (B * T, C))
        w = _f64(weight, (OC, C))
        gi = (np.zeros((B * T, C)) if dinp_prefill is None
              else _f64(dinp_prefill, (B * T, C)).copy())
        gw = (np.zeros((OC, C)) if dweight_prefill is None
              else _f64(dweight_prefill, (OC, C)).copy())
        gb = np.full(OC, np.nan) if with_bias else None
        self.lib.mmb_oracle_backward(_ptr(gi), _ptr(gw),
                                     _ptr(gb) if with_bias else None,
                                     _ptr(d), _ptr(x), _ptr(w), B, T, C, OC)
        return gi, gw, gb

    def forward(self, inp, weight, bias=None, *, B, T, C, OC):
        """inp @ weight^T (+ bias), shape [B*T, OC]; assigned, not accumulated."""
        x = _f64(inp, (B * T, C))
        w = _f64(weight, (OC, C))
        b = None if bias is None else _f64(bias, (OC,))
        out = np.full((B * T, OC), np.nan)
        self.lib.mmb_oracle_forward(_ptr(out), _ptr(x), _ptr(w),
                                    None if b is None else _ptr(b), B, T, C, OC)
        return out

    def philox(self, ctr, key):
        """Philox-4x64-10 of a 4-word counter and a 2-word key (ints)."""
        u64 = ctypes.c_uint64
        c, k, o = (u64 * 4)(*ctr), (u64 * 2)(*key), (u64 * 4)()
        self.lib.mmb_oracle_philox4x64_10(c, k, o)
        return [int(v) for v in o]

    def sr_bits(self, seed, tag, row, col) -> int:
        """The 16 random bits of element (row, col) of gradient `tag`."""
        return int(self.lib.mmb_oracle_sr_bits(seed, tag, row, col))

    def sr_bf16(self, x, r16) -> int:
        """bf16 bits of the float x rounded with random bits r16."""
        return int(self.lib.mmb_oracle_sr_bf16(float(x), int(r16)))

    def round_sr(self, exact, seed, tag):
        """Stochastic bf16 rounding (uint16 bits) of a 2-D array of exact
        values, element (r, c) with its own random bits."""
        e = np.ascontiguousarray(np.asarray(exact, dtype=np.float64))
        if e.ndim == 1:
            e = e.reshape(1, -1)
        out = np.zeros(e.shape, np.uint16)
        self.lib.mmb_oracle_round_sr(out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                     _ptr(e), e.shape[0], e.shape[1], seed, tag)
        return out

    def backward_sr(self, dout, inp, weight, dinp_prefill=None, dweight_prefill=None,
                    with_bias=True, *, seed, B, T, C, OC):
        """The bf16 backward pass with stochastic rounding of the parameter
        gradients: (dinp exact, dweight bf16 bits, dbias bf16 bits or None).
        dinp is returned exact (it is rounded to nearest on the GPU side)."""
        gi, gw, gb = self.backward(dout, inp, weight, dinp_prefill, dweight_prefill, with_bias,
                                   B=B, T=T, C=C, OC=OC)
        return (gi, self.round_sr(gw, seed, 1),
                self.round_sr(gb, seed, 2).ravel() if with_bias else None)

    def layernorm_backward(self, dout, inp, weight, mean, rstd, dinp_prefill=None,
                           dweight_prefill=None, dbias_prefill=None, *, B, T, C):
        """LayerNorm backward: (dinp [BT,C], dweight [C], dbias [C]), each
        added onto its prefill (zeros when None)."""
        BT = B * T
        d, x = _f64(dout, (BT, C)), _f64(inp, (BT, C))
        w, m, s = _f64(weight, (C,)), _f64(mean, (BT,)), _f64(rstd, (BT,))
        gi = np.zeros((BT, C)) if dinp_prefill is None else _f64(dinp_prefill, (BT, C)).copy()
        gw = np.zeros(C) if dweight_prefill is None else _f64(dweight_prefill, (C,)).copy()
        gb = np.zeros(C) if dbias_prefill is None else _f64(dbias_prefill, (C,)).copy()
        self.lib.mmb_oracle_layernorm_backward(_ptr(gi), _ptr(gw), _ptr(gb), _ptr(d), _ptr(x),
                                               _ptr(w), _ptr(m), _ptr(s), B, T, C)
        return gi, gw, gb

    def threads(self) -> int:
        """OpenMP threads the parallel loops use."""
        return int(self.lib.mmb_oracle_threads())


_default = None


def _get() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default


def dinp(*a, **k):
    return _get().dinp(*a, **k)


def dweight(*a, **k):
    return _get().dweight(*a, **k)


def dbias(*a, **k):
    return _get().dbias(*a, **k)


def backward(*a, **k):
    return _get().backward(*a, **k)


def forward(*a, **k):
    return _get().forward(*a, **k)


def philox(*a, **k):
    return _get().philox(*a, **k)


def sr_bits(*a, **k):
    return _get().sr_bits(*a, **k)


def sr_bf16(*a, **k):
    return _get().sr_bf16(*a, **k)


def round_sr(*a, **k):
    return _get().round_sr(*a, **k)


def backward_sr(*a, **k):
    return _get().backward_sr(*a, **k)


def layernorm_backward(*a, **k):
    return _get().layernorm_backward(*a, **k)


def threads() -> int:
    return _get().threads()


def case_backward(case, o: Oracle | None = None):
    """Run the oracle on a workloads.Case (any object with the same fields)."""
    o = o or _get()
    return o.backward(case.dout, case.inp, case.weight, case.dinp0, case.dweight0,
                      case.dbias0 is not None,
                      B=case.B, T=case.T, C=case.C, OC=case.OC)
