"""Seeded synthetic inputs for the linear-layer backward workloads.

Both sides of every parity check (the HIP library and the CPU oracle) take
their inputs from here, so this module holds none of the backward pass's
arithmetic: it only draws numbers, shapes them into the tensors a GPT-2
linear layer sees, and rounds them to the storage dtype.  It imports neither
the HIP binding nor the oracle.

Layouts are dense row-major, as on the llm.c page "dev/cuda/matmul_backward.cu"
(CPU reference ``matmul_backward_cpu``): inp [B*T, C], weight [OC, C],
dout [B*T, OC], dinp [B*T, C], dweight [OC, C], dbias [OC].

Every float tensor is returned as float32 whose values are exactly
representable in the case's storage dtype ("f32" or "bf16"); ``storage``
turns it into the bytes a device buffer holds.  Seeds: numpy
``Generator(PCG64(seed))`` with ``seed = 1000 * config + tensor_id``
(inp 0, weight 1, dout 2, dinp prefill 3, dweight prefill 4, logits 5,
targets 6; the second layer of the MLP pair adds 100).  N(0, s) means
standard deviation s.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

DTYPES = ("f32", "bf16")

# tensor ids inside a config's seed block
INP, WEIGHT, DOUT, DINP0, DWEIGHT0, LOGITS, TARGETS = range(7)

GPT2_VOCAB = 50257
GPT2_VOCAB_PADDED = 50304


@dataclass
class Case:
    """One call's worth of inputs and initial output-buffer contents."""
    name: str
    dtype: str
    B: int
    T: int
    C: int
    OC: int
    inp: np.ndarray
    weight: np.ndarray
    dout: np.ndarray
    dinp0: np.ndarray
    dweight0: np.ndarray
    dbias0: Optional[np.ndarray]          # None: the call passes dbias = NULL
    meta: dict = field(default_factory=dict)

    @property
    def BT(self) -> int:
        return self.B * self.T

    @property
    def with_bias(self) -> bool:
        return self.dbias0 is not None

    def flops(self) -> int:
        """4*B*T*C*OC multiply-adds counted as 2 flops, plus one add per
        dout element for the bias reduction when dbias is present."""
        f = 4 * self.BT * self.C * self.OC
        if self.with_bias:
            f += self.BT * self.OC
        return f


# ---------------------------------------------------------------------------
# rounding to the storage dtype (input preparation only)

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits.
    Inputs must be finite."""
    # finite float32 bit patterns are <= 0xFF7FFFFF, so the biased sum stays
    # below 2**32 and uint32 arithmetic cannot wrap
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_dtype_values(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64/float32 draw -> float32 values exactly representable in dtype."""
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(x32)
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(x32))
    raise ValueError(f"unknown dtype {dtype!r}")


def storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """The raw contents of a device buffer holding x in dtype: float32, or
    uint16 bfloat16 bits.  x must already be representable (no rounding
    happens for bf16 values that came from to_dtype_values)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def from_storage(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Inverse of storage(): device buffer contents -> float32 values."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(np.asarray(raw).view(np.uint16))
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# draws

def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(seed: int, shape, std: float, dtype: str) -> np.ndarray:
    x = _rng(seed).standard_normal(shape, dtype=np.float64) * std
    return to_dtype_values(x, dtype)


def _gelu(x: np.ndarray) -> np.ndarray:
    # exact GELU, x * Phi(x); only shapes the fc_proj input distribution
    from scipy.special import erf
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def lm_head_dout(seed_logits: int, seed_targets: int, BT: int, vocab: int,
                 padded: int, dtype: str, chunk: int = 512) -> np.ndarray:
    """dout of a softmax cross-entropy loss averaged over BT rows:
    (softmax(logits) - onehot(target)) / BT over the first `vocab` columns,
    exact zeros in the padded columns.  logits ~ N(0,1), targets uniform."""
    g_logits = _rng(seed_logits)
    targets = _rng(seed_targets).integers(0, vocab, size=BT)
    out = np.zeros((BT, padded), dtype=np.float32)
    for r0 in range(0, BT, chunk):
        r1 = min(BT, r0 + chunk)
        z = g_logits.standard_normal((r1 - r0, vocab), dtype=np.float64)
        z -= z.max(axis=1, keepdims=True)
        np.exp(z, out=z)
        z /= z.sum(axis=1, keepdims=True)
        z[np.arange(r1 - r0), targets[r0:r1]] -= 1.0
        z /= BT
        out[r0:r1, :vocab] = to_dtype_values(z, dtype)
    return out


# ---------------------------------------------------------------------------
# the five GPT-2 124M workloads

CONFIG_NAMES = {
    1: "tiny fp32 B=2 T=16 C=64 OC=192 (prefilled dinp/dweight)",
    2: "GPT-2 124M qkv backward fp32 B=8 T=1024 C=768 OC=2304",
    3: "GPT-2 124M MLP pair fp32 B=8 T=1024: fc C=768 OC=3072 then fc_proj C=3072 OC=768",
    4: "GPT-2 124M MLP fc backward bf16 B=16 T=1024 C=768 OC=3072",
    5: "GPT-2 124M LM head backward bf16 B=8 T=1024 C=768 OC=50304, no bias",
}

# short file-name forms of the workloads (profile summaries)
CONFIG_SLUGS = {
    1: "tiny_f32_B2_T16_C64_OC192",
    2: "gpt2_qkv_f32_B8_T1024_C768_OC2304",
    3: "gpt2_mlp_pair_f32_B8_T1024",
    4: "gpt2_fc_bf16_B16_T1024_C768_OC3072",
    5: "gpt2_lm_head_bf16_B8_T1024_C768_OC50304",
}


def _case(name, cfg, dtype, B, T, C, OC, inp_std, w_std, dout_std,
          prefill_std, with_bias, inp_gelu=False, seed_add=0):
    s = 1000 * cfg + seed_add
    BT = B * T
    if inp_gelu:
        raw = _rng(s + INP).standard_normal((BT, C), dtype=np.float64) * inp_std
        inp = to_dtype_values(_gelu(raw), dtype)
    else:
        inp = normal(s + INP, (BT, C), inp_std, dtype)
    weight = normal(s + WEIGHT, (OC, C), w_std, dtype)
    dout = normal(s + DOUT, (BT, OC), dout_std, dtype)
    if prefill_std:
        dinp0 = normal(s + DINP0, (BT, C), prefill_std, dtype)
        dweight0 = normal(s + DWEIGHT0, (OC, C), prefill_std, dtype)
    else:
        dinp0 = np.zeros((BT, C), np.float32)
        dweight0 = np.zeros((OC, C), np.float32)
    dbias0 = np.zeros(OC, np.float32) if with_bias else None
    return Case(name, dtype, B, T, C, OC, inp, weight, dout, dinp0, dweight0, dbias0,
                meta={"config": cfg, "seed_base": s})


def config_cases(cfg: int) -> list:
    """The calls that make up one workload (two for the MLP pair)."""
    if cfg == 1:
        return [_case("tiny fp32 B2 T16 C64 OC192", 1, "f32", 2, 16, 64, 192, 1.0, 0.02, 1.0, 0.1, True)]
    if cfg == 2:
        return [_case("qkv fp32 B8 T1024 C768 OC2304", 2, "f32", 8, 1024, 768, 2304, 1.0, 0.02, 1e-3, 0.0, True)]
    if cfg == 3:
        return [_case("fc fp32 B8 T1024 C768 OC3072", 3, "f32", 8, 1024, 768, 3072, 1.0, 0.02, 1e-3, 0.0, True),
                _case("fc_proj fp32 B8 T1024 C3072 OC768", 3, "f32", 8, 1024, 3072, 768, 1.0, 0.02, 1e-3, 0.0,
                      True, inp_gelu=True, seed_add=100)]
    if cfg == 4:
        return [_case("fc bf16 B16 T1024 C768 OC3072", 4, "bf16", 16, 1024, 768, 3072, 1.0, 0.02, 1e-3, 0.0, True)]
    if cfg == 5:
        B, T, C, OC = 8, 1024, 768, GPT2_VOCAB_PADDED
        s = 5000
        inp = normal(s + INP, (B * T, C), 1.0, "bf16")
        weight = normal(s + WEIGHT, (OC, C), 0.02, "bf16")
        dout = lm_head_dout(s + LOGITS, s + TARGETS, B * T, GPT2_VOCAB, OC, "bf16")
        return [Case("lm_head bf16 B8 T1024 C768 OC50304", "bf16", B, T, C, OC, inp, weight, dout,
                     np.zeros((B * T, C), np.float32), np.zeros((OC, C), np.float32),
                     None, meta={"config": 5, "seed_base": s, "vocab": GPT2_VOCAB})]
    raise ValueError(f"no config {cfg}")


def lm_head_unpadded_case() -> Case:
    """The LM-head workload at the real GPT-2 vocabulary, OC = 50257 columns
    (not a multiple of 8): the same draws as config 5 without its 47 zero pad
    columns of dout and pad rows of the weight."""
    B, T, C, OC = 8, 1024, 768, GPT2_VOCAB
    s = 5000
    inp = normal(s + INP, (B * T, C), 1.0, "bf16")
    weight = normal(s + WEIGHT, (OC, C), 0.02, "bf16")
    dout = lm_head_dout(s + LOGITS, s + TARGETS, B * T, GPT2_VOCAB, OC, "bf16")
    return Case("lm_head bf16 B8 T1024 C768 OC50257", "bf16", B, T, C, OC, inp, weight, dout,
                np.zeros((B * T, C), np.float32), np.zeros((OC, C), np.float32),
                None, meta={"config": 5, "seed_base": s, "vocab": GPT2_VOCAB})


# ---------------------------------------------------------------------------
# cases for tests

def random_case(B, T, C, OC, dtype="f32", seed=0, with_bias=True, prefill=True,
                inp_std=1.0, w_std=0.02, dout_std=1.0, prefill_std=0.1) -> Case:
    """Arbitrary shape with the tiny config's distributions."""
    s = 10_000_000 + 1000 * seed
    return _case(f"random B={B} T={T} C={C} OC={OC} {dtype}", 0, dtype, B, T, C, OC,
                 inp_std, w_std, dout_std, prefill_std if prefill else 0.0,
                 with_bias, seed_add=s)


def small_integers(seed: int, shape, lo: int = -2, hi: int = 2) -> np.ndarray:
    """Integers drawn uniformly from [lo, hi] as int8: one byte per element,
    for tensors of billions of elements (the values are exact in fp32 and
    bf16, like integer_case's)."""
    assert -128 <= lo <= hi <= 127
    return _rng(30_000_000 + seed).integers(lo, hi + 1, size=shape, dtype=np.int8)


def integer_case(B, T, C, OC, dtype="f32", seed=0, with_bias=True, prefill=True,
                 lo=-2, hi=2) -> Case:
    """Every input and prefill drawn uniformly from the integers [lo, hi].
    Such values are exact in fp32 and bf16, so with small enough sums every
    product and partial sum is an exact integer in any order."""
    g = _rng(20_000_000 + seed)
    BT = B * T

    def draw(shape):
        return g.integers(lo, hi + 1, size=shape).astype(np.float32)

    inp, weight, dout = draw((BT, C)), draw((OC, C)), draw((BT, OC))
    dinp0 = draw((BT, C)) if prefill else np.zeros((BT, C), np.float32)
    dweight0 = draw((OC, C)) if prefill else np.zeros((OC, C), np.float32)
    dbias0 = np.zeros(OC, np.float32) if with_bias else None
    return Case(f"integer B={B} T={T} C={C} OC={OC} {dtype}", dtype, B, T, C, OC,
                inp, weight, dout, dinp0, dweight0, dbias0, meta={"integer": True})


# ---------------------------------------------------------------------------
# LayerNorm backward inputs (the adjacent op of the same model; page
# "dev/cuda/layernorm_backward.cu", whose benchmark runs B=8, T=1024, C=1600
# with every input from make_random_float, read here as uniform on [-1, 1))

@dataclass
class LNCase:
    """One LayerNorm-backward call: inputs and initial output contents."""
    name: str
    dtype: str
    B: int
    T: int
    C: int
    dout: np.ndarray      # [BT, C]
    inp: np.ndarray       # [BT, C]
    weight: np.ndarray    # [C]
    mean: np.ndarray      # [BT], the forward's saved row means
    rstd: np.ndarray      # [BT], the forward's saved 1/sqrt(var + eps)
    dinp0: np.ndarray     # [BT, C]
    dweight0: np.ndarray  # [C]
    dbias0: np.ndarray    # [C]

    @property
    def BT(self) -> int:
        return self.B * self.T


LN_EPS = 1e-5


def layernorm_stats(inp: np.ndarray, eps: float = LN_EPS):
    """Row statistics the LayerNorm forward saves for its backward (input
    preparation only): mean and 1/sqrt(biased variance + eps), in fp64."""
    x = np.asarray(inp, np.float64)
    m = x.mean(axis=1)
    v = ((x - m[:, None]) ** 2).mean(axis=1)
    return m, 1.0 / np.sqrt(v + eps)


def layernorm_case(B, T, C, dtype="bf16", seed=0, prefill=False) -> LNCase:
    """inp, weight and dout uniform on [-1, 1) (seeded, rounded to dtype);
    mean and rstd from the rounded inp, rounded to dtype as the forward
    stores them; outputs zero or, with prefill, uniform on [-0.1, 0.1)."""
    g = _rng(30_000_000 + seed)
    BT = B * T

    def uni(shape, scale=1.0):
        return to_dtype_values(g.uniform(-scale, scale, size=shape), dtype)

    inp, weight, dout = uni((BT, C)), uni((C,)), uni((BT, C))
    m, r = layernorm_stats(inp)
    mean, rstd = to_dtype_values(m, dtype), to_dtype_values(r, dtype)
    if prefill:
        dinp0, dweight0, dbias0 = uni((BT, C), 0.1), uni((C,), 0.1), uni((C,), 0.1)
    else:
        dinp0 = np.zeros((BT, C), np.float32)
        dweight0, dbias0 = np.zeros(C, np.float32), np.zeros(C, np.float32)
    return LNCase(name=f"layernorm backward {dtype} B{B} T{T} C{C}", dtype=dtype, B=B, T=T, C=C,
                  dout=dout, inp=inp, weight=weight, mean=mean, rstd=rstd, dinp0=dinp0,
                  dweight0=dweight0, dbias0=dbias0)
