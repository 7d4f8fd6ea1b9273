"""Seeded synthetic inputs for the MoE expert layer.

This module only draws random numbers and lays them out in the storage
formats the layer consumes.  It holds none of the layer's arithmetic: no
dequantisation, no router, no expert MLP.  Both the oracle-based tests and
the benchmark draw their inputs here, so the two sides always see the same
bytes for a given (workload, seed).

Workloads follow the five shapes of the expert layer described on the
"Laguna-S-2.1 decode" / "batched prefill" commit pages (sigmoid top-10
router with score-correction bias and a shared expert, Q4 expert weights):
a tiny correctness case, single-token decode, 64-token batched decode, a
2048-token prefill chunk and an 8192-token prefill chunk.

Storage formats (the library's boundary formats):
  x          bf16 bit patterns, uint16 [T, d]
  w_router   float32 [E, d]
  bias       float32 [E]
  Q4 matrix  [rows, K]  ->  qs uint8 [rows, K/2]   (element 2i in the low
             nibble of byte i, element 2i+1 in the high nibble)
                            scales uint16 [rows, K/32] (IEEE fp16 bits)
  w13        [E, 2I, d]   gate rows 0..I-1, up rows I..2I-1
  w2         [E, d, I]
  s13        [2Is, d],  s2 [d, Is]   (shared expert)

Draw order from numpy.random.default_rng(seed) (PCG64):
  x (normal), w_router (normal), bias (uniform or permutation), outlier rows,
  then w13 qs, w13 scales, w2 qs, w2 scales, s13 qs, s13 scales, s2 qs,
  s2 scales.  A uniformly random byte holds two independent uniform nibbles,
  so drawing qs bytes uniformly in 0..255 is the same as drawing every q
  uniformly in 0..15.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = ["Dims", "CONFIGS", "make_inputs", "bf16_bits_from_f32", "default_seed"]


@dataclasses.dataclass(frozen=True)
class Dims:
    T: int
    d: int
    E: int
    k: int
    I: int
    I_shared: int

    @property
    def P(self) -> int:
        return self.T * self.k


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    dims: Dims
    bias: str            # "uniform" -> U(-0.1, 0.1); "zipf" -> Zipf(1.2) pmf over a random permutation
    outlier_frac: float  # fraction of token rows scaled by 8 before bf16 rounding
    index: int           # position in the workload list (seed = 1000 + index)


_BIG = dict(d=4096, E=256, k=10, I=1024, I_shared=1024)

CONFIGS = {
    "tiny": Config("tiny", Dims(T=8, d=256, E=16, k=4, I=128, I_shared=128), "uniform", 0.0, 0),
    "decode": Config("decode", Dims(T=1, **_BIG), "uniform", 0.0, 1),
    "batched_decode": Config("batched_decode", Dims(T=64, **_BIG), "uniform", 0.0, 2),
    "prefill": Config("prefill", Dims(T=2048, **_BIG), "zipf", 0.0, 3),
    "long_prefill": Config("long_prefill", Dims(T=8192, **_BIG), "uniform", 0.01, 4),
}


def default_seed(cfg: Config) -> int:
    return 1000 + cfg.index


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _scales(rng: np.random.Generator, shape) -> np.ndarray:
    # d ~ U(0.005, 0.02), rounded to fp16 (numpy's float64 -> float16 cast rounds to nearest even)
    return rng.uniform(0.005, 0.02, size=shape).astype(np.float16).view(np.uint16)


def _qs(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.integers(0, 256, size=shape, dtype=np.uint8)


def make_inputs(cfg: Config | Dims, seed: int | None = None, *, bias: str | None = None,
                outlier_frac: float | None = None, weights: bool = True) -> dict:
    """Draw one layer's inputs.  Returns a dict of numpy arrays (see module docstring).

    `cfg` may be a named Config or bare Dims (then bias="uniform", no outliers
    unless given).  With weights=False only x / w_router / bias are drawn.
    """
    if isinstance(cfg, Config):
        dims = cfg.dims
        bias = cfg.bias if bias is None else bias
        outlier_frac = cfg.outlier_frac if outlier_frac is None else outlier_frac
        seed = default_seed(cfg) if seed is None else seed
    else:
        dims = cfg
        bias = "uniform" if bias is None else bias
        outlier_frac = 0.0 if outlier_frac is None else outlier_frac
        seed = 0 if seed is None else seed
    T, d, E, k, I, Is = dims.T, dims.d, dims.E, dims.k, dims.I, dims.I_shared
    rng = np.random.default_rng(seed)

    xf = rng.standard_normal((T, d)).astype(np.float32)
    w_router = (rng.standard_normal((E, d)) * 0.02).astype(np.float32)
    if bias == "uniform":
        b = rng.uniform(-0.1, 0.1, size=E).astype(np.float32)
    elif bias == "zipf":
        perm = rng.permutation(E)
        ranks = np.arange(1, E + 1, dtype=np.float64)
        pmf = ranks ** -1.2
        pmf /= pmf.sum()
        b = np.empty(E, dtype=np.float32)
        b[perm] = pmf.astype(np.float32)
    elif bias == "zero":
        b = np.zeros(E, dtype=np.float32)
    else:
        raise ValueError(f"unknown bias recipe {bias!r}")
    n_out = int(round(outlier_frac * T))
    outlier_rows = np.sort(rng.permutation(T)[:n_out]) if n_out else np.zeros(0, dtype=np.int64)
    if n_out:
        xf[outlier_rows] *= 8.0  # a power of two: commutes with the bf16 rounding below
    out = dict(
        dims=dims, seed=seed, bias_recipe=bias, outlier_rows=outlier_rows,
        x=bf16_bits_from_f32(xf), w_router=w_router, bias=b,
    )
    if not weights:
        return out
    out["w13_qs"] = _qs(rng, (E, 2 * I, d // 2))
    out["w13_sc"] = _scales(rng, (E, 2 * I, d // 32))
    out["w2_qs"] = _qs(rng, (E, d, I // 2))
    out["w2_sc"] = _scales(rng, (E, d, I // 32))
    out["s13_qs"] = _qs(rng, (2 * Is, d // 2))
    out["s13_sc"] = _scales(rng, (2 * Is, d // 32))
    out["s2_qs"] = _qs(rng, (d, Is // 2))
    out["s2_sc"] = _scales(rng, (d, Is // 32))
    return out
