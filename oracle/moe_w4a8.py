"""Plain CPU oracle of the fp8-activation variants of the layer: W4A8 (MXFP4 expert weights times FP8
activations) and W8A8 (MXFP8 expert weights times FP8 activations).

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and the CPU baseline leg of
``bench.py`` may import or call this module.  It shares no code with the HIP library.

What it computes, and where the pages say so
--------------------------------------------
[nemotron] thewafflehaus/FFAI pull request 72 ("Nemotron-Nano-30B GB10 prefill quality + speed
    wins"): W4A8 (fp8 activations times fp4 weights) and W8A8 grouped MoE paths beside the Q4
    W4A16 kernel; the fp4 MoE weights there are Q4 weights requantised to a block-scaled fp4 grid
    (a different-but-valid grid, so the deeper reference outputs move), and the fp8 activations
    carry a per-token scale folded back after the product (per-token-act FP8 with the scales
    applied to the GEMM output).

The same page pairs a W8A8 path (fp8 activations times fp8 weights), argmax-exact on its prefill
with near-lossless fp8 weights.

Readings taken where the pages are silent (stated in the repository's design notes too):
  * fp4 means e2m1 (1 sign, 2 exponent, 1 mantissa bit, exponent bias 1; no inf or NaN): the
    values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives, in blocks of 32 sharing a power-of-two
    scale 2^E stored as an 8-bit biased exponent (E + 127); this is the block format the MI355X's
    scaled MFMA consumes, the same shape as a Q4 block;
  * the requantisation of a Q4 block (values w_i = (q_i - 8) * d) takes the shared exponent
    E = floor(log2(max_i |w_i|)) - 2 (2 being the largest exponent of an e2m1 value), the element
    codes round w_i / 2^E to the nearest e2m1 value (ties to the even mantissa) and saturate at +-6;
    an all-zero block gets E = -127 and zero codes;
  * fp8 means e4m3 (4 exponent bits, bias 7, 3 mantissa bits; largest finite 448, no inf); an
    activation row is scaled by s = amax / 448 (float32 division; s = 1 for an all-zero row), each
    element becomes the e4m3 value nearest to fl32(x / s) (ties to the even mantissa, saturating at
    +-448), and the row's product is multiplied back by s;
  * W8A8's fp8 weights are the Q4 blocks requantised to MXFP8: e4m3 elements in the same blocks of 32
    with a shared 2^E, E = floor(log2(max_i |w_i|)) - 8 (8 being the largest exponent of an e4m3
    value), elements w_i / 2^E rounded to the nearest e4m3 value (ties to even, saturating at +-448),
    E = -127 for an all-zero block;
  * the gate+up result h = silu(g) * u is rounded to fp16 (saturating at +-65504, as on the W4A16
    path) before its own per-row fp8 quantisation for the down projection;
  * routing (router, selection, weights) and the combine order are those of the W4A16 layer.
Everything else is evaluated in float64.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import (bf16_bits_to_f64, fp16_bits_to_f64, router_logits, select_experts, routing_weights,
                         sigmoid)

__all__ = ["e2m1_value", "e4m3_value", "round_e2m1", "round_e4m3", "mx_requant", "mx_dequant",
           "mx8_requant", "mx8_dequant", "quant_rows_fp8", "dequant_rows_fp8", "forward_w4a8", "forward_w8a8",
           "E4M3_MAX", "FP16_MAX"]

E4M3_MAX = 448.0
FP16_MAX = 65504.0


# ----------------------------------------------------------------------------- element formats

def e2m1_value(code) -> np.ndarray:
    """e2m1 code (low 4 bits) -> value: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
    exponent 0 is subnormal (0.5 * mantissa)."""
    c = np.asarray(code, dtype=np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(s == 1, -mag, mag)


def e4m3_value(code) -> np.ndarray:
    """e4m3 code (8 bits) -> value: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
    exponent 0 is subnormal (mantissa/8 * 2^-6); code 0x7F / 0xFF (NaN) is never produced here."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where(s == 1, -mag, mag)


def _round_to_grid(v, codes: np.ndarray, values: np.ndarray, max_mag: float) -> np.ndarray:
    """Nearest grid value to each v (ties to the code with the even mantissa bit, i.e. even code),
    magnitudes above max_mag saturating to it; returns codes.  `codes`/`values` list the
    non-negative half of the grid in increasing order; the sign is applied afterwards."""
    v = np.asarray(v, dtype=np.float64)
    mag = np.minimum(np.abs(v), max_mag)
    idx = np.searchsorted(values, mag)            # values[idx-1] < mag <= values[idx]
    idx = np.clip(idx, 1, len(values) - 1)
    lo, hi = values[idx - 1], values[idx]
    take_hi = (mag - lo > hi - mag) | ((mag - lo == hi - mag) & ((codes[idx] & 1) == 0))
    out = np.where(mag <= values[0], codes[0], np.where(take_hi, codes[idx], codes[idx - 1]))
    return out, np.signbit(v)


_E2M1_CODES = np.arange(8)
_E2M1_VALUES = e2m1_value(_E2M1_CODES)
_E4M3_CODES = np.arange(0x7F)          # 0x00 .. 0x7E (0x7F is NaN)
_E4M3_VALUES = e4m3_value(_E4M3_CODES)


def round_e2m1(v) -> np.ndarray:
    """Nearest e2m1 code to v (ties to even mantissa), saturating at +-6.  -0 keeps its sign bit."""
    c, neg = _round_to_grid(v, _E2M1_CODES, _E2M1_VALUES, 6.0)
    return (c | np.where(neg, 8, 0)).astype(np.uint8)


def round_e4m3(v) -> np.ndarray:
    """Nearest e4m3 code to v (ties to even mantissa), saturating at +-448."""
    c, neg = _round_to_grid(v, _E4M3_CODES, _E4M3_VALUES, E4M3_MAX)
    return (c | np.where(neg, 0x80, 0)).astype(np.uint8)


# ----------------------------------------------------------------------------- requantisation

def _q4_values(qs: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Row-major Q4 (uint8 [rows, K/2], fp16 bits [rows, K/32]) -> the values (q - 8) * d, float64."""
    qs = np.asarray(qs, dtype=np.uint8)
    rows, half = qs.shape
    q = np.empty((rows, 2 * half), dtype=np.int64)
    q[:, 0::2] = qs & 0x0F
    q[:, 1::2] = qs >> 4
    d = fp16_bits_to_f64(scales)
    return (q - 8).astype(np.float64) * np.repeat(d, 32, axis=1)


def mx_requant(qs: np.ndarray, scales: np.ndarray):
    """Q4 block matrix (row-major: uint8 [rows, K/2], fp16 bits [rows, K/32]) -> MXFP4.

    Returns (codes uint8 [rows, K/2], element 2i in the low nibble of byte i as in the Q4 format;
    exp uint8 [rows, K/32], the biased shared exponent E + 127 of each 32-element block)."""
    w = _q4_values(qs, scales)
    rows, K = w.shape
    wb = w.reshape(rows, K // 32, 32)
    amax = np.abs(wb).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127).astype(np.int64)
    e = np.clip(e, -127, 127)
    v = wb / np.ldexp(1.0, e)[:, :, None]
    c = round_e2m1(v).reshape(rows, K).astype(np.uint8)
    codes = (c[:, 0::2] & 0x0F) | ((c[:, 1::2] & 0x0F) << 4)
    return codes.astype(np.uint8), (e + 127).astype(np.uint8)


def mx_dequant(codes: np.ndarray, exp: np.ndarray) -> np.ndarray:
    """MXFP4 (codes [rows, K/2], biased exponents [rows, K/32]) -> float64 [rows, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    c = np.empty((rows, 2 * half), dtype=np.int64)
    c[:, 0::2] = codes & 0x0F
    c[:, 1::2] = codes >> 4
    scale = np.ldexp(1.0, np.asarray(exp, dtype=np.int64) - 127)
    return e2m1_value(c) * np.repeat(scale, 32, axis=1)


def mx8_requant(qs: np.ndarray, scales: np.ndarray):
    """Q4 block matrix (row-major: uint8 [rows, K/2], fp16 bits [rows, K/32]) -> MXFP8.

    Returns (codes uint8 [rows, K], e4m3 element k of the row at byte k; exp uint8 [rows, K/32], the
    biased shared exponent E + 127 of each 32-element block)."""
    w = _q4_values(qs, scales)
    rows, K = w.shape
    wb = w.reshape(rows, K // 32, 32)
    amax = np.abs(wb).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127).astype(np.int64)
    e = np.clip(e, -127, 127)
    codes = round_e4m3(wb / np.ldexp(1.0, e)[:, :, None]).reshape(rows, K)
    return codes.astype(np.uint8), (e + 127).astype(np.uint8)


def mx8_dequant(codes: np.ndarray, exp: np.ndarray) -> np.ndarray:
    """MXFP8 (codes [rows, K], biased exponents [rows, K/32]) -> float64 [rows, K]."""
    scale = np.ldexp(1.0, np.asarray(exp, dtype=np.int64) - 127)
    return e4m3_value(codes) * np.repeat(scale, 32, axis=1)


# ----------------------------------------------------------------------------- activations

def quant_rows_fp8(X) -> tuple[np.ndarray, np.ndarray]:
    """Rows of float32 values -> (e4m3 codes uint8 [n, K], float32 row scales [n]).

    s = fl32(amax / 448) (1 for an all-zero row); code = nearest e4m3 to fl32(x / s)."""
    X = np.asarray(X, dtype=np.float32)
    amax = np.abs(X).max(axis=1)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (X / s[:, None]).astype(np.float32)
    return round_e4m3(q.astype(np.float64)), s


def dequant_rows_fp8(codes, s) -> np.ndarray:
    return e4m3_value(codes) * np.asarray(s, dtype=np.float64)[:, None]


def _fp16_sat(v):
    """fp16 rounding (nearest even) with saturation at +-65504."""
    return np.clip(np.asarray(v, dtype=np.float64), -FP16_MAX, FP16_MAX).astype(np.float16).astype(np.float64)


def _mlp_w4a8(Xq: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """One expert on fp8-quantised rows Xq (float64 values): h = fp16(silu(g) * u), h quantised per
    row to fp8, then the down projection."""
    I = w13.shape[0] // 2
    g = Xq @ w13[:I].T
    u = Xq @ w13[I:].T
    h = _fp16_sat(g * sigmoid(g) * u)
    hq = dequant_rows_fp8(*quant_rows_fp8(h.astype(np.float32)))
    return hq @ w2.T


def _forward_fp8act(inp: dict, tokens, ids_override, mx, requant, dequant) -> dict:
    dims = inp["dims"]
    k, d = dims.k, dims.d
    tokens = np.arange(dims.T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    xb = inp["x"][tokens]
    s = sigmoid(router_logits(xb, inp["w_router"]))
    ids, margin = select_experts(s, inp["bias"], k)
    if ids_override:
        pos = {int(t): i for i, t in enumerate(tokens)}
        for t, sel in ids_override.items():
            ids[pos[int(t)]] = np.asarray(sel, dtype=np.int32)
    w = routing_weights(s, ids)
    x = bf16_bits_to_f64(xb).astype(np.float32)
    xq = dequant_rows_fp8(*quant_rows_fp8(x))

    def mat(name, e=None):
        if mx is not None and (name, e) in mx:
            return dequant(*mx[(name, e)])
        qs = inp[name + "_qs"] if e is None else inp[name + "_qs"][e]
        sc = inp[name + "_sc"] if e is None else inp[name + "_sc"][e]
        return dequant(*requant(qs, sc))

    n = len(tokens)
    y_routed = np.zeros((n, d))
    for e in np.unique(ids):
        rows, slots = np.nonzero(ids == e)
        Y = _mlp_w4a8(xq[rows], mat("w13", e), mat("w2", e))
        y_routed[rows] += w[rows, slots][:, None] * Y
    y_shared = _mlp_w4a8(xq, mat("s13"), mat("s2"))
    return dict(y=y_routed + y_shared, ids=ids, w=w, margin=margin, tokens=tokens)


def forward_w4a8(inp: dict, tokens=None, ids_override: dict | None = None, mx: dict | None = None) -> dict:
    """The W4A8 layer for the chosen tokens (all by default), same routing as the W4A16 layer.

    mx: optional precomputed {(name, e): (codes, exp)} of mx_requant for w13/w2 per expert and s13/s2
    (e None; computed here when absent).  Returns dict(y [n,d], ids, w, margin, tokens)."""
    return _forward_fp8act(inp, tokens, ids_override, mx, mx_requant, mx_dequant)


def forward_w8a8(inp: dict, tokens=None, ids_override: dict | None = None, mx: dict | None = None) -> dict:
    """The W8A8 layer: as forward_w4a8 with MXFP8 weights (mx8_requant; `mx` holds its outputs)."""
    return _forward_fp8act(inp, tokens, ids_override, mx, mx8_requant, mx8_dequant)
