"""Plain fp64 CPU oracle of the sigmoid-routed Q4 MoE expert layer.

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import or call this module.  It shares no
code with the HIP library and imports nothing from it.

What it computes, and where the pages say so
--------------------------------------------
[decode] thewafflehaus/butter pull request 69, commit "feat(laguna):
    Laguna-S-2.1 decode on the CUDA engine": the hybrid MoE routes each token
    with a sigmoid top-10 router carrying a score-correction bias, adds a
    shared expert, loads Q4-requantised expert weights, and runs the experts
    as gathered Q4 GEMVs (a plain one and one fused with SwiGLU), with gate
    and up fused.
[prefill] same pull request (and thewafflehaus/FFAI pull request 70),
    commit "feat(laguna): batched prefill with tensor-core projections,
    fused MoE, CTA scheduling": grouped-GEMM MoE with descriptors built on
    the device and fused gate+up expert stacks.
[nemotron] thewafflehaus/FFAI pull request 72, the Nemotron MoE commits:
    routing kept as CSR offsets plus router-sorted token indices with the
    expert id of every sorted row expanded from the offsets, a deterministic
    (non-atomic) scatter-add of the per-pair expert outputs, and the
    "ffai_add3" commit, where routed and shared outputs are summed first
    because the other order changed an argmax.

Readings taken where the pages are silent:
  * router logits l = x . W_r^T, no router bias term, no temperature; s = 1/(1+exp(-l));
  * the score-correction bias b is added to s for *selection only*: key = s + b;
  * the k experts with the largest key are chosen, ties going to the lower
    expert index, listed by descending key;
  * routing weights are the unbiased scores of the chosen experts normalised
    to sum to 1 (routed scaling factor 1);
  * expert MLP is SwiGLU: h = silu(x W_g^T) * (x W_u^T), silu(z) = z/(1+exp(-z)),
    y_e = h W_d^T; in the fused gate+up stack the gate rows come first;
  * the shared expert is always on and added with weight 1;
  * layer output y[t] = sum_j w[t,j] * y_{e_tj}(x_t)  +  shared(x_t)  (no residual);
  * Q4 block format: a row of K values is K/32 blocks; value = (q - 8) * d with
    q the 4-bit code and d the block's fp16 scale; byte i of a row holds
    element 2i in its low nibble and element 2i+1 in its high nibble.

Everything is evaluated in float64.  bf16 and fp16 inputs convert exactly.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "fp16_bits_to_f64", "dequant_q4",
    "router_logits", "sigmoid", "select_experts", "routing_weights",
    "swiglu_mlp", "forward", "routing_build", "group_order",
    "f64_to_bf16_bits", "decode_chain", "rms_norm",
]


# ----------------------------------------------------------------------------- formats

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.  A bf16 value is the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), rounding to nearest with ties to even.

    bf16 is float32 with the low 16 bits dropped: 8 exponent bits and 7
    fraction bits.  The value is rounded once, straight from float64, by
    comparing it with the two neighbouring bf16 values.  NaN -> 0x7FC0.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    flat_v, flat_o = v.ravel(), out.ravel()
    for i, x in enumerate(flat_v):
        if np.isnan(x):
            flat_o[i] = 0x7FC0
            continue
        # candidates: truncate the float32 nearest below |x|, and the next bf16 up
        lo = int(np.array(np.float32(min(abs(x), 3.4028234663852886e38))).view(np.uint32)) >> 16
        while lo > 0 and bf16_bits_to_f64(np.uint16(lo))[()] > abs(x):
            lo -= 1
        hi = lo + 1
        vlo = bf16_bits_to_f64(np.uint16(lo))[()]
        # above the largest finite bf16 the next step up is 2^128, which is infinity
        vhi = bf16_bits_to_f64(np.uint16(hi))[()] if hi < 0x7F80 else 2.0 ** 128
        if abs(x) == np.inf:
            m = 0x7F80
        elif abs(x) - vlo < vhi - abs(x):
            m = lo
        elif abs(x) - vlo > vhi - abs(x):
            m = hi
        else:
            m = lo if lo % 2 == 0 else hi
        flat_o[i] = m | (0x8000 if np.signbit(x) else 0)
    return out


def fp16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequant_q4(qs: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Q4 block matrix -> float64 [rows, K].

    qs: uint8 [rows, K/2]; scales: fp16 bits [rows, K/32].  Element 2i of a
    row is the low nibble of byte i, element 2i+1 the high nibble, and every
    value is (q - 8) times the fp16 scale of its 32-element block ([decode]:
    Q4-requantised weights; the nibble order and offset are this library's
    stated format).
    """
    qs = np.asarray(qs, dtype=np.uint8)
    rows, half = qs.shape
    K = 2 * half
    if scales.shape != (rows, K // 32):
        raise ValueError("scale array does not match the code array")
    q = np.empty((rows, K), dtype=np.int16)
    q[:, 0::2] = qs & 0x0F
    q[:, 1::2] = qs >> 4
    d = fp16_bits_to_f64(scales)
    return (q.astype(np.float64) - 8.0) * np.repeat(d, 32, axis=1)


# ----------------------------------------------------------------------------- router

def router_logits(x_bits: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """l[t, e] = sum_c x[t, c] * W_r[e, c], in fp64 ([decode]: the router scores every expert)."""
    x = bf16_bits_to_f64(x_bits)
    return x @ np.asarray(w_router, dtype=np.float64).T


def sigmoid(z: np.ndarray) -> np.ndarray:
    """Logistic function 1 / (1 + exp(-z)) ([decode]: a sigmoid, not a softmax, router)."""
    return 1.0 / (1.0 + np.exp(-z))


def select_experts(s: np.ndarray, bias: np.ndarray, k: int):
    """Biased top-k selection ([decode]: top-10 with a score-correction bias).

    key = s + b.  For every token the experts are ordered by (-key, e) with
    a stable sort, and the first k are taken.  Returns (ids [T,k] int32,
    margin [T]) where margin = key of the k-th choice minus key of the
    (k+1)-th (infinity when k == E).
    """
    key = s + np.asarray(bias, dtype=np.float64)[None, :]
    T, E = key.shape
    ids = np.empty((T, k), dtype=np.int32)
    margin = np.full(T, np.inf)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-key[t, e], e))
        ids[t] = order[:k]
        if k < E:
            margin[t] = key[t, order[k - 1]] - key[t, order[k]]
    return ids, margin


def routing_weights(s: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w[t, j] = s[t, ids[t,j]] / sum_j' s[t, ids[t,j']]: unbiased scores normalised to sum 1."""
    chosen = np.take_along_axis(s, np.asarray(ids, dtype=np.int64), axis=1)
    return chosen / chosen.sum(axis=1, keepdims=True)


# ----------------------------------------------------------------------------- experts

def swiglu_mlp(X: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """One expert on the rows of X ([decode]: fused gate+up SwiGLU, then the down projection).

    w13: fp64 [2I, d] with gate rows 0..I-1 and up rows I..2I-1; w2: fp64 [d, I].
    Returns (silu(X W_g^T) * (X W_u^T)) W_d^T.
    """
    I = w13.shape[0] // 2
    g = X @ w13[:I].T
    u = X @ w13[I:].T
    h = g * sigmoid(g) * u
    return h @ w2.T


def forward(inp: dict, tokens=None, ids_override: dict | None = None, residual=None) -> dict:
    """The whole layer for the chosen tokens (all tokens by default).

    inp: a dict as produced by the input generator (x bf16 bits, w_router,
    bias, w13_qs/w13_sc, w2_qs/w2_sc, s13_qs/s13_sc, s2_qs/s2_sc, dims).
    ids_override: {token: [k expert ids]} to evaluate the layer on a given
    selection (the weights still come from the fp64 scores).
    residual: optional fp32 [T,d]; added after the routed and shared sum
    ([nemotron], "ffai_add3": routed + shared first, then the residual).
    Returns dict(y [n,d] fp64, ids [n,k], w [n,k], margin [n], s [n,E], tokens).
    """
    dims = inp["dims"]
    E, k, d = dims.E, dims.k, dims.d
    tokens = np.arange(dims.T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    xb = inp["x"][tokens]
    x = bf16_bits_to_f64(xb)
    s = sigmoid(router_logits(xb, inp["w_router"]))
    ids, margin = select_experts(s, inp["bias"], k)
    if ids_override:
        pos = {int(t): i for i, t in enumerate(tokens)}
        for t, sel in ids_override.items():
            ids[pos[int(t)]] = np.asarray(sel, dtype=np.int32)
    w = routing_weights(s, ids)

    n = len(tokens)
    y_routed = np.zeros((n, d))
    # One expert at a time, its rows in token order ([prefill]: grouped by expert).
    for e in np.unique(ids):
        rows, slots = np.nonzero(ids == e)
        w13 = dequant_q4(inp["w13_qs"][e], inp["w13_sc"][e])
        w2 = dequant_q4(inp["w2_qs"][e], inp["w2_sc"][e])
        Y = swiglu_mlp(x[rows], w13, w2)
        y_routed[rows] += w[rows, slots][:, None] * Y
    s13 = dequant_q4(inp["s13_qs"], inp["s13_sc"])
    s2 = dequant_q4(inp["s2_qs"], inp["s2_sc"])
    y_shared = swiglu_mlp(x, s13, s2)
    # Routed sum first, then the shared expert ([nemotron], "ffai_add3"), then the residual if any.
    y = y_routed + y_shared
    if residual is not None:
        y = y + np.asarray(residual, dtype=np.float64)[tokens]
    return dict(y=y, ids=ids, w=w, margin=margin, s=s, tokens=tokens)


# ----------------------------------------------------------------------------- routing build

def routing_build(ids: np.ndarray, E: int) -> dict:
    """CSR grouping of the (token, slot) pairs by expert ([prefill], [nemotron]).

    Pair p = t*k + j.  Pairs are ordered by expert, and within an expert by
    pair id (a stable sort, so token order).  Returns
      counts[E], offsets[E+1] (exclusive prefix sums), sorted_pair[P] (pair at
      each sorted position), pair_pos[P] (inverse), row_expert[P] (expert of
      each sorted position).
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_pair = np.argsort(flat, kind="stable").astype(np.int32)
    pair_pos = np.empty_like(sorted_pair)
    pair_pos[sorted_pair] = np.arange(flat.size, dtype=np.int32)
    row_expert = flat[sorted_pair].astype(np.int32)
    return dict(counts=counts, offsets=offsets, sorted_pair=sorted_pair,
                pair_pos=pair_pos, row_expert=row_expert)


def group_order(counts: np.ndarray, T: int) -> np.ndarray:
    """Schedule order of the expert groups plus the shared expert (group id E, T rows).

    Descending group size, ties to the lower id ([prefill]: descending-size
    expert order).  Empty groups are kept, at the end.
    """
    c = np.concatenate([np.asarray(counts, dtype=np.int64), [T]])
    return np.array(sorted(range(c.size), key=lambda g: (-c[g], g)), dtype=np.int32)


# ----------------------------------------------------------------------------- pre-MoE norm

def rms_norm(h, gamma, eps: float) -> np.ndarray:
    """RMSNorm of each row: h / sqrt(mean(h^2) + eps) * gamma, in float64.

    The pages name RMSNorm (per-head QK RMSNorm in [decode]'s attention, a
    fused add-RMSNorm op) but never define the norm in front of the MoE
    block; this is the standard definition of RMSNorm (Zhang and Sennrich,
    2019), with the caller's per-channel gamma and eps.
    """
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + float(eps)) * np.asarray(gamma, dtype=np.float64)


# ----------------------------------------------------------------------------- multi-layer decode

def decode_chain(layers: list, h0) -> dict:
    """A residual stream through a stack of MoE layers, one after another.

    [decode] runs single-stream decode as one captured graph over every layer
    with a persistent workspace (the LagunaDecodeCtx of "feat(laguna):
    Laguna-S-2.1 decode on the CUDA engine"); between two MoE layers of the
    model sit attention and norms; attention is out of scope here, so each
    layer takes its input straight from the stream:
        x = bf16(h)                (round to nearest even; the layer's input is bf16)
        h = (routed + shared)(x) + h
    the residual added after the routed and shared sum ([nemotron], "ffai_add3").
    A layer dict with "norm_weight" (gamma [d]) and "norm_eps" takes its input
    through the pre-MoE norm instead: x = bf16(rms_norm(h, gamma, eps)).
    layers: input dicts as for forward() (their "x" is ignored); h0: [T,d].
    Returns dict(h [T,d] fp64, margins [L,T]: each layer's selection margin).
    """
    h = np.asarray(h0, dtype=np.float64)
    margins = []
    for inp in layers:
        lay = dict(inp)
        if inp.get("norm_weight") is not None:
            lay["x"] = f64_to_bf16_bits(rms_norm(h, inp["norm_weight"], inp["norm_eps"]))
        else:
            lay["x"] = f64_to_bf16_bits(h)
        out = forward(lay, residual=h)
        h = out["y"]
        margins.append(out["margin"])
    return dict(h=h, margins=np.array(margins))
