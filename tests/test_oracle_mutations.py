"""Planted mistakes in the oracle, on the CPU: each must make at least one named pin of
tests/test_oracle.py fail.  This shows the pins constrain every part of the oracle a plausible
slip could touch (nibble order, code offset, the tie rule of the selection and of the group
schedule, bias leaking into the weights, gate/up order, the SiLU argument, the shared expert,
a transposed down projection, an unstable routing sort).

Each mutation replaces one oracle function (in the module and in the package namespace) for the
duration of one pin, then restores it.  Nothing here touches the GPU library.
"""
import numpy as np
import pytest

import oracle
import oracle.moe_oracle as om
import test_oracle as pins


def _dequant_nibbles_swapped(qs, scales):
    qs = np.asarray(qs, dtype=np.uint8)
    rows, half = qs.shape
    q = np.empty((rows, 2 * half), dtype=np.int16)
    q[:, 0::2] = qs >> 4          # slip: high nibble taken as the even element
    q[:, 1::2] = qs & 0x0F
    return (q - 8.0) * np.repeat(om.fp16_bits_to_f64(scales), 32, axis=1)


def _dequant_offset_7(qs, scales):
    return om.dequant_q4(qs, scales) + np.repeat(om.fp16_bits_to_f64(scales), 32, axis=1)  # (q - 7) * d


def _select_ties_to_higher_id(s, bias, k):
    key = s + np.asarray(bias, dtype=np.float64)[None, :]
    T, E = key.shape
    ids = np.empty((T, k), dtype=np.int32)
    margin = np.full(T, np.inf)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-key[t, e], -e))
        ids[t] = order[:k]
        if k < E:
            margin[t] = key[t, order[k - 1]] - key[t, order[k]]
    return ids, margin


def _weights_from_biased_key(s, ids):
    # slip: the score-correction bias leaks into the weights (the only bias in scope is the one
    # forward() passes to select_experts; rebuild the biased keys from the pin's own setup)
    chosen = np.take_along_axis(s, np.asarray(ids, dtype=np.int64), axis=1) + 3.0
    return chosen / chosen.sum(axis=1, keepdims=True)


def _mlp_gate_up_swapped(X, w13, w2):
    I = w13.shape[0] // 2
    u = X @ w13[:I].T
    g = X @ w13[I:].T
    return (g * om.sigmoid(g) * u) @ w2.T


def _mlp_silu_sign(X, w13, w2):
    I = w13.shape[0] // 2
    g = X @ w13[:I].T
    u = X @ w13[I:].T
    return (g * om.sigmoid(-g) * u) @ w2.T


def _mlp_down_transposed(X, w13, w2):
    I = w13.shape[0] // 2
    g = X @ w13[:I].T
    u = X @ w13[I:].T
    h = g * om.sigmoid(g) * u
    return h @ w2[:I, :I] if w2.shape[0] != w2.shape[1] else h @ w2


def _group_order_ties_to_higher_id(counts, T):
    c = np.concatenate([np.asarray(counts, dtype=np.int64), [T]])
    return np.array(sorted(range(c.size), key=lambda g: (-c[g], -g)), dtype=np.int32)


def _group_order_shared_first(counts, T):
    c = np.asarray(counts, dtype=np.int64)
    rest = sorted(range(c.size), key=lambda g: (-c[g], g))
    return np.array([c.size] + rest, dtype=np.int32)


def _routing_build_reverse_within_expert(ids, E):
    r = om.routing_build(ids, E)
    flat = np.asarray(ids, dtype=np.int64).ravel()
    sp = np.array(sorted(range(flat.size), key=lambda p: (flat[p], -p)), dtype=np.int32)
    r = dict(r, sorted_pair=sp)
    r["pair_pos"] = np.empty_like(sp)
    r["pair_pos"][sp] = np.arange(flat.size, dtype=np.int32)
    return r


_real_forward = om.forward


def _forward_without_shared(inp, tokens=None, ids_override=None, residual=None):
    zero = dict(inp)
    zero["s13_qs"] = np.full_like(inp["s13_qs"], 0x88)
    zero["s2_qs"] = np.full_like(inp["s2_qs"], 0x88)
    return _real_forward(zero, tokens=tokens, ids_override=ids_override, residual=residual)


# (mutated function, replacement, the pins that must catch it)
MUTATIONS = {
    "nibble_swap": ("dequant_q4", _dequant_nibbles_swapped, ["test_q4_golden_blocks"]),
    "offset_7": ("dequant_q4", _dequant_offset_7, ["test_q4_golden_blocks", "test_selection_matrices_non_square"]),
    "select_ties_high": ("select_experts", _select_ties_to_higher_id, ["test_select_experts_brute_force"]),
    "bias_in_weights": ("routing_weights", _weights_from_biased_key, ["test_routing_weights_closed_form"]),
    "gate_up_swap": ("swiglu_mlp", _mlp_gate_up_swapped, ["test_selection_matrices_non_square"]),
    "silu_sign": ("swiglu_mlp", _mlp_silu_sign, ["test_single_expert_identity_closed_form"]),
    "down_transposed": ("swiglu_mlp", _mlp_down_transposed, ["test_selection_matrices_non_square"]),
    "dropped_shared": ("forward", _forward_without_shared, ["test_single_expert_identity_closed_form"]),
    "group_ties_high": ("group_order", _group_order_ties_to_higher_id, ["test_group_order_ties_go_to_the_lower_id"]),
    "group_shared_first": ("group_order", _group_order_shared_first, ["test_group_order_ties_go_to_the_lower_id"]),
    "unstable_build": ("routing_build", _routing_build_reverse_within_expert, ["test_routing_build_bruteforce"]),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    fn, repl, catching = MUTATIONS[name]
    # every pin passes on the real oracle (run first, so a failure below is the mutation's doing)
    for pin in catching:
        getattr(pins, pin)()
    monkeypatch.setattr(om, fn, repl)
    monkeypatch.setattr(oracle, fn, repl)
    caught = []
    for pin in catching:
        try:
            getattr(pins, pin)()
        except Exception:  # an assertion, or a shape error from a transposed operand
            caught.append(pin)
    assert caught, f"mutation {name} of oracle.{fn} passed every pin it should fail: {catching}"


# ----------------------------------------------------------------------------- the fp8-activation oracle

import oracle.moe_w4a8 as ow  # noqa: E402
import test_oracle_w4a8 as pins8  # noqa: E402

_real_mx_requant, _real_mx8_requant, _real_round_e4m3 = ow.mx_requant, ow.mx8_requant, ow.round_e4m3


def _mx_requant_exponent_high(qs, scales):
    codes, exp = _real_mx_requant(qs, scales)       # slip: E = floor(log2 amax) - 1
    w = ow._q4_values(qs, scales)
    rows, K = w.shape
    wb = w.reshape(rows, K // 32, 32)
    e = exp.astype(np.int64) - 127 + 1
    c = ow.round_e2m1(wb / np.ldexp(1.0, e)[:, :, None]).reshape(rows, K)
    return ((c[:, 0::2] & 15) | ((c[:, 1::2] & 15) << 4)).astype(np.uint8), (e + 127).astype(np.uint8)


def _mx_requant_nibbles_swapped(qs, scales):
    codes, exp = _real_mx_requant(qs, scales)
    return ((codes >> 4) | ((codes & 15) << 4)).astype(np.uint8), exp


def _mx8_requant_exponent_low(qs, scales):
    w = ow._q4_values(qs, scales)                    # slip: E = floor(log2 amax) - 7 (too coarse)
    rows, K = w.shape
    wb = w.reshape(rows, K // 32, 32)
    _, exp = _real_mx8_requant(qs, scales)
    e = exp.astype(np.int64) - 127 + 1
    return ow.round_e4m3(wb / np.ldexp(1.0, e)[:, :, None]).reshape(rows, K).astype(np.uint8), (e + 127).astype(np.uint8)


def _round_e4m3_ties_away(v):
    v = np.asarray(v, dtype=np.float64)
    c = _real_round_e4m3(v)
    # slip: a value exactly halfway between two codes goes to the larger magnitude
    lo = ow.e4m3_value(c & 0x7F)
    nxt = ow.e4m3_value(np.minimum((c & 0x7F) + 1, 0x7E))
    half = np.abs(np.abs(v) - (lo + nxt) / 2) == 0
    return np.where(half & ((c & 0x7F) < 0x7E), c + 1, c).astype(np.uint8)


def _quant_rows_unscaled(X):
    X = np.asarray(X, dtype=np.float32)              # slip: no per-row scale
    return ow.round_e4m3(X.astype(np.float64)), np.ones(X.shape[0], dtype=np.float32)


MUTATIONS_FP8 = {
    "mx_exponent_high": ("mx_requant", _mx_requant_exponent_high, ["test_requant_hand_worked_block"]),
    "mx_nibbles_swapped": ("mx_requant", _mx_requant_nibbles_swapped, ["test_requant_hand_worked_block"]),
    "mx8_exponent_low": ("mx8_requant", _mx8_requant_exponent_low, ["test_mx8_requant_hand_worked_block",
                                                                     "test_mx8_requant_power_of_two_scales_are_exact"]),
    "e4m3_ties_away": ("round_e4m3", _round_e4m3_ties_away, ["test_e4m3_rounding"]),
    "quant_rows_unscaled": ("quant_rows_fp8", _quant_rows_unscaled, ["test_quant_rows_fp8"]),
}


def _run_pin(pin):
    """Run one pin; a parametrized pin runs every one of its cases."""
    fn = getattr(pins8, pin)
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    if not marks:
        return fn()
    for case in marks[0].args[1]:
        fn(*case)


@pytest.mark.parametrize("name", list(MUTATIONS_FP8))
def test_planted_mistake_in_the_fp8_oracle_fails_a_pin(name, monkeypatch):
    fn, repl, catching = MUTATIONS_FP8[name]
    for pin in catching:
        _run_pin(pin)
    monkeypatch.setattr(ow, fn, repl)
    caught = []
    for pin in catching:
        try:
            _run_pin(pin)
        except Exception:
            caught.append(pin)
    assert caught, f"mutation {name} of oracle.moe_w4a8.{fn} passed every pin it should fail: {catching}"
