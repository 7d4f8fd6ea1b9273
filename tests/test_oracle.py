"""Pins for the fp64 oracle: hand-built values, closed forms, brute force.

Each test fixes the oracle to something other than itself, chosen so that a
plausible slip (swapped nibbles, a dropped offset, bias leaking into the
weights, gate/up swapped, a transposed matrix, a lost shared term, the wrong
tie rule) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers

def pack_q4(q: np.ndarray) -> np.ndarray:
    """Test-side packer written from the format definition: byte i = q[2i] | q[2i+1] << 4."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def fp16_bits(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float16).view(np.uint16)


def q4_from_values(vals: np.ndarray, scale: float = 1.0):
    """Integer-valued matrix with entries in [-8, 7] -> (qs, scales) with a uniform scale."""
    vals = np.asarray(vals)
    assert vals.min() >= -8 and vals.max() <= 7
    rows, K = vals.shape
    q = (vals + 8).astype(np.uint8)
    return pack_q4(q), np.full((rows, K // 32), fp16_bits(scale), dtype=np.uint16)


def layer(dims, x_f32, w_router, bias, w13, w2, s13, s2):
    """Assemble an input dict from integer-valued weight matrices (unit scales)."""
    E = dims.E
    w13_qs, w13_sc = zip(*[q4_from_values(w13[e]) for e in range(E)])
    w2_qs, w2_sc = zip(*[q4_from_values(w2[e]) for e in range(E)])
    s13_qs, s13_sc = q4_from_values(s13)
    s2_qs, s2_sc = q4_from_values(s2)
    return dict(
        dims=dims, x=synth.bf16_bits_from_f32(np.asarray(x_f32, dtype=np.float32)),
        w_router=np.asarray(w_router, dtype=np.float32), bias=np.asarray(bias, dtype=np.float32),
        w13_qs=np.stack(w13_qs), w13_sc=np.stack(w13_sc), w2_qs=np.stack(w2_qs), w2_sc=np.stack(w2_sc),
        s13_qs=s13_qs, s13_sc=s13_sc, s2_qs=s2_qs, s2_sc=s2_sc,
    )


def x_values(inp):
    """The bf16 inputs as float64, decoded here from the bit layout (top half of a float32)."""
    u = inp["x"].astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- Q4 format

def test_q4_golden_blocks():
    g = json.load(open(os.path.join(GOLDEN, "q4_blocks.json")))
    for case in g["cases"]:
        qs = np.frombuffer(bytes.fromhex(case["qs_hex"]), dtype=np.uint8)[None, :]
        sc = np.array([[int(case["scale_fp16_hex"], 16)]], dtype=np.uint16)
        w = oracle.dequant_q4(qs, sc)
        np.testing.assert_array_equal(w[0], np.array(case["expected"], dtype=np.float64), err_msg=case["name"])


def test_q4_scale_extremes_exact():
    q = np.arange(32) % 16
    qs = pack_q4(q[None, :])
    for bits, val in [(0x3C00, 1.0), (0x0400, 2.0 ** -14), (0x0001, 2.0 ** -24), (0x7BFF, 65504.0), (0xBC00, -1.0)]:
        w = oracle.dequant_q4(qs, np.array([[bits]], dtype=np.uint16))
        np.testing.assert_array_equal(w[0], (q - 8) * val)


def test_q4_per_block_and_per_row_scales():
    rng = np.random.default_rng(5)
    rows, K = 3, 128
    q = rng.integers(0, 16, size=(rows, K))
    scales = np.array([[1.0, 0.5, 2.0, 0.25], [4.0, 1.0, 0.125, 8.0], [0.0625, 16.0, 1.0, 2.0]])
    w = oracle.dequant_q4(pack_q4(q), fp16_bits(scales))
    for r in range(rows):
        for b in range(K // 32):
            np.testing.assert_array_equal(w[r, 32 * b:32 * b + 32], (q[r, 32 * b:32 * b + 32] - 8) * scales[r, b])


def test_q4_roundtrip_random_bytes():
    rng = np.random.default_rng(6)
    qs = rng.integers(0, 256, size=(7, 64), dtype=np.uint8)
    w = oracle.dequant_q4(qs, np.full((7, 4), 0x3C00, dtype=np.uint16))
    q_back = (w + 8).astype(np.uint8)
    np.testing.assert_array_equal(pack_q4(q_back), qs)


def test_bf16_and_fp16_decode():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x7F7F, 0x0001], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(bits),
                                  [1.0, -2.0, 0.0, 3.3895313892515355e38, 2.0 ** -133])
    np.testing.assert_array_equal(oracle.fp16_bits_to_f64(np.array([0x3C00, 0x2C00, 0x7BFF], dtype=np.uint16)),
                                  [1.0, 0.0625, 65504.0])


# ----------------------------------------------------------------------------- router

def test_sigmoid_closed_forms():
    np.testing.assert_allclose(oracle.sigmoid(np.array([0.0, math.log(3), -math.log(3), math.log(9)])),
                               [0.5, 0.75, 0.25, 0.9], rtol=0, atol=1e-15)


def brute_topk(key_row, k):
    E = len(key_row)
    best = None
    # every k-subset, ordered; the chosen set must dominate all others lexicographically
    order = sorted(range(E), key=lambda e: (-key_row[e], e))
    for comb in itertools.combinations(range(E), k):
        srt = sorted(comb, key=lambda e: (-key_row[e], e))
        cand = [(-key_row[e], e) for e in srt]
        if best is None or cand < best[0]:
            best = (cand, srt)
    assert best[1] == order[:k]
    return best[1]


def test_select_experts_brute_force():
    rng = np.random.default_rng(7)
    T, E, k = 40, 9, 3
    s = rng.uniform(size=(T, E))
    b = rng.uniform(-0.2, 0.2, size=E)
    # force some exact ties in the key
    s[0, 2] = s[0, 5] = 0.99
    b[2] = b[5] = 0.3  # key 1.29, above every other key (at most 1.2)
    ids, margin = oracle.select_experts(s, b, k)
    key = s + b
    for t in range(T):
        assert list(ids[t]) == brute_topk(list(key[t]), k)
        rest = sorted(set(range(E)) - set(ids[t]), key=lambda e: (-key[t, e], e))
        assert margin[t] == pytest.approx(key[t, ids[t, -1]] - key[t, rest[0]], abs=0)
    assert list(ids[0][:2]) == [2, 5]  # tie -> lower index first


def test_zero_bias_is_topk_of_logits():
    inp = synth.make_inputs(synth.Dims(T=16, d=64, E=12, k=4, I=32, I_shared=32), seed=3, bias="zero", weights=False)
    l = oracle.router_logits(inp["x"], inp["w_router"])
    ids, _ = oracle.select_experts(oracle.sigmoid(l), inp["bias"], 4)
    ref = np.argsort(-l, axis=1, kind="stable")[:, :4]
    np.testing.assert_array_equal(ids, ref)


def test_bias_dominance():
    inp = synth.make_inputs(synth.Dims(T=32, d=64, E=10, k=3, I=32, I_shared=32), seed=4, weights=False)
    S = [1, 6, 8]
    b = np.zeros(10)
    b[S] = 10.0
    s = oracle.sigmoid(oracle.router_logits(inp["x"], inp["w_router"]))
    ids, margin = oracle.select_experts(s, b, 3)
    for t in range(32):
        assert sorted(ids[t]) == S
        assert margin[t] > 9.0


def test_routing_weights_closed_form():
    # One input direction; W_r rows put chosen logits on it: l = [0, ln3, -ln3, 5, 5, ...]
    dims = synth.Dims(T=1, d=32, E=6, k=2, I=32, I_shared=32)
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 1.0
    wr = np.zeros((6, 32), dtype=np.float64)
    wr[:, 0] = [0.0, math.log(3), -math.log(3), 5.0, 5.0, 5.0]
    # the bias selects experts 0 and 1, whose scores are 0.5 and 0.75
    bias = np.array([3.0, 3.0, 0.0, 0.0, 0.0, 0.0])
    s = oracle.sigmoid(oracle.router_logits(synth.bf16_bits_from_f32(x), wr.astype(np.float32)))
    ids, _ = oracle.select_experts(s, bias, 2)
    assert list(ids[0]) == [1, 0]  # keys 3.75, 3.5
    w = oracle.routing_weights(s, ids)
    np.testing.assert_allclose(w[0], [0.6, 0.4], rtol=0, atol=2e-8)  # 0.75/1.25, 0.5/1.25


def test_weights_sum_to_one_and_k1():
    inp = synth.make_inputs(synth.CONFIGS["tiny"], weights=False)
    s = oracle.sigmoid(oracle.router_logits(inp["x"], inp["w_router"]))
    ids, _ = oracle.select_experts(s, inp["bias"], 4)
    w = oracle.routing_weights(s, ids)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(w > 0)
    ids1, _ = oracle.select_experts(s, inp["bias"], 1)
    np.testing.assert_array_equal(oracle.routing_weights(s, ids1), 1.0)


# ----------------------------------------------------------------------------- experts / layer

def _identity_layer(d, shared_identity):
    dims = synth.Dims(T=6, d=d, E=1, k=1, I=d, I_shared=d)
    eye = np.eye(d, dtype=np.int64)
    w13 = np.concatenate([eye, eye])[None]
    w2 = eye[None]
    z13 = np.zeros((2 * d, d), dtype=np.int64)
    if shared_identity:
        s13, s2 = np.concatenate([eye, eye]), eye
    else:
        s13, s2 = z13, np.zeros((d, d), dtype=np.int64)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((6, d)).astype(np.float32) * 2
    return layer(dims, x, np.zeros((1, d)), np.zeros(1), w13, w2, s13, s2)


def test_single_expert_identity_closed_form():
    inp = _identity_layer(64, shared_identity=False)
    out = oracle.forward(inp)
    x = x_values(inp)
    np.testing.assert_allclose(out["y"], x * x / (1 + np.exp(-x)), rtol=1e-14, atol=0)
    inp2 = _identity_layer(64, shared_identity=True)
    out2 = oracle.forward(inp2)
    np.testing.assert_allclose(out2["y"], 2 * x * x / (1 + np.exp(-x)), rtol=1e-14, atol=0)


def test_selection_matrices_non_square():
    """Gate, up and down are 0/1 selection matrices of different shapes (d=64, I=32).

    Then y[pd(i)] = silu(x[pg(i)]) * x[pu(i)] and every other y is 0: a
    transposed matrix, a swapped gate/up half or a wrong silu argument all
    change the result.
    """
    d, I = 64, 32
    rng = np.random.default_rng(9)
    pg, pu, pd = rng.permutation(d)[:I], rng.permutation(d)[:I], rng.permutation(d)[:I]
    w13 = np.zeros((2 * I, d), dtype=np.int64)
    w13[np.arange(I), pg] = 1
    w13[I + np.arange(I), pu] = 1
    w2 = np.zeros((d, I), dtype=np.int64)
    w2[pd, np.arange(I)] = 1
    dims = synth.Dims(T=5, d=d, E=1, k=1, I=I, I_shared=I)
    x = rng.standard_normal((5, d)).astype(np.float32)
    inp = layer(dims, x, np.zeros((1, d)), np.zeros(1), w13[None], w2[None],
                np.zeros((2 * I, d), dtype=np.int64), np.zeros((d, I), dtype=np.int64))
    xv = x_values(inp)
    want = np.zeros((5, d))
    g, u = xv[:, pg], xv[:, pu]
    want[:, pd] = g / (1 + np.exp(-g)) * u
    np.testing.assert_allclose(oracle.forward(inp)["y"], want, rtol=1e-14, atol=0)


def naive_mlp(x, w13, w2):
    """Triple loops, no BLAS."""
    I2, d = len(w13), len(w13[0])
    I = I2 // 2
    y = [0.0] * d
    h = []
    for i in range(I):
        g = sum(x[c] * w13[i][c] for c in range(d))
        u = sum(x[c] * w13[I + i][c] for c in range(d))
        h.append(g / (1.0 + math.exp(-g)) * u)
    for n in range(d):
        y[n] = sum(w2[n][i] * h[i] for i in range(I))
    return y


def test_single_expert_layer_is_dense_swiglu_bruteforce():
    dims = synth.Dims(T=3, d=32, E=1, k=1, I=32, I_shared=32)
    inp = synth.make_inputs(dims, seed=11)
    out = oracle.forward(inp)
    x = x_values(inp)
    w13 = oracle.dequant_q4(inp["w13_qs"][0], inp["w13_sc"][0]).tolist()
    w2 = oracle.dequant_q4(inp["w2_qs"][0], inp["w2_sc"][0]).tolist()
    s13 = oracle.dequant_q4(inp["s13_qs"], inp["s13_sc"]).tolist()
    s2 = oracle.dequant_q4(inp["s2_qs"], inp["s2_sc"]).tolist()
    for t in range(3):
        r = naive_mlp(x[t].tolist(), w13, w2)
        s = naive_mlp(x[t].tolist(), s13, s2)
        np.testing.assert_allclose(out["y"][t], np.array(r) + np.array(s), rtol=1e-12, atol=1e-12)


def test_full_mixture_k_equals_E():
    dims = synth.Dims(T=4, d=64, E=5, k=5, I=32, I_shared=32)
    inp = synth.make_inputs(dims, seed=12)
    out = oracle.forward(inp)
    assert np.all(np.sort(out["ids"], axis=1) == np.arange(5))
    assert np.all(np.isinf(out["margin"]))
    x = x_values(inp)
    s = out["s"]
    for t in range(4):
        want = np.array(naive_mlp(x[t].tolist(), oracle.dequant_q4(inp["s13_qs"], inp["s13_sc"]).tolist(),
                                  oracle.dequant_q4(inp["s2_qs"], inp["s2_sc"]).tolist()))
        for e in range(5):
            ye = naive_mlp(x[t].tolist(), oracle.dequant_q4(inp["w13_qs"][e], inp["w13_sc"][e]).tolist(),
                           oracle.dequant_q4(inp["w2_qs"][e], inp["w2_sc"][e]).tolist())
            want = want + s[t, e] / s[t].sum() * np.array(ye)
        np.testing.assert_allclose(out["y"][t], want, rtol=1e-12, atol=1e-12)


def test_shared_only_when_routed_weights_are_zero():
    dims = synth.Dims(T=5, d=64, E=6, k=2, I=32, I_shared=64)
    inp = synth.make_inputs(dims, seed=13)
    inp["w13_qs"][:] = 0x88
    inp["w2_qs"][:] = 0x88
    out = oracle.forward(inp)
    x = x_values(inp)
    s13 = oracle.dequant_q4(inp["s13_qs"], inp["s13_sc"]).tolist()
    s2 = oracle.dequant_q4(inp["s2_qs"], inp["s2_sc"]).tolist()
    for t in range(5):
        np.testing.assert_allclose(out["y"][t], naive_mlp(x[t].tolist(), s13, s2), rtol=1e-12, atol=1e-12)


def test_residual_alone_when_every_expert_is_zero():
    """All codes 8 (every routed and shared weight 0): the layer output is the residual itself, exactly,
    and without a residual it is exactly 0 ([nemotron] "ffai_add3": the residual comes after the
    routed + shared sum)."""
    dims = synth.Dims(T=5, d=64, E=6, k=2, I=32, I_shared=64)
    inp = synth.make_inputs(dims, seed=15)
    for key in ("w13_qs", "w2_qs", "s13_qs", "s2_qs"):
        inp[key][:] = 0x88
    r = np.random.default_rng(16).standard_normal((5, 64)).astype(np.float32)
    np.testing.assert_array_equal(oracle.forward(inp)["y"], 0.0)
    np.testing.assert_array_equal(oracle.forward(inp, residual=r)["y"], r.astype(np.float64))
    sub = oracle.forward(inp, tokens=[3, 1], residual=r)["y"]
    np.testing.assert_array_equal(sub, r[[3, 1]].astype(np.float64))


def test_identity_layer_plus_residual_closed_form():
    """Identity expert (y = x^2 sigma(x)) plus a residual r: y = x^2 sigma(x) + r."""
    inp = _identity_layer(64, shared_identity=False)
    x = x_values(inp)
    r = np.random.default_rng(17).standard_normal(x.shape).astype(np.float32)
    np.testing.assert_allclose(oracle.forward(inp, residual=r)["y"], x * x / (1 + np.exp(-x)) + r,
                               rtol=1e-14, atol=1e-15)


def test_doubling_down_scales_doubles_output_exactly():
    dims = synth.Dims(T=6, d=64, E=8, k=3, I=32, I_shared=32)
    inp = synth.make_inputs(dims, seed=14)
    y1 = oracle.forward(inp)["y"]
    inp2 = dict(inp)
    inp2["w2_sc"] = fp16_bits(oracle.fp16_bits_to_f64(inp["w2_sc"]) * 2)
    inp2["s2_sc"] = fp16_bits(oracle.fp16_bits_to_f64(inp["s2_sc"]) * 2)
    np.testing.assert_array_equal(oracle.forward(inp2)["y"], 2 * y1)


def test_token_permutation_equivariance():
    inp = synth.make_inputs(synth.CONFIGS["tiny"])
    out = oracle.forward(inp)
    perm = np.random.default_rng(15).permutation(inp["dims"].T)
    inp2 = dict(inp)
    inp2["x"] = inp["x"][perm]
    out2 = oracle.forward(inp2)
    np.testing.assert_array_equal(out2["ids"], out["ids"][perm])
    np.testing.assert_allclose(out2["y"], out["y"][perm], rtol=1e-13, atol=1e-13)


def test_token_subset_matches_full():
    inp = synth.make_inputs(synth.CONFIGS["tiny"])
    full = oracle.forward(inp)
    sub = oracle.forward(inp, tokens=[5, 2, 7])
    np.testing.assert_allclose(sub["y"], full["y"][[5, 2, 7]], rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(sub["ids"], full["ids"][[5, 2, 7]])


def test_ids_override_uses_given_experts_and_fp64_weights():
    inp = synth.make_inputs(synth.CONFIGS["tiny"])
    full = oracle.forward(inp)
    sel = [0, 1, 2, 3]
    ov = oracle.forward(inp, ids_override={4: sel})
    np.testing.assert_array_equal(ov["ids"][4], sel)
    s = full["s"][4]
    np.testing.assert_allclose(ov["w"][4], s[sel] / s[sel].sum(), rtol=1e-15)
    # other tokens are untouched (BLAS may round differently when the row groups change)
    np.testing.assert_allclose(ov["y"][[0, 1, 2, 3, 5, 6, 7]], full["y"][[0, 1, 2, 3, 5, 6, 7]], rtol=1e-13, atol=1e-15)
    assert not np.allclose(ov["y"][4], full["y"][4])


# ----------------------------------------------------------------------------- routing build

def test_routing_build_bruteforce():
    rng = np.random.default_rng(16)
    T, E, k = 37, 11, 3
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    r = oracle.routing_build(ids, E)
    P = T * k
    seq = []
    for e in range(E):
        for p in range(P):
            if ids.ravel()[p] == e:
                seq.append(p)
    np.testing.assert_array_equal(r["sorted_pair"], seq)
    for e in range(E):
        assert r["counts"][e] == sum(1 for p in range(P) if ids.ravel()[p] == e)
        assert r["offsets"][e] == sum(r["counts"][:e])
    assert r["offsets"][E] == P
    for pos, p in enumerate(seq):
        assert r["pair_pos"][p] == pos
        assert r["row_expert"][pos] == ids.ravel()[p]
    order = oracle.group_order(r["counts"], T)
    assert order[0] == E  # the shared group holds every token, so it is the largest
    sizes = [T if g == E else r["counts"][g] for g in order]
    assert all(sizes[i] >= sizes[i + 1] for i in range(len(sizes) - 1))
    assert sorted(order.tolist()) == list(range(E + 1))


def test_group_order_ties_go_to_the_lower_id():
    """Hand-built sizes with ties at every level, the expected schedule written out: descending size,
    equal sizes in ascending group id, the shared group (id E, T rows) ranked by its size like any other
    group, empty groups last.  A 'ties to the higher id' or 'shared first' slip gives another order."""
    counts = np.array([3, 5, 3, 0, 5, 3, 0, 7])   # groups 0..7; group 8 is the shared one
    T = 5                                        # ties the shared group with groups 1 and 4
    want = [7, 1, 4, 8, 0, 2, 5, 3, 6]
    np.testing.assert_array_equal(oracle.group_order(counts, T), want)
    # every group the same size: plain id order, shared last
    np.testing.assert_array_equal(oracle.group_order(np.full(4, 2), 2), [0, 1, 2, 3, 4])
    # a shared group larger than every expert comes first
    np.testing.assert_array_equal(oracle.group_order(np.array([1, 2, 2]), 9), [3, 1, 2, 0])


# ----------------------------------------------------------------------------- generator

def test_generator_deterministic_and_distributions():
    a = synth.make_inputs(synth.CONFIGS["tiny"])
    b = synth.make_inputs(synth.CONFIGS["tiny"])
    for key in ("x", "w_router", "bias", "w13_qs", "w13_sc", "w2_qs", "w2_sc", "s13_qs", "s13_sc", "s2_qs", "s2_sc"):
        np.testing.assert_array_equal(a[key], b[key])
    c = synth.make_inputs(synth.CONFIGS["tiny"], seed=1)
    assert not np.array_equal(a["w13_qs"], c["w13_qs"])
    sc = a["w13_sc"].view(np.float16).astype(np.float64)
    assert sc.min() >= 0.005 - 1e-5 and sc.max() <= 0.02 + 1e-5
    assert np.all(np.abs(a["bias"]) <= 0.1)
    dims = a["dims"]
    assert a["w13_qs"].shape == (dims.E, 2 * dims.I, dims.d // 2)
    assert a["w2_sc"].shape == (dims.E, dims.d, dims.I // 32)


def test_generator_zipf_and_outliers():
    z = synth.make_inputs(synth.Dims(T=4, d=64, E=256, k=10, I=32, I_shared=32), bias="zipf", weights=False)
    b = np.sort(z["bias"].astype(np.float64))[::-1]
    assert b.sum() == pytest.approx(1.0, abs=1e-6)
    assert b[0] == pytest.approx(1.0 / sum(i ** -1.2 for i in range(1, 257)), rel=1e-6)
    o = synth.make_inputs(synth.Dims(T=8192, d=32, E=4, k=1, I=32, I_shared=32), outlier_frac=0.01, weights=False)
    assert len(o["outlier_rows"]) == 82


# ----------------------------------------------------------------------------- multi-layer decode chain

def bf16_carry(f32: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 by the bit-carry rule on the float32 pattern (written here
    from the format definition: add 0x7FFF plus the lowest kept bit, keep the top 16 bits)."""
    u = np.asarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_bf16_rounding_matches_the_carry_rule_on_float32_inputs():
    rng = np.random.default_rng(21)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-60, 60, 20000))).astype(np.float32)
    f[:4] = [0.0, -0.0, 1.0, -2.5]
    np.testing.assert_array_equal(oracle.f64_to_bf16_bits(f.astype(np.float64)), bf16_carry(f))


def test_bf16_rounding_ties_and_ends():
    # bf16 spacing at 1 is 2^-7: halfway points go to the even neighbour
    vals = [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 2.0 ** -133 * 1.5, 3.5e38, -1e39]
    want = [0x3F80, 0x3F82, 0xBF80, 0x0002, 0x7F80, 0xFF80]
    np.testing.assert_array_equal(oracle.f64_to_bf16_bits(np.array(vals)), np.array(want, dtype=np.uint16))
    assert oracle.f64_to_bf16_bits(np.array([np.nan]))[0] == 0x7FC0


def _stream(T, d, seed):
    return np.random.default_rng(seed).standard_normal((T, d)).astype(np.float32) * 2


def test_decode_chain_with_zero_experts_keeps_the_stream():
    """Every code 8 in every layer: each layer adds exactly zero, so the stream passes through unchanged."""
    dims = synth.Dims(T=4, d=64, E=6, k=2, I=32, I_shared=64)
    layers = []
    for s in range(3):
        inp = synth.make_inputs(dims, seed=30 + s)
        for key in ("w13_qs", "w2_qs", "s13_qs", "s2_qs"):
            inp[key][:] = 0x88
        layers.append(inp)
    h0 = _stream(4, 64, 31)
    out = oracle.decode_chain(layers, h0)
    np.testing.assert_array_equal(out["h"], h0.astype(np.float64))
    assert out["margins"].shape == (3, 4)


def test_decode_chain_identity_expert_recurrence():
    """One identity expert per layer and no shared expert: every element follows
    h <- h + x^2 sigma(x) with x = bf16(h), a scalar recurrence evaluated here element by element."""
    d = 32
    base = _identity_layer(d, shared_identity=False)
    T = base["dims"].T
    h0 = _stream(T, d, 33)
    out = oracle.decode_chain([base, base, base], h0)
    for t in range(T):
        for c in range(d):
            h = float(h0[t, c])
            for _ in range(3):
                x = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(np.array([h])))[0]
                h = h + x * x / (1.0 + math.exp(-x))
            assert abs(out["h"][t, c] - h) <= 1e-12 * max(1.0, abs(h)), (t, c)


def test_decode_chain_tokens_are_independent():
    """The chain never mixes tokens: permuting the stream's rows permutes the result exactly."""
    dims = synth.Dims(T=5, d=64, E=8, k=2, I=32, I_shared=32)
    layers = [synth.make_inputs(dims, seed=40 + s) for s in range(2)]
    h0 = _stream(5, 64, 41)
    perm = np.array([3, 0, 4, 1, 2])
    a = oracle.decode_chain(layers, h0)["h"]
    b = oracle.decode_chain(layers, h0[perm])["h"]
    np.testing.assert_array_equal(b, a[perm])


# ----------------------------------------------------------------------------- pre-MoE norm

def test_rms_norm_closed_forms():
    # a row of equal values c: mean square c^2, so every output is c / sqrt(c^2 + eps) * gamma
    g = np.linspace(0.5, 2.0, 16)
    for c, eps in [(3.0, 0.0), (0.25, 1e-6), (-2.0, 0.5)]:
        out = oracle.rms_norm(np.full((1, 16), c), g, eps)
        np.testing.assert_allclose(out[0], c / math.sqrt(c * c + eps) * g, rtol=1e-15)
    # a row with mean square 1 and gamma 1, eps 0: unchanged
    h = np.array([[1.0, -1.0, 1.0, -1.0, math.sqrt(2), 0.0, 1.0, -1.0]])
    assert abs(np.mean(h * h) - 1.0) < 1e-15
    np.testing.assert_allclose(oracle.rms_norm(h, np.ones(8), 0.0), h, rtol=1e-15, atol=1e-15)


def test_rms_norm_invariances():
    rng = np.random.default_rng(61)
    h = rng.standard_normal((5, 64))
    g = rng.uniform(0.5, 1.5, 64)
    base = oracle.rms_norm(h, g, 0.0)
    # positive scaling of a row leaves it unchanged (eps = 0); a negative one flips its sign
    np.testing.assert_allclose(oracle.rms_norm(7.5 * h, g, 0.0), base, rtol=1e-13)
    np.testing.assert_allclose(oracle.rms_norm(-h, g, 0.0), -base, rtol=1e-13)
    # every output row has mean square mean(gamma^2 * (normalised)^2) -> with gamma = 1 exactly 1
    unit = oracle.rms_norm(h, np.ones(64), 0.0)
    np.testing.assert_allclose(np.mean(unit * unit, axis=1), 1.0, rtol=1e-13)
    # rows are independent: a permutation of rows permutes the result
    perm = np.array([4, 2, 0, 1, 3])
    np.testing.assert_array_equal(oracle.rms_norm(h[perm], g, 1e-5), oracle.rms_norm(h, g, 1e-5)[perm])


def test_decode_chain_with_norm_keeps_zero_layers_identity_and_normalises_input():
    """With the pre-MoE norm and zero experts the stream still passes unchanged; with identity experts
    each element follows h <- h + x^2 sigma(x), now with x = bf16(rms_norm(h) * gamma)."""
    dims = synth.Dims(T=3, d=32, E=1, k=1, I=32, I_shared=32)
    base = _identity_layer(32, shared_identity=False)
    T = base["dims"].T
    gamma = np.random.default_rng(62).uniform(0.5, 1.5, 32)
    lay = dict(base, norm_weight=gamma, norm_eps=1e-5)
    h0 = _stream(T, 32, 63)
    out = oracle.decode_chain([lay, lay], h0)
    h = h0.astype(np.float64)
    for _ in range(2):
        xn = h / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + 1e-5) * gamma
        x = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(xn))
        h = h + x * x / (1.0 + np.exp(-x))
    np.testing.assert_allclose(out["h"], h, rtol=1e-12, atol=1e-12)
    zero = synth.make_inputs(synth.Dims(T=3, d=64, E=4, k=2, I=32, I_shared=32), seed=64)
    for key in ("w13_qs", "w2_qs", "s13_qs", "s2_qs"):
        zero[key][:] = 0x88
    zero = dict(zero, norm_weight=np.ones(64), norm_eps=1e-6)
    h1 = _stream(3, 64, 65)
    np.testing.assert_array_equal(oracle.decode_chain([zero, zero], h1)["h"], h1.astype(np.float64))
