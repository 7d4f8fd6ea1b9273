"""Pins of the W4A8 oracle (MXFP4 weights x FP8 activations), on the CPU.

The element formats are pinned to the value tables of their definitions (written out here, not
recomputed), the rounding to hand-picked ties and saturations, the block requantisation to
hand-worked blocks, and the layer to exact invariants (power-of-two scalings pass through the
shared exponents unchanged) and to the W4A16 oracle where the two must agree exactly.
"""
import numpy as np
import pytest

import oracle
import oracle.moe_w4a8 as w4
import synth

# e2m1 values of codes 0..7 (sign bit 3 negates): the fp4 grid
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
# e4m3 spot values: (code, value)
E4M3_POINTS = [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x30, 0.5),
               (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x78, 256.0), (0x7E, 448.0),
               (0xB8, -1.0), (0xFE, -448.0)]


def test_e2m1_table():
    assert w4.e2m1_value(np.arange(8)).tolist() == E2M1_TABLE
    assert w4.e2m1_value(np.arange(8, 16)).tolist() == [-v for v in E2M1_TABLE]


def test_e4m3_points_and_round_trip():
    for c, v in E4M3_POINTS:
        assert float(w4.e4m3_value(c)) == v, hex(c)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    back = w4.round_e4m3(w4.e4m3_value(codes))
    # every finite code rounds back to itself (the negative zero 0x80 included)
    assert np.array_equal(back, codes.astype(np.uint8))
    # the grid is strictly increasing over the non-negative codes
    vals = w4.e4m3_value(np.arange(0x7F))
    assert np.all(np.diff(vals) > 0)


@pytest.mark.parametrize("v, code", [
    (1.0625, 0x38),     # halfway 1 .. 1.125: even mantissa (1.0)
    (1.1875, 0x3A),     # halfway 1.125 .. 1.25: even mantissa (1.25)
    (1.07, 0x39),       # nearer to 1.125
    (448.0, 0x7E), (460.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE),   # saturation
    (2.0 ** -10, 0x00),  # halfway 0 .. 2^-9: even (zero)
    (3 * 2.0 ** -10, 0x02),  # halfway 2^-9 .. 2^-8: even
    (-2.0 ** -12, 0x80),  # rounds to zero, keeps the sign bit
])
def test_e4m3_rounding(v, code):
    assert int(w4.round_e4m3(v)) == code


@pytest.mark.parametrize("v, code", [
    (0.25, 0x0), (0.75, 0x2), (1.25, 0x2), (1.75, 0x4), (2.5, 0x4), (3.5, 0x6), (5.0, 0x6),  # ties to even
    (5.5, 0x7), (6.0, 0x7), (7.0, 0x7), (100.0, 0x7), (-5.0, 0xE), (-0.1, 0x8),
])
def test_e2m1_rounding(v, code):
    assert int(w4.round_e2m1(v)) == code


def _q4_block(qvals, d):
    """One row of 32 Q4 values (codes 0..15) with fp16 scale d, row-major format."""
    q = np.asarray(qvals, dtype=np.uint8)
    qs = (q[0::2] | (q[1::2] << 4)).astype(np.uint8)[None, :]
    sc = np.array([[np.float16(d).view(np.uint16)]], dtype=np.uint16)
    return qs, sc


def test_requant_hand_worked_block():
    # codes 0..15 twice: values -8..7 times d = 1; amax 8 -> E = floor(log2 8) - 2 = 1, so the elements
    # are (q - 8) / 2 rounded to the e2m1 grid: -4 -3.5 -3 -2.5 -2 -1.5 -1 -0.5 0 0.5 1 1.5 2 2.5 3 3.5
    qs, sc = _q4_block(list(range(16)) * 2, 1.0)
    codes, exp = w4.mx_requant(qs, sc)
    assert exp.tolist() == [[128]]
    vals = w4.mx_dequant(codes, exp)[0, :16] / 2.0
    expect = [-4, -4, -3, -2, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 2, 3, 4]  # ties to even mantissa
    assert vals.tolist() == expect


def test_requant_exact_cases_and_zero_block():
    # values in {0, +-1, +-2, +-4, -8} * d with d a power of two: amax 8d, every element exact
    q = np.array([8, 9, 7, 10, 6, 12, 4, 0] * 4, dtype=np.int64)
    for d in (1.0, 0.25, 2.0 ** -14, 64.0):
        qs, sc = _q4_block(q, d)
        codes, exp = w4.mx_requant(qs, sc)
        assert np.array_equal(w4.mx_dequant(codes, exp), oracle.dequant_q4(qs, sc))
    qs, sc = _q4_block([8] * 32, 1.0)   # all values zero
    codes, exp = w4.mx_requant(qs, sc)
    assert exp.tolist() == [[0]] and not codes.any()
    qs, sc = _q4_block([3] * 32, 0.0)   # zero scale
    codes, exp = w4.mx_requant(qs, sc)
    assert exp.tolist() == [[0]] and np.all(w4.mx_dequant(codes, exp) == 0)


def test_requant_error_bound():
    # the nearest-value rounding on a grid whose relative spacing is at most 1/2 (between 4 and 6)
    # keeps every element within a quarter of its block's largest magnitude
    rng = np.random.default_rng(5)
    qs = rng.integers(0, 256, size=(16, 64), dtype=np.uint8)
    sc = np.float16(rng.uniform(0.005, 0.02, size=(16, 4))).view(np.uint16)
    ref = oracle.dequant_q4(qs, sc).reshape(16, 4, 32)
    got = w4.mx_dequant(*w4.mx_requant(qs, sc)).reshape(16, 4, 32)
    amax = np.abs(ref).max(axis=2, keepdims=True)
    assert np.all(np.abs(got - ref) <= 0.25 * amax + 1e-12)


def test_quant_rows_fp8():
    X = np.array([[448.0, 1.0, -2.0, 0.5], [896.0, -896.0, 3.0, 0.0], [0.0, 0.0, 0.0, 0.0]], dtype=np.float32)
    codes, s = w4.quant_rows_fp8(X)
    assert s.tolist() == [1.0, 2.0, 1.0]
    assert codes[0].tolist() == [0x7E, 0x38, 0xC0, 0x30]
    assert codes[1].tolist() == [0x7E, 0xFE, 0x3C, 0x00]      # 1.5 = 0x3C
    assert not codes[2].any()
    # scale by a power of two: same codes, doubled scale (an all-zero row keeps scale 1)
    c2, s2 = w4.quant_rows_fp8(2 * X)
    assert np.array_equal(c2, codes) and np.array_equal(s2[:2], 2 * s[:2]) and s2[2] == 1.0


def test_layer_doubling_down_scales_doubles_y():
    inp = synth.make_inputs(synth.CONFIGS["tiny"])
    base = w4.forward_w4a8(inp)["y"]
    inp2 = dict(inp)
    for name in ("w2_sc", "s2_sc"):
        inp2[name] = (inp[name].view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
    y2 = w4.forward_w4a8(inp2)["y"]
    assert np.array_equal(y2, 2 * base)


def test_layer_matches_w4a16_where_quantisation_is_exact():
    # Q4 values with power-of-two scales whose blocks requantise exactly (see above) and inputs that are
    # fp8-exact after their row scale: the W4A8 layer differs from the W4A16 oracle only by the fp16
    # and fp8 roundings of h, so it selects the same experts and lands within a few percent.
    inp = synth.make_inputs(synth.CONFIGS["tiny"])
    dims = inp["dims"]
    rng = np.random.default_rng(11)
    grid = np.array([8, 9, 7, 10, 6, 12, 4, 0], dtype=np.uint8)   # (q-8) in {0,1,-1,2,-2,4,-4,-8}
    for name in ("w13", "w2", "s13", "s2"):
        shape = inp[name + "_qs"].shape
        q = grid[rng.integers(0, 8, size=shape[:-1] + (shape[-1] * 2,))]
        inp[name + "_qs"] = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
        inp[name + "_sc"] = np.full(inp[name + "_sc"].shape, np.float16(0.25).view(np.uint16), dtype=np.uint16)
    # x: values from the e4m3 grid times 2^-3 with each row's largest magnitude 448 * 2^-3
    vals = w4.e4m3_value(rng.integers(0x30, 0x50, size=(dims.T, dims.d))) * rng.choice([-1, 1], size=(dims.T, dims.d))
    vals[:, 0] = 448.0
    xf = (vals * 2.0 ** -3).astype(np.float32)
    inp["x"] = (xf.view(np.uint32) >> 16).astype(np.uint16)   # exact in bf16 (4 significant bits)
    r4 = w4.forward_w4a8(inp)
    r16 = oracle.forward(inp)
    assert np.array_equal(r4["ids"], r16["ids"])
    # h differs by its fp16 and fp8 roundings only: relative to the layer's scale, a few percent at most
    err = np.linalg.norm(r4["y"] - r16["y"]) / np.linalg.norm(r16["y"])
    assert 0 < err < 0.05


def test_layer_permutation_equivariance_and_token_subsets():
    inp = synth.make_inputs(synth.CONFIGS["tiny"])
    full = w4.forward_w4a8(inp)
    sub = w4.forward_w4a8(inp, tokens=[5, 1, 3])
    assert np.array_equal(sub["y"], full["y"][[5, 1, 3]])


# ----------------------------------------------------------------------------- W8A8 (MXFP8 weights)

def test_mx8_requant_power_of_two_scales_are_exact():
    # d a power of two: amax = 8d, E = log2(8d) - 8, so the elements are (q - 8) * 2^5 = -256 .. 224,
    # integers with at most 3 significant bits times a power of two: every one is an e4m3 value
    for d in (1.0, 0.25, 2.0 ** -14, 2.0 ** -24, 64.0):
        qs, sc = _q4_block(list(range(16)) * 2, d)
        codes, exp = w4.mx8_requant(qs, sc)
        assert exp.tolist() == [[int(np.log2(8 * d)) - 8 + 127]]
        assert np.array_equal(w4.mx8_dequant(codes, exp), oracle.dequant_q4(qs, sc))
    qs, sc = _q4_block([8] * 32, 1.0)          # all values zero
    codes, exp = w4.mx8_requant(qs, sc)
    assert exp.tolist() == [[0]] and not codes.any()


def test_mx8_requant_hand_worked_block():
    # d = fp16(0.0113) = 0.01129913330078125; amax = 8d = 0.0904 -> floor(log2) = -4, E = -12 (byte 115);
    # the elements (q - 8) * d * 4096 = -370.25, -323.97, -277.69, -231.41, -185.13, -138.84, -92.56,
    # -46.28, 0, 46.28, ... round to the nearest e4m3 value: -384 (0xFC), -320 (0xFA), -288 (0xF9),
    # -224 (0xF6), -192 (0xF4), -144 (0xF1), -96 (0xEC), -48 (0xE4), 0, 48 (0x64), 96 (0x6C),
    # 144 (0x71), 192 (0x74), 224 (0x76), 288 (0x79), 320 (0x7A)
    qs, sc = _q4_block(list(range(16)) * 2, 0.0113)
    codes, exp = w4.mx8_requant(qs, sc)
    assert exp.tolist() == [[115]]
    expect = [0xFC, 0xFA, 0xF9, 0xF6, 0xF4, 0xF1, 0xEC, 0xE4, 0x00, 0x64, 0x6C, 0x71, 0x74, 0x76, 0x79, 0x7A]
    assert codes[0, :16].tolist() == expect and codes[0, 16:].tolist() == expect


def test_mx8_requant_error_bound():
    # below the saturation point each element is within half an e4m3 step of its Q4 value (2^-4 of its
    # magnitude, or 2^(E-10) in the subnormal range); elements past 448 * 2^E sit at +-448 * 2^E
    rng = np.random.default_rng(6)
    qs = rng.integers(0, 256, size=(32, 64), dtype=np.uint8)
    sc = np.float16(rng.uniform(0.005, 0.02, size=(32, 4)) * rng.choice([-1, 1], size=(32, 4))).view(np.uint16)
    ref = oracle.dequant_q4(qs, sc).reshape(32, 4, 32)
    codes, exp = w4.mx8_requant(qs, sc)
    got = w4.mx8_dequant(codes, exp).reshape(32, 4, 32)
    scale = np.ldexp(1.0, exp.astype(np.int64) - 127)[:, :, None]
    sat = np.abs(ref) > 448 * scale
    inside = ~sat
    assert np.all(np.abs(got - ref)[inside] <= (2.0 ** -4 * np.abs(ref) + 2.0 ** -10 * scale)[inside] + 1e-15)
    assert np.array_equal(np.abs(got)[sat], (448 * np.broadcast_to(scale, got.shape))[sat])
    assert sat.any()   # the test draws blocks whose largest value saturates


def test_w8a8_layer_doubling_down_scales_doubles_y():
    inp = synth.make_inputs(synth.CONFIGS["tiny"])
    base = w4.forward_w8a8(inp)["y"]
    inp2 = dict(inp)
    for name in ("w2_sc", "s2_sc"):
        inp2[name] = (inp[name].view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
    assert np.array_equal(w4.forward_w8a8(inp2)["y"], 2 * base)


def test_w8a8_layer_matches_w4a16_with_power_of_two_scales():
    # with power-of-two scales the MXFP8 weights equal the Q4 weights exactly (above), for every code, so
    # the layers differ only by the fp8 roundings of x and h and the fp16 rounding of h
    inp = synth.make_inputs(synth.CONFIGS["tiny"])
    rng = np.random.default_rng(12)
    for name in ("w13", "w2", "s13", "s2"):
        e = rng.integers(-9, -5, size=inp[name + "_sc"].shape)
        inp[name + "_sc"] = np.float16(np.ldexp(1.0, e)).view(np.uint16)
    r8 = w4.forward_w8a8(inp)
    r16 = oracle.forward(inp)
    assert np.array_equal(r8["ids"], r16["ids"])
    err = np.linalg.norm(r8["y"] - r16["y"]) / np.linalg.norm(r16["y"])
    assert 0 < err < 0.08
    # and W8A8 is closer to W4A16 than W4A8 is (the fp4 grid is the coarser one)
    r4 = w4.forward_w4a8(inp)
    assert np.linalg.norm(r4["y"] - r16["y"]) > 1.5 * np.linalg.norm(r8["y"] - r16["y"])
