"""The grouped GEMM's fp16 dequantisation identities, checked exhaustively on the host.

The kernel turns a Q4 code q and its fp16 block scale d into the MFMA operand (q - 8) * d / 16 with
one packed fp16 FMA: the code, masked in place into a zero-exponent fp16, is the subnormal q * 2^-24
(bits 0..3) or q * 2^-20 (bits 4..7), and the FMA multiplies it by d * 2^20 or d * 2^16 and adds -d/2.
The GEMM's accumulators are multiplied by 16 afterwards.  These tests emulate that arithmetic (an FMA
is exact before its one rounding, which float64 holds for these operands) and check, for every fp16
scale of the common range [2^-10, 2^-4) and every code, that it equals round((q - 8) * d) / 16 -- the
plain Q4 value (the format of "feat(laguna): Laguna-S-2.1 decode on the CUDA engine": value =
(q - 8) * scale) rounded once to fp16, then scaled by an exact power of two -- and that the general
form the kernel falls back to outside that range agrees wherever that value is an fp16 normal.
"""
import numpy as np

F16 = np.float16


def fp16_bits(v):
    return np.asarray(v, dtype=F16).view(np.uint16)


def from_bits(b):
    return np.asarray(b, dtype=np.uint16).view(F16)


def all_scales(lo_exp, hi_exp):
    """Every positive fp16 with lo_exp <= exponent < hi_exp (unbiased)."""
    bits = np.arange((lo_exp + 15) << 10, (hi_exp + 15) << 10, dtype=np.uint32).astype(np.uint16)
    return from_bits(bits)


def fma16(a, b, c):
    """fp16 FMA: exact product and sum (float64 holds them here), one rounding to fp16."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(F16)


def common_form(q, d, high_nibble):
    """(q - 8) * d / 16 as the kernel's common form computes it."""
    code = from_bits((q.astype(np.uint16) << (4 if high_nibble else 0)))  # subnormal q * 2^-24 or 2^-20
    mul = (d.astype(np.float64) * (2.0 ** (16 if high_nibble else 20))).astype(F16)
    add = (d.astype(np.float64) * -0.5).astype(F16)
    # the constants are exact: d * 2^k and -d/2 are fp16 values in this range
    assert np.all(mul.astype(np.float64) == d.astype(np.float64) * 2.0 ** (16 if high_nibble else 20))
    assert np.all(add.astype(np.float64) == d.astype(np.float64) * -0.5)
    return fma16(code, mul, add)


def general_form(q, d):
    """((1024 + q) - 1032) * d, rounded, then * 1/16, rounded: the kernel's general form."""
    p = from_bits(np.uint16(0x6400) | q.astype(np.uint16))  # 1024 + q, exact
    assert np.all(p.astype(np.float64) == 1024 + q)
    t = (p - F16(1032.0)).astype(F16)  # q - 8, exact
    return ((t * d).astype(F16) * F16(0.0625)).astype(F16)


def plain_value(q, d):
    """round((q - 8) * d) / 16 in fp16."""
    return ((q.astype(np.float64) - 8) * d.astype(np.float64)).astype(F16).astype(np.float64) / 16.0


def grid(d):
    q = np.arange(16, dtype=np.int64)
    return np.repeat(q[None, :], d.size, 0).ravel(), np.repeat(d[:, None], 16, 1).ravel()


def test_common_form_is_the_plain_value_over_sixteen_for_every_scale_and_code():
    d = all_scales(-10, -4)
    assert d.size == 6 * 1024
    for sign in (1, -1):
        q, dd = grid((d * F16(sign)).astype(F16))
        want = plain_value(q, dd)
        for high in (False, True):
            got = common_form(q, dd, high).astype(np.float64)
            np.testing.assert_array_equal(got, want)


def test_zero_scale_gives_zero():
    q = np.arange(16)
    for high in (False, True):
        assert np.all(common_form(q, np.zeros(16, F16), high) == 0)
    assert np.all(general_form(q, np.zeros(16, F16)) == 0)


def test_general_form_matches_where_the_result_is_normal():
    # large scales: every nonzero result is an fp16 normal, so the two roundings are one
    d = all_scales(-4, 9)  # up to 2^9: (q - 8) * d stays finite
    q, dd = grid(d)
    np.testing.assert_array_equal(general_form(q, dd).astype(np.float64), plain_value(q, dd))
    # the common range: the fallback gives the same bits as the common form
    d = all_scales(-10, -4)
    q, dd = grid(d)
    np.testing.assert_array_equal(general_form(q, dd), common_form(q, dd, False))


def test_tiny_scales_stay_within_half_an_fp16_subnormal_step():
    # below 2^-10 the value / 16 can fall under the fp16 normal range; the general form then rounds
    # twice, and its error stays below half a subnormal spacing (2^-25) on top of the first rounding
    d = all_scales(-14, -10)
    q, dd = grid(d)
    err = np.abs(general_form(q, dd).astype(np.float64) - plain_value(q, dd))
    assert err.max() <= 2.0 ** -25


def test_scale_ranges_match_the_kernel_test():
    # the kernel takes the common form when (bits & 0x7FFF) - 0x1400 < 0x1800 (unsigned) or the
    # magnitude is zero: exactly the exponents -10 .. -5 and zero
    bits = np.arange(0, 0x10000, dtype=np.uint32)
    m = bits & 0x7FFF
    ok = (((m - 0x1400) & 0xFFFFFFFF) < 0x1800) | (m == 0)
    v = np.abs(from_bits(bits.astype(np.uint16)).astype(np.float64))
    finite = np.isfinite(v)
    want = finite & (((v >= 2.0 ** -10) & (v < 2.0 ** -4)) | (v == 0))
    np.testing.assert_array_equal(ok, want)
