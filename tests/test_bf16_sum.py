"""The kernels form the new prefix bf16(prefix + delta) with one float32
addition followed by round-to-nearest-even to bfloat16. That equals the
correctly rounded bfloat16 sum the plain definition names (attn_res.kernel
page, ClusterAttnRes.post: the prefix update is rounded to bf16) because
float32 carries 24 >= 2 * 8 + 2 significant bits (the double-rounding bound for
addition, Figueroa 1995). This checks the claim on random and adversarial
bfloat16 pairs against exact rounding, with an exact-rounding helper written
here (independent of the oracle's C code)."""
from __future__ import annotations

import numpy as np


def rne_bf16_from_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even); returns bits."""
    x = np.asarray(x, np.float64)
    sign = np.signbit(x)
    a = np.abs(x)
    m, e = np.frexp(a)            # a = m 2^e, m in [0.5, 1)
    q = np.maximum(e - 8, -133)   # quantum 2^q: 8 significant bits, subnormal floor 2^-133
    r = np.rint(np.ldexp(a, -q))  # round half to even
    v = np.ldexp(r, q)
    bits = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(a == 0, 0, bits).astype(np.uint16)
    return np.where(sign, bits | 0x8000, bits).astype(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def kernel_sum_bits(a_bits, b_bits):
    s = bf16_values(a_bits) + bf16_values(b_bits)   # float32, round to nearest even
    return rne_bf16_from_f64(s.astype(np.float64))


def exact_sum_bits(a_bits, b_bits):
    # exact in float64 while the exponents differ by at most 45
    return rne_bf16_from_f64(bf16_values(a_bits).astype(np.float64) +
                             bf16_values(b_bits).astype(np.float64))


def test_rne_helper_on_known_values():
    assert rne_bf16_from_f64(np.array([1.0]))[0] == 0x3F80
    # 1 + 2^-8 is the tie between 1 and 1 + 2^-7: even mantissa wins (1.0)
    assert rne_bf16_from_f64(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    # 1 + 3 * 2^-8 ties between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert rne_bf16_from_f64(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82
    assert rne_bf16_from_f64(np.array([-2.5]))[0] == 0xC020
    assert rne_bf16_from_f64(np.array([2.0 ** -133]))[0] == 0x0001


def test_float32_sum_rounds_like_the_exact_sum():
    rng = np.random.default_rng(7)
    n = 1 << 21
    # random signs, exponents within 40 of each other, random 7-bit fractions
    ea = rng.integers(100, 155, n)
    eb = ea + rng.integers(-20, 21, n)
    fa, fb = rng.integers(0, 128, n), rng.integers(0, 128, n)
    sa, sb = rng.integers(0, 2, n), rng.integers(0, 2, n)
    a = ((sa << 15) | (ea << 7) | fa).astype(np.uint16)
    b = ((sb << 15) | (np.clip(eb, 1, 254) << 7) | fb).astype(np.uint16)
    assert np.array_equal(kernel_sum_bits(a, b), exact_sum_bits(a, b))


def test_float32_sum_near_ties_and_cancellation():
    # b a few ulps of a around half-ulp ties, both signs, and exact cancellation
    base = np.arange(0x3F00, 0x4100, dtype=np.uint16)           # [0.5, 8)
    small = np.array([0x3B00 + i for i in range(0, 256, 3)], np.uint16)  # ~2^-9 .. 2^-8
    a = np.repeat(base, small.size)
    b = np.tile(small, base.size)
    for sb in (0, 0x8000):
        bb = (b | sb).astype(np.uint16)
        assert np.array_equal(kernel_sum_bits(a, bb), exact_sum_bits(a, bb))
    assert np.all(kernel_sum_bits(base, base | 0x8000) == 0)       # x + (-x) = +0


def test_float32_sum_subnormal_range():
    a = np.arange(0x0000, 0x0200, dtype=np.uint16)
    b = np.arange(0x0080, 0x0280, dtype=np.uint16)
    for sb in (0, 0x8000):
        bb = (b | sb).astype(np.uint16)
        assert np.array_equal(kernel_sum_bits(a, bb), exact_sum_bits(a, bb))
