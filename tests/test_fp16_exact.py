"""The 96-row path's claim of exact weights, checked on the CPU by emulating
its fp16 arithmetic in numpy (IEEE binary16, round to nearest even).

A routed weight is (u - 8) * s for a 4-bit code u and a bf16 group scale s
(Kimi-K2.6 catalog entry, QUANT paragraph: symmetric int4, group 32). With 8
significant bits in s and |u - 8| <= 8 the product has at most 11 significant
bits, so it is exactly an fp16 whenever its last bit is at or above 2^-24 and
it does not overflow. The kernel forms it as fp16 arithmetic on bit patterns.
Its default form: the field shifted to bits 6-9 of a 16-bit half and OR-ed
into 0x4C00 is 16 + u, and one fused multiply-add fma(16 + u, s, -24 s) gives
(u - 8) * s with a single rounding -- exact as long as -24 s is an fp16, i.e.
for every bf16 scale with exponent -17 .. 10 (and up to 2720). Its other form
(a compile-time option): a field OR-ed into 0x6400 is 1024 + u (or 1024 + 16 u
for a field in bits 4-7), then (1024 + u) - 1032 or fma(1024 + 16 u, 1/16,
-72), then a multiply by the scale: exact for exponents -17 .. 12.
Activations are converted to fp16 with one power-of-two scale per token that
puts the token's largest |x| in [2^14, 2^15)."""
import numpy as np

import moe_inputs as mi


def bf16_values(exp_lo, exp_hi):
    """Every positive bf16 value with unbiased exponent in [exp_lo, exp_hi]."""
    bits = [((e + 127) << 7) | m for e in range(exp_lo, exp_hi + 1) for m in range(128)]
    return mi.bf16_bits_to_f32(np.array(bits, np.uint16)).astype(np.float64)


def f16(bits):
    return np.array(bits, np.uint16).view(np.float16)


def kernel_weights(s):
    """The kernel's default dequantisation of all 16 codes against scales s:
    [len(s), 16]."""
    u = np.arange(16, dtype=np.uint16)
    s16 = np.float16(0) + s.astype(np.float16)  # bf16 -> fp16 (exact in range)
    with np.errstate(over="ignore"):
        c16 = s16 * np.float16(-24.0)           # packed fp16 multiply, one rounding
    h = f16(0x4C00 | (u << 6))                  # 16 + u (field in bits 6-9)
    # packed fp16 fma: exact product and sum (exact in float64), one rounding
    with np.errstate(over="ignore", invalid="ignore"):
        return (h.astype(np.float64)[None, :] * s16.astype(np.float64)[:, None]
                + c16.astype(np.float64)[:, None]).astype(np.float16)


def kernel_weights_two_step(s):
    """The kernel's other form (add or fma, then multiply): [len(s), 16]."""
    u = np.arange(16, dtype=np.uint16)
    s16 = np.float16(0) + s.astype(np.float16)
    low = f16(0x6400 | u)              # 1024 + u   (fields in bits 0-3)
    high = f16(0x6400 | (u << 4))      # 1024 + 16u (fields in bits 4-7)
    q_low = low - np.float16(1032)     # packed fp16 add
    # packed fp16 fma: exact product and sum, one rounding
    q_high = (high.astype(np.float64) * 0.0625 - 72.0).astype(np.float16)
    assert np.array_equal(q_low, q_high)
    assert np.array_equal(q_low.astype(np.float64), u.astype(np.float64) - 8)
    with np.errstate(over="ignore"):
        return (q_low[None, :] * s16[:, None]).astype(np.float16)  # packed fp16 multiply


def test_bit_patterns_are_the_codes():
    u = np.arange(16, dtype=np.uint16)
    assert np.array_equal(f16(0x4C00 | (u << 6)).astype(np.float64), 16 + u)
    # the four shifts of a word put each field pair in bits 6-9 of its half
    w = np.uint32(0x76543210)
    for shift, fields in [(6, (0, 4)), (2, (1, 5)), (-2, (2, 6)), (-6, (3, 7))]:
        v = int(w) << shift if shift > 0 else int(w) >> -shift
        v &= 0x03C003C0
        assert ((v >> 6) & 0xF, (v >> 22) & 0xF) == fields
    assert np.array_equal(f16(0x6400 | u).astype(np.float64), 1024 + u)
    assert np.array_equal(f16(0x6400 | (u << 4)).astype(np.float64), 1024 + 16 * u)


def test_weights_exact_over_the_whole_scale_range():
    for form, (lo, hi), top in [(kernel_weights, (-17, 10), 2040.0),
                                (kernel_weights_two_step, (-17, 12), 8160.0)]:
        s = bf16_values(lo, hi)
        s = np.concatenate([s, -s])
        w = form(s)
        exact = (np.arange(16) - 8.0)[None, :] * s[:, None]
        assert np.isfinite(w).all()
        assert np.array_equal(w.astype(np.float64), exact)
        assert float(np.abs(s).max()) == top and float(np.abs(s).min()) == 2.0 ** -17


def test_default_form_reaches_2720():
    s = bf16_values(11, 11)
    s = s[s <= 2720.0]
    assert float(s.max()) == 2720.0
    w = kernel_weights(np.concatenate([s, -s]))
    exact = (np.arange(16) - 8.0)[None, :] * np.concatenate([s, -s])[:, None]
    assert np.array_equal(w.astype(np.float64), exact)


def test_range_is_tight():
    for form, hi in [(kernel_weights, 11), (kernel_weights_two_step, 13)]:
        # one exponent below: some products fall off the fp16 grid
        s = bf16_values(-18, -18)
        w = form(s)
        exact = (np.arange(16) - 8.0)[None, :] * s[:, None]
        assert not np.array_equal(w.astype(np.float64), exact)
        # above the range: the offset -24 s (default form) or -8 s overflows
        s = bf16_values(hi, hi)
        assert not np.isfinite(form(s)).all()


def test_activation_conversion_exact():
    rng = np.random.default_rng(0)
    for scale in [1e-30, 1e-3, 1.0, 7.0, 1e4, 3e30]:
        x = mi.bf16_bits_to_f32(mi.f32_to_bf16_bits(
            (rng.standard_normal(4096) * scale).astype(np.float32))).astype(np.float64)
        m = np.abs(x).max()
        k = int(np.frexp(m)[1]) - 15
        y = (x * 2.0 ** -k).astype(np.float16)
        assert 2 ** 14 <= np.abs(y.astype(np.float64)).max() < 2 ** 15
        back = y.astype(np.float64) * 2.0 ** k
        keep = np.abs(x) >= m * 2.0 ** -32
        assert np.array_equal(back[keep], x[keep])
        # below 2^-32 of the largest: off by at most half an fp16 step at the bottom
        assert np.all(np.abs(back - x) <= 2.0 ** (k - 25))
