"""Number codecs of the oracle: E4M3 (fn), E8M0 and BF16.  Test infrastructure.

All arithmetic is exact: values are held in float64, which represents every
BF16, FP32, E4M3 and power-of-two-scaled E4M3 value used here without error,
and rounding decisions are taken with ``numpy.rint`` (round half to even) on
exactly scaled quantities.
"""

import numpy as np

# E4M3 (fn) layout: 1 sign, 4 exponent, 3 mantissa bits, bias 7.
# [FPBLOG] §二.2, bit-layout figure and format table.
E4M3_BIAS = 7
E4M3_MAX = 448.0            # S.1111.110 = 1.75 * 2^8 ([FPBLOG] §二.2, E4M3 note)
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_MIN_SUBNORMAL = 2.0 ** -9
E4M3_NAN_CODE = 0x7F        # S.1111.111 is the only NaN pattern; there is no Inf
E4M3_EMAX = 8               # floor(log2(448))

E8M0_BIAS = 127             # same bias as the FP32 exponent field
E8M0_NAN_CODE = 0xFF


def e4m3_decode(codes):
    """Decode E4M3 (fn) codes to float64.

    Value formula from [FPBLOG] §二.1: a normal number is (-1)^s * 1.m *
    2^(e - bias); exponent field 0 is subnormal, (-1)^s * 0.m * 2^(1 - bias).
    E4M3 departs from the IEEE convention for exponent field all-ones
    ([FPBLOG] §二.2, E4M3 note): S.1111.110 is the largest finite value 448 and
    only S.1111.111 is NaN.
    """
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    normal = sign * (1.0 + m / 8.0) * np.ldexp(1.0, e - E4M3_BIAS)
    subnormal = sign * (m / 8.0) * np.ldexp(1.0, 1 - E4M3_BIAS)
    val = np.where(e == 0, subnormal, normal)
    val = np.where((e == 0xF) & (m == 0x7), np.copysign(np.nan, sign), val)
    return val.astype(np.float64)


def e4m3_encode(values):
    """Round exact float64 values to E4M3 (fn) codes (uint8).

    Round to nearest, ties to even mantissa; any magnitude >= 448 (and +-Inf)
    saturates to 448; NaN maps to 0x7F with the input's sign bit; the sign of
    zero is kept.  Grid: subnormals are k * 2^-9 for k = 0..7 ([FPBLOG] §二.1
    subnormal rule with bias 7), normals in binade [2^E, 2^(E+1)) are spaced
    2^(E-3).
    """
    v = np.asarray(values, dtype=np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    nan = np.isnan(v)
    a_safe = np.where(nan | np.isinf(a), 0.0, a)

    # Subnormal range (below the smallest normal 2^-6): multiples of 2^-9.
    # k == 8 rounds up into the smallest normal, whose code is also 8.
    k_sub = np.rint(np.ldexp(np.minimum(a_safe, 1.0), 9)).astype(np.int64)

    # Normal range: binade exponent E = floor(log2 a); frexp is exact.
    _, fx = np.frexp(np.where(a_safe > 0, a_safe, 1.0))
    E = fx.astype(np.int64) - 1
    q = np.rint(np.ldexp(a_safe, (3 - E))).astype(np.int64)   # in [8, 16]
    carry = q == 16
    E = np.where(carry, E + 1, E)
    q = np.where(carry, 8, q)
    k_norm = ((E + E4M3_BIAS) << 3) | (q - 8)

    code = np.where(a_safe < E4M3_MIN_NORMAL, k_sub, k_norm)
    code = np.where(a >= E4M3_MAX, 0x7E, code)          # saturate, incl. Inf
    code = code | np.where(neg, 0x80, 0)
    code = np.where(nan, E4M3_NAN_CODE | np.where(neg, 0x80, 0), code)
    return code.astype(np.uint8)


def e8m0_decode(codes):
    """E8M0 scale code -> float64 power of two 2^(c - 127); 0xFF is NaN."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == E8M0_NAN_CODE, np.nan, np.ldexp(1.0, c - E8M0_BIAS))


def bf16_bits_to_f64(bits):
    """BF16 bit patterns (uint16) -> float64.

    BF16 is the upper 16 bits of FP32 ([FPBLOG] §二.2, BF16 note), so the
    value is the FP32 whose bits are ``b << 16``; widening is exact.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):       # signalling-NaN patterns
        return b.view(np.float32).astype(np.float64)


def bf16_round(values):
    """Round float64 values to the nearest BF16 value, ties to even, as float64.

    [FPBLOG] §二.2 (BF16 note): conversion to BF16 rounds to nearest even
    rather than truncating.  BF16 has 8 significant bits; normal binade
    [2^E, 2^(E+1)) is spaced 2^(E-7); below 2^-126 the spacing is 2^-133.
    Magnitudes at or above the midpoint past the largest finite BF16 become
    Inf.
    """
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    finite = np.isfinite(v)
    a_safe = np.where(finite & (a > 0), a, 1.0)
    _, fx = np.frexp(a_safe)
    E = np.maximum(fx.astype(np.int64) - 1, -126)
    step_exp = E - 7
    r = np.ldexp(np.rint(np.ldexp(a_safe, -step_exp)), step_exp)
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(r > bf16_max, np.inf, r)
    r = np.where(finite & (a > 0), r, a)
    return np.copysign(r, v)


def bf16_round_to_bits(values):
    """float64 -> BF16 bit patterns (uint16), via :func:`bf16_round`."""
    r = bf16_round(values)
    bits = r.astype(np.float32).view(np.uint32)   # exact: r is a BF16 value
    out = (bits >> np.uint32(16)).astype(np.uint16)
    # NaN inputs: a quiet NaN with the input's sign.
    nan = np.isnan(np.asarray(values, dtype=np.float64))
    return np.where(nan, (out & np.uint16(0x8000)) | np.uint16(0x7FC0), out).astype(np.uint16)
