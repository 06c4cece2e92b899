"""Pins of the oracle's E4M3 / E8M0 / BF16 codecs against the pages' printed
values, the library casts the pages use (torch float8_e4m3fn, bfloat16), and
brute force.  CPU only."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codec
from tests.conftest import read_golden

ALL = np.arange(256, dtype=np.uint8)


def torch_e4m3_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ---- decode ------------------------------------------------------------

def test_format_table_golden():
    """E4M3 row of the format table ([FPBLOG] §二.2)."""
    g = {k: float(v) for k, v in read_golden("e4m3_format_table.txt")}
    vals = codec.e4m3_decode(ALL)
    finite = vals[np.isfinite(vals)]
    pos = finite[finite > 0]
    assert finite.max() == g["max"]
    min_normal = codec.e4m3_decode(0x08)
    assert float(f"{min_normal:.2e}") == g["min_normal"]
    assert float(f"{pos.min():.2e}") == g["min_subnormal"]
    assert codec.e4m3_decode(0x39) - codec.e4m3_decode(0x38) == g["eps"]
    assert codec.e4m3_decode(0x38) == 1.0
    # General formula of §二.1 with E=4, M=3 for min normal / subnormal.
    assert min_normal == 2.0 ** (2 - 2 ** 3)
    assert pos.min() == 2.0 ** (2 - 2 ** 3 - 3)
    assert g["bias"] == codec.E4M3_BIAS


def test_bit_patterns_golden():
    """Printed values of individual codes ([FPBLOG] §九.1)."""
    for code, value in read_golden("e4m3_bit_patterns.txt"):
        got = codec.e4m3_decode(int(code, 16))
        if value == "nan":
            assert np.isnan(got)
        else:
            assert got == float(value)


def test_decode_matches_torch_for_all_codes():
    ours = codec.e4m3_decode(ALL)
    ref = torch_e4m3_decode(ALL)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(ours[m], ref[m])
    assert np.array_equal(np.signbit(ours[m]), np.signbit(ref[m]))


def test_only_nan_codes_are_s1111111():
    nan_codes = ALL[np.isnan(codec.e4m3_decode(ALL))]
    assert sorted(nan_codes.tolist()) == [0x7F, 0xFF]
    assert not np.isinf(codec.e4m3_decode(ALL)).any()


def test_decode_monotone_positive():
    v = codec.e4m3_decode(np.arange(0, 0x7F))
    assert np.all(np.diff(v) > 0)


# ---- encode ------------------------------------------------------------

def test_exhaustive_round_trip():
    vals = codec.e4m3_decode(ALL)
    enc = codec.e4m3_encode(vals)
    finite = ~np.isnan(vals)
    assert np.array_equal(enc[finite], ALL[finite])     # incl. -0 -> 0x80
    assert set(enc[~finite].tolist()) == {0x7F, 0xFF}


def _positive_grid():
    return codec.e4m3_decode(np.arange(0, 0x7F))        # 0 .. 448


def test_midpoints_go_to_even_code():
    g = _positive_grid()
    mids = (g[:-1] + g[1:]) / 2                          # exact in float64
    lo = np.arange(0, 0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(codec.e4m3_encode(mids), expect)
    assert np.array_equal(codec.e4m3_encode(-mids), expect | 0x80)
    # One float64 ulp either side of the midpoint goes to the nearer code.
    below = np.nextafter(mids, 0)
    above = np.nextafter(mids, np.inf)
    assert np.array_equal(codec.e4m3_encode(below), lo.astype(np.uint8))
    assert np.array_equal(codec.e4m3_encode(above), (lo + 1).astype(np.uint8))


def _brute_force_encode(v):
    """Nearest positive grid value by exhaustive search, ties to the even
    code, saturating above 448.  Exact comparisons with Fractions."""
    grid = [Fraction(float(x)) for x in _positive_grid()]
    a = Fraction(abs(v))
    if a >= 448:
        code = 0x7E
    else:
        best = min(range(len(grid)), key=lambda i: (abs(grid[i] - a), i % 2))
        code = best
    return code | (0x80 if np.signbit(v) else 0)


def test_encode_matches_brute_force():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(300) * 10.0 ** rng.uniform(-4, 3, 300),
        rng.uniform(-500, 500, 100),
        [0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -10 * 1.0000001,
         0.0146484375, 447.9, 448.0, 460.0, 464.0, 470.0, 1e30, -1e30],
    ])
    got = codec.e4m3_encode(vals)
    for v, c in zip(vals, got):
        assert c == _brute_force_encode(v), v


def test_encode_matches_torch_cast_in_range():
    """torch's float32 -> float8_e4m3fn cast rounds to nearest even; it is an
    independent implementation for |v| <= 448."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-5, 2.6, 200000))
    x = x.astype(np.float32)
    x = x[np.abs(x) <= 448]
    ours = codec.e4m3_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_saturation_nan_and_signed_zero():
    enc = codec.e4m3_encode
    assert enc(np.array([448.0, 449.0, 1e9, np.inf]))[()].tolist() == [0x7E] * 4
    assert enc(np.array([-448.0, -1e9, -np.inf])).tolist() == [0xFE] * 3
    assert enc(np.array([np.nan])).tolist() == [0x7F]
    assert enc(np.array([-np.nan])).tolist() == [0xFF]
    assert enc(np.array([0.0, -0.0, -1e-30])).tolist() == [0x00, 0x80, 0x80]
    # subnormal / normal boundary: 15/16 * 2^-6 is the midpoint of 7*2^-9 and 2^-6
    assert enc(np.array([0.0146484375])).tolist() == [0x08]
    # tie at 1.0625 between 1.0 (0x38) and 1.125 (0x39) -> even 0x38
    assert enc(np.array([1.0625, 1.1875])).tolist() == [0x38, 0x3A]


class _HalfUpNumpy:
    """numpy with rint replaced by round-half-up: a plausible planted mistake."""

    def __getattr__(self, k):
        return getattr(np, k)

    @staticmethod
    def rint(x):
        return np.floor(np.asarray(x) + 0.5)


def test_planted_rounding_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(codec, "np", _HalfUpNumpy())
    with pytest.raises(AssertionError):
        test_midpoints_go_to_even_code()


# ---- E8M0 ----------------------------------------------------------------

def test_e8m0_decode():
    c = np.arange(256)
    v = codec.e8m0_decode(c)
    assert np.isnan(v[255]) and np.isfinite(v[:255]).all()
    assert v[127] == 1.0 and v[0] == 2.0 ** -127 and v[254] == 2.0 ** 127
    # E8M0 with bias 127 is the FP32 exponent field: 2^(c-127) has FP32 bits c<<23
    f32 = np.array(v[1:255], dtype=np.float32).view(np.uint32)
    assert np.array_equal(f32, (c[1:255].astype(np.uint32) << 23))


# ---- BF16 --------------------------------------------------------------

def test_bf16_rne_golden():
    for x, expect in read_golden("bf16_rne_examples.txt"):
        assert codec.bf16_round(np.array([float(x)]))[0] == float(expect)


def test_bf16_round_matches_torch_from_float32():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-40, 38, 200000))
    x = x.astype(np.float32)
    x = x[np.isfinite(x)]
    ours = codec.bf16_round_to_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_all_patterns_fixed_points():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = codec.bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    assert np.array_equal(codec.bf16_round_to_bits(v[fin]), bits[fin])
    # float32 widening agrees with torch's bfloat16 -> float32
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(v[fin], ref[fin].astype(np.float64))
