"""Pins of the oracle's MX block quantization (row, col, grouped col) against
a hand-worked block, brute force over every BF16 pattern, and invariants the
definition implies.  CPU only."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import codec, mx
from block_quant_gemm_amd import workloads
from tests.conftest import read_golden

GRID = codec.e4m3_decode(np.arange(0, 0x7F))          # 0 .. 448, increasing


def bf16(vals):
    import torch
    t = torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def brute_exponent(amax):
    """Smallest e >= -127 with amax < 2^(e+9), found by search."""
    e = -127
    while amax >= 2.0 ** (e + 9):
        e += 1
    return e


def brute_codes(scaled):
    """Nearest positive grid point by bracketing search (ties to even code),
    saturating at 448; sign applied afterwards."""
    a = np.abs(scaled)
    idx = np.searchsorted(GRID, a)                    # GRID[idx-1] < a <= GRID[idx]
    idx = np.clip(idx, 1, len(GRID) - 1)
    lo, hi = GRID[idx - 1], GRID[idx]
    dlo, dhi = a - lo, hi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (idx % 2 == 0))
    code = np.where(pick_hi, idx, idx - 1)
    code = np.where(a == 0, 0, code)
    code = np.where(a >= 448, 0x7E, code)
    return (code | np.where(np.signbit(scaled), 0x80, 0)).astype(np.uint8)


def test_hand_worked_block():
    rows = read_golden("mx_block_hand.txt")
    assert rows[0][0] == "scale"
    scale = int(rows[0][1], 16)
    x = np.zeros((1, 32), np.uint16)
    exp = np.zeros(32, np.uint8)
    for i, (b, c) in enumerate(rows[1:]):
        x[0, i] = int(b, 16)
        exp[i] = int(c, 16)
    codes, scales = mx.mx_quantize_rowwise(x)
    assert scales.tolist() == [[scale]]
    assert codes[0].tolist() == exp.tolist()


ANCHORS = [2.0 ** -133, 2.0 ** -126, 2.0 ** -119, 2.0 ** -60, 1.0 / 3, 1.0,
           255.0, 448.0, 3.0e4, 2.0 ** 100, 3.0e38]


@pytest.mark.parametrize("anchor", ANCHORS)
def test_every_bf16_pattern_against_brute_force(anchor):
    """Block = [anchor, p, 0, ...] for each of the 65536 BF16 patterns p."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = np.zeros((65536, 32), np.uint16)
    x[:, 0] = bf16([anchor])[0]
    x[:, 1] = pats
    codes, scales = mx.mx_quantize_rowwise(x)

    a_val = codec.bf16_bits_to_f64(x[0, 0])
    p_val = codec.bf16_bits_to_f64(pats)
    finite = np.isfinite(p_val)
    amax = np.maximum(np.abs(p_val[finite]), a_val)
    e_tab = {}
    e = np.array([e_tab.setdefault(v, brute_exponent(v)) for v in amax.tolist()])
    assert np.array_equal(scales[finite, 0], (e + 127).astype(np.uint8))
    exp_p = brute_codes(p_val[finite] * 2.0 ** (-e.astype(np.float64)))
    exp_a = brute_codes(a_val * 2.0 ** (-e.astype(np.float64)))
    assert np.array_equal(codes[finite, 1], exp_p)
    assert np.array_equal(codes[finite, 0], exp_a)
    assert np.all(codes[finite, 2:] == 0)
    # NaN / Inf patterns poison the whole block.
    assert np.all(scales[~finite, 0] == 0xFF)
    assert np.all(codes[~finite] == 0x7F)


def _sample(M=96, K=256, seed=5):
    return workloads.bf16_normal((M, K), 1.0, seed=seed, name="mxpin",
                                 outlier_frac=0.01, outlier_scale=100.0)


def test_largest_code_in_top_binade():
    x = _sample()
    codes, scales = mx.mx_quantize_rowwise(x)
    cb = codes.reshape(x.shape[0], -1, 32) & 0x7F
    top = cb.max(axis=-1)
    assert np.all((top >= 0x78) & (top <= 0x7E))
    assert np.all(scales > 0)


def test_power_of_two_equivariance():
    x = _sample()
    v = codec.bf16_bits_to_f64(x)
    for j in (-7, -1, 3, 20):
        xj = bf16(v * 2.0 ** j)
        assert np.array_equal(codec.bf16_bits_to_f64(xj), v * 2.0 ** j)   # exact
        c0, s0 = mx.mx_quantize_rowwise(x)
        c1, s1 = mx.mx_quantize_rowwise(xj)
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1.astype(int), s0.astype(int) + j)


def test_dequant_error_bound():
    x = _sample()
    v = codec.bf16_bits_to_f64(x)
    codes, scales = mx.mx_quantize_rowwise(x)
    d = mx.mx_dequantize(codes, scales)
    s = np.repeat(codec.e8m0_decode(scales), 32, axis=1)
    a = np.abs(v) / s                         # magnitude on the E4M3 grid scale
    # half the grid step at that magnitude
    step = np.where(a < 2.0 ** -6, 2.0 ** -9,
                    2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    bound = np.where(a >= 448, (a - 448), step / 2) * s
    assert np.all(np.abs(d - v) <= bound)


def test_special_blocks():
    x = np.zeros((1, 96), np.uint16)
    x[0, 32:64] = bf16(np.linspace(-1, 1, 32))
    x[0, 40] = 0x7F80                     # +Inf in block 1
    x[0, 64:96] = bf16(np.linspace(-1, 1, 32))
    x[0, 70] = 0x7FC1                     # NaN in block 2
    x[0, 5] = 0x8000                      # -0 in the all-zero block 0
    codes, scales = mx.mx_quantize_rowwise(x)
    assert scales.tolist() == [[0, 0xFF, 0xFF]]
    assert np.all(codes[0, 32:] == 0x7F)
    assert codes[0, 5] == 0x80 and np.all(np.delete(codes[0, :32], 5) == 0)


def test_tiny_amax_clamps_exponent():
    x = np.zeros((1, 32), np.uint16)
    x[0, 0] = 0x0001                      # 2^-133, smallest BF16 subnormal
    x[0, 1] = 0x0080                      # 2^-126
    codes, scales = mx.mx_quantize_rowwise(x)
    assert scales[0, 0] == 0
    # 2^-133 * 2^127 = 2^-6 -> 0x08 ; 2^-126 * 2^127 = 2 -> 0x40
    assert codes[0, 0] == 0x08 and codes[0, 1] == 0x40


def test_colwise_is_blocks_down_columns():
    x = _sample(M=64, K=96, seed=7)
    cT, sT = mx.mx_quantize_colwise(x)
    assert cT.shape == (96, 64) and sT.shape == (96, 2)
    v = codec.bf16_bits_to_f64(x)
    for k in range(0, 96, 13):
        for b in range(2):
            col = v[32 * b: 32 * b + 32, k]
            c, s = mx.quantize_blocks(col.reshape(1, 32))
            assert np.array_equal(cT[k, 32 * b: 32 * b + 32], c[0])
            assert sT[k, b] == s[0]


def test_grouped_colwise_pads_each_group():
    K = 64
    counts = np.array([40, 0, 1, 32, 0, 70, 0])
    offs = workloads.offsets_from_counts(counts)
    x = _sample(M=int(counts.sum()), K=K, seed=9)
    cT, sT, poff = mx.mx_quantize_grouped_colwise(x, offs)
    assert poff.tolist() == [0, 64, 64, 96, 128, 128, 224, 224]
    assert cT.shape == (K, 224) and sT.shape == (K, 7)
    for g in range(len(counts)):
        lo, hi, plo, phi = offs[g], offs[g + 1], poff[g], poff[g + 1]
        if phi == plo:
            continue
        pad = np.zeros((phi - plo, K), np.uint16)
        pad[: hi - lo] = x[lo:hi]
        # group alone, padded with +0 rows, then quantized down the columns
        ref_c = np.zeros((K, phi - plo), np.uint8)
        ref_s = np.zeros((K, (phi - plo) // 32), np.uint8)
        v = codec.bf16_bits_to_f64(pad)
        for k in range(K):
            c, s = mx.quantize_blocks(v[:, k].reshape(-1, 32))
            ref_c[k] = c.ravel()
            ref_s[k] = s
        assert np.array_equal(cT[:, plo:phi], ref_c)
        assert np.array_equal(sT[:, plo // 32: phi // 32], ref_s)
        assert np.all(cT[:, plo + (hi - lo): phi] == 0)     # padding rows


def test_exponent_rule_fraction_check():
    """floor(log2 amax) - 8 checked exactly with Fractions on random amax."""
    rng = np.random.default_rng(11)
    v = codec.bf16_bits_to_f64(bf16(rng.standard_normal(2000) * 10.0 **
                                    rng.uniform(-30, 30, 2000)))
    v = np.abs(v[v != 0])
    e, nf = mx.block_shared_exponent(v)
    assert not nf.any()
    for a, ee in zip(v.tolist(), e.tolist()):
        fa = Fraction(a)
        if ee > -127:
            assert Fraction(2) ** (ee + 8) <= fa < Fraction(2) ** (ee + 9)
        else:
            assert fa < Fraction(2) ** (-127 + 9)
