"""Pins of the oracle's SwiGLU and of the MX copies of its output (the fused
gate/up producer), and of the interval checker used on the kernel's codes.
Closed forms of the logistic function, torch's SiLU in float64 as an
independent routine, a hand-worked block, brute force per block on a tiny
grouped case, and planted mistakes.  CPU only."""

import math

import numpy as np
import torch

from oracle import swiglu as sw
from oracle.mx import padded_offsets
from tests.mx_interval import mx_valid
from tests.test_oracle_mx import brute_codes, brute_exponent


def test_silu_closed_forms():
    # sigmoid(ln k) = k / (k + 1), so silu(ln k) = ln k * k / (k + 1)
    for k in (1, 2, 3, 7, 100):
        x = math.log(k)
        assert abs(sw.silu(x) - x * k / (k + 1)) <= 1e-15 * max(1.0, abs(x))
    assert sw.silu(0.0) == 0.0


def test_silu_odd_part_is_identity():
    # sigmoid(x) + sigmoid(-x) = 1  =>  silu(x) - silu(-x) = x
    x = np.random.default_rng(1).normal(0, 6, 10_000)
    np.testing.assert_allclose(sw.silu(x) - sw.silu(-x), x, rtol=1e-14, atol=1e-14)


def test_silu_limits():
    assert sw.silu(50.0) == 50.0                      # 50 e^-50 is below half an ulp of 50
    assert sw.silu(800.0) == 800.0
    r = sw.silu(-800.0)                               # exp overflows: -800 / inf
    assert r == 0.0 and math.copysign(1.0, r) == -1.0


def test_silu_matches_torch_float64():
    x = np.random.default_rng(2).normal(0, 4, 100_000)
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(sw.silu(x), ref, rtol=2e-16 * 4, atol=1e-300)


def test_swiglu_is_silu_times_up():
    rng = np.random.default_rng(3)
    g, u = rng.normal(size=(8, 64)), rng.normal(size=(8, 64))
    np.testing.assert_array_equal(sw.swiglu(g, np.ones_like(u)), sw.silu(g))
    np.testing.assert_allclose(sw.swiglu(g, 3 * u), 3 * sw.swiglu(g, u), rtol=1e-15)


def test_split_gate_up_takes_halves():
    G = np.arange(12.0).reshape(2, 6)
    U = -G
    g, u = sw.split_gate_up(np.concatenate([G, U], axis=1))
    np.testing.assert_array_equal(g, G)
    np.testing.assert_array_equal(u, U)


def test_hand_worked_block():
    """Row block with h = [50, -50, 0, ..., 0]: amax 50, floor(log2 50) = 5,
    shared exponent 5 - 8 = -3 (scale code 124); 50 * 2^3 = 400 lies halfway
    between the E4M3 neighbours 384 = 1.100b * 2^8 (even mantissa) and
    416 = 1.101b * 2^8, so it rounds to 384: code 0x7C (sign 0, exponent
    field 8 + 7 = 15, mantissa 100b); -50 gives 0xFC."""
    g = np.zeros((1, 32))
    u = np.zeros((1, 32))
    g[0, 0], u[0, 0] = 50.0, 1.0
    g[0, 1], u[0, 1] = 50.0, -1.0
    hq, hs, hqT, hsT, poff = sw.swiglu_mx(g, u, np.array([0, 1]))
    assert hs[0, 0] == 124
    assert hq[0, 0] == 0x7C and hq[0, 1] == 0xFC and not hq[0, 2:].any()
    # the column copy pads the single row to a block of 32
    assert list(poff) == [0, 32]
    assert hqT.shape == (32, 32)
    # column 0 is the block [50, 0 x 31] and column 1 [-50, 0 x 31]: the same
    # amax, scale and codes
    assert hsT[0, 0] == 124 and hsT[1, 0] == 124 and not hsT[2:, 0].any()
    assert hqT[0, 0] == 0x7C and hqT[1, 0] == 0xFC and not hqT[:, 1:].any()


def _brute_block(vals):
    amax = float(np.max(np.abs(vals)))
    e = brute_exponent(amax) if amax > 0 else -127
    return brute_codes(np.asarray(vals) * 2.0 ** (-e)), e + 127


def test_swiglu_mx_against_brute_force_per_block():
    rng = np.random.default_rng(4)
    counts = [5, 0, 40, 33, 1]
    offs = np.concatenate([[0], np.cumsum(counts)])
    M, F = int(offs[-1]), 64
    g = rng.normal(0, 3, (M, F)) * np.exp2(rng.integers(-6, 6, (M, F)))
    u = rng.normal(0, 1, (M, F))
    h = sw.swiglu(g, u)
    hq, hs, hqT, hsT, poff = sw.swiglu_mx(g, u, offs)
    np.testing.assert_array_equal(poff, padded_offsets(offs))
    for m in range(M):
        for b in range(F // 32):
            c, s = _brute_block(h[m, 32 * b:32 * b + 32])
            np.testing.assert_array_equal(hq[m, 32 * b:32 * b + 32], c)
            assert hs[m, b] == s
    for e in range(len(counts)):
        lo, hi, plo = int(offs[e]), int(offs[e + 1]), int(poff[e])
        rows = np.zeros((int(poff[e + 1]) - plo, F))
        rows[:hi - lo] = h[lo:hi]
        for k in range(F):
            for b in range(rows.shape[0] // 32):
                c, s = _brute_block(rows[32 * b:32 * b + 32, k])
                np.testing.assert_array_equal(hqT[k, plo + 32 * b:plo + 32 * b + 32], c)
                assert hsT[k, plo // 32 + b] == s


def _sample_h(seed=6, R=16, C=128):
    rng = np.random.default_rng(seed)
    return rng.normal(0, 1, (R, C)) * np.exp2(rng.integers(-3, 3, (R, C)))


def test_interval_checker_exact_bounds_equal_oracle():
    h = _sample_h()
    from oracle.mx import quantize_blocks
    q, s = quantize_blocks(h.reshape(16, 4, 32))
    q = q.reshape(16, 128)
    ok_c, ok_s, unique = mx_valid(q, s, h, h)
    assert ok_c.all() and ok_s.all() and unique.all()
    # a planted code one step off is rejected where the value is not zero
    bad = q.copy()
    i = np.flatnonzero(bad.reshape(-1) & 0x7F)[7]
    bad.reshape(-1)[i] ^= 1
    assert not mx_valid(bad, s, h, h)[0].reshape(-1)[i]
    # a planted scale one step off is rejected
    bad_s = s.copy()
    bad_s[3, 2] += 1
    assert not mx_valid(q, bad_s, h, h)[1][3, 2]


def test_interval_checker_accepts_either_side_of_a_tie():
    # 400 * 2^-3 = 50: a tiny interval around 50 admits codes 0x7C (384) and
    # 0x7D (416) at scale code 124, and nothing else
    lo = np.zeros((1, 32)); hi = np.zeros((1, 32))
    lo[0, 0], hi[0, 0] = 50.0 - 1e-9, 50.0 + 1e-9
    lo[0, 1], hi[0, 1] = 60.0, 60.0                  # amax pins the scale to 124
    s = np.array([[124]], np.uint8)
    for code, want in ((0x7C, True), (0x7D, True), (0x7B, False), (0x7E, False)):
        q = np.zeros((1, 32), np.uint8)
        q[0, 0] = code
        q[0, 1] = 0x7E                                # 60 * 8 = 480 saturates to 448
        ok_c, ok_s, unique = mx_valid(q, s, lo, hi)
        assert ok_s.all() and ok_c[0, 0] == want
        assert not unique[0, 0] and unique[0, 1]


def test_interval_checker_scale_at_a_binade_edge():
    # amax in [255.99, 256.01] straddles 2^8: exponents 7-8 = -1 and 0 both valid
    lo = np.zeros((1, 32)); hi = np.zeros((1, 32))
    lo[0, 0], hi[0, 0] = 255.99, 256.01
    q = np.zeros((1, 32), np.uint8)
    for code, want in ((126, True), (127, True), (125, False), (128, False)):
        s = np.array([[code]], np.uint8)
        q[0, 0] = 0x7E if code == 126 else 0x78     # 448 at 2^-1 scale; 256 at 2^0
        assert mx_valid(q, s, lo, hi)[1][0, 0] == want
