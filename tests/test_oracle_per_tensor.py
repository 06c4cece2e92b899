"""Pins of the oracle's per-tensor current-scaling E4M3 quantization: the
scale rule of "DeepSeek-V3 16B FSDP2 MXFP8/HiF8 训练设计" §3.2, torch's
float8_e4m3fn cast as an independent encoder, and invariants.  CPU only."""

import numpy as np
import torch

from oracle import codec, per_tensor
from block_quant_gemm_amd import workloads


def bf16(vals):
    t = torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_scale_rule_special_cases():
    assert per_tensor.pt_scale(bf16([448.0, -3.0])) == np.float32(1.0)
    assert per_tensor.pt_scale(bf16([0.0, -0.0])) == np.float32(1.0)       # amax 0
    assert per_tensor.pt_scale(bf16([1.0, np.nan])) == np.float32(1.0)     # invalid
    assert per_tensor.pt_scale(bf16([1.0, -np.inf])) == np.float32(1.0)
    assert per_tensor.pt_scale(np.zeros(0, np.uint16)) == np.float32(1.0)
    s = per_tensor.pt_scale(bf16([-896.0, 2.0]))
    assert s == np.float32(2.0)
    # FP32 division rounds: 1/448 is not exact
    s = per_tensor.pt_scale(bf16([1.0]))
    assert s == np.float32(np.float32(1.0) / np.float32(448.0))
    assert float(s) != 1.0 / 448.0


def test_amax_element_maps_to_448():
    x = workloads.bf16_normal((4096,), 1.0, seed=3, name="pt", outlier_frac=0.01,
                              outlier_scale=50.0)
    codes, s = per_tensor.pt_quantize(x)
    v = codec.bf16_bits_to_f64(x)
    i = np.argmax(np.abs(v))
    assert codes[i] & 0x7F == 0x7E
    assert np.all((codes & 0x7F) <= 0x7E)


def test_codes_match_torch_division_and_cast():
    """Independent route: torch float32 division then torch's e4m3fn cast."""
    x = workloads.bf16_normal((64, 512), 0.02, seed=4, name="pt2",
                              outlier_frac=0.005, outlier_scale=50.0)
    codes, s = per_tensor.pt_quantize(x)
    xt = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).float()
    q = xt / torch.tensor(s, dtype=torch.float32)
    ref = q.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_power_of_two_equivariance():
    x = workloads.bf16_normal((2048,), 1.0, seed=6, name="pt3")
    v = codec.bf16_bits_to_f64(x)
    c0, s0 = per_tensor.pt_quantize(x)
    for j in (-10, 5):
        c1, s1 = per_tensor.pt_quantize(bf16(v * 2.0 ** j))
        assert np.array_equal(c0, c1)
        assert s1 == np.float32(s0 * np.float32(2.0 ** j))


def test_nonfinite_inputs():
    x = np.array([0x3F80, 0x7FC0, 0xFF80, 0x7F80, 0xC000, 0xFFC0], np.uint16)
    codes, s = per_tensor.pt_quantize(x)        # 1, +NaN, -Inf, +Inf, -2, -NaN
    assert s == 1.0
    assert codes.tolist() == [0x38, 0x7F, 0xFE, 0x7E, 0xC0, 0xFF]


def test_given_amax_scale_rule():
    """The rule of §3.2 applied to a given amax: amax / 448 in FP32 when
    valid, 1.0 for zero, negative, NaN and infinite values."""
    assert per_tensor.pt_scale_of_amax(896.0) == np.float32(2.0)
    assert per_tensor.pt_scale_of_amax(1.0) == np.float32(np.float32(1.0) / np.float32(448.0))
    for bad in (0.0, -0.0, -5.0, np.nan, np.inf, -np.inf):
        assert per_tensor.pt_scale_of_amax(bad) == np.float32(1.0)


def test_given_amax_equals_two_pass_at_true_amax():
    """With the tensor's own max |x| (found here by numpy) the given-amax
    quantization is the two-pass one, special values included."""
    x = workloads.bf16_normal((4096,), 1.0, seed=12, name="pta", outlier_frac=0.01,
                              outlier_scale=30.0)
    v = codec.bf16_bits_to_f64(x)
    c0, s0 = per_tensor.pt_quantize(x)
    c1, s1 = per_tensor.pt_quantize_given_amax(x, np.abs(v).max())
    assert s0 == s1 and np.array_equal(c0, c1)
    y = np.array([0x3F80, 0x7FC0, 0xFF80, 0x7F80, 0xC000, 0xFFC0], np.uint16)
    c2, s2 = per_tensor.pt_quantize_given_amax(y, np.nan)
    assert s2 == 1.0 and c2.tolist() == [0x38, 0x7F, 0xFE, 0x7E, 0xC0, 0xFF]


def test_given_amax_power_of_two_closed_form():
    """amax = 448 * 2^j gives the scale 2^j exactly, so the codes are those of
    x * 2^-j (an exact scaling) encoded by torch's e4m3fn cast."""
    x = workloads.bf16_normal((2048,), 1.0, seed=13, name="ptb")
    xt = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).float()
    for j in (-3, 0, 4):
        c, s = per_tensor.pt_quantize_given_amax(x, 448.0 * 2.0 ** j)
        assert s == np.float32(2.0 ** j)
        ref = (xt * 2.0 ** -j).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(c, ref)


def test_dequant_error_relative():
    x = workloads.bf16_normal((8192,), 1.0, seed=8, name="pt4")
    codes, s = per_tensor.pt_quantize(x)
    v = codec.bf16_bits_to_f64(x)
    d = per_tensor.pt_dequantize(codes, s)
    a = np.abs(v) / np.float64(s)
    step = np.where(a < 2.0 ** -6, 2.0 ** -9,
                    2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    # two roundings: FP32 quotient (relative 2^-24) then E4M3 (half a step)
    bound = (step / 2 + a * 2.0 ** -23) * np.float64(s)
    assert np.all(np.abs(d - v) <= bound)


# ---------------------------------------------------------------------------
# per-group (per-expert) current scaling: [HP329] §3 and §3.2, one FP32 scale
# per leading group
# ---------------------------------------------------------------------------

def _groups(counts):
    counts = np.asarray(counts, np.int64)
    return workloads.offsets_from_counts(counts)


def test_per_group_scales_closed_form_and_empty_groups():
    """Each group's scale is its own amax / 448 (hand-picked amaxes whose
    quotients are exact), an empty group gets 1.0 ([HP329] §3.2: a scale of 1
    when there is no usable amax)."""
    offs = _groups([2, 0, 3, 1])
    x = bf16([[1.0, -3.5], [0.5, 2.0],                  # group 0: amax 3.5
              [-896.0, 1.0], [7.0, 0.0], [0.25, 448.0],  # group 2: amax 896
              [0.0, -0.0]])                             # group 3: amax 0
    codes, s = per_tensor.pg_quantize(x, offs)
    assert s.dtype == np.float32
    assert s.tolist() == [0.0078125, 1.0, 2.0, 1.0]
    # 3.5 / 0.0078125 = 448 -> 0x7E with its sign; 896 / 2 = 448
    assert codes[0, 1] == 0xFE and codes[2, 0] == 0xFE
    assert codes[4, 1] == 0x76            # 448 / 2 = 224 = 1.75 * 2^7: exponent field 14, mantissa 6
    assert codes[5].tolist() == [0x00, 0x80]             # signed zeros kept


def test_per_group_amax_elements_map_to_448():
    counts = [300, 1, 0, 77, 512]
    offs = _groups(counts)
    x = workloads.bf16_normal((sum(counts), 96), 1.0, seed=11, name="pg",
                              outlier_frac=0.01, outlier_scale=50.0)
    codes, s = per_tensor.pg_quantize(x, offs)
    v = codec.bf16_bits_to_f64(x)
    for e in range(len(counts)):
        lo, hi = offs[e], offs[e + 1]
        if hi == lo:
            assert s[e] == 1.0
            continue
        blk = np.abs(v[lo:hi])
        r, c = np.unravel_index(np.argmax(blk), blk.shape)
        assert codes[lo + r, c] & 0x7F == 0x7E
        assert np.all((codes[lo:hi] & 0x7F) <= 0x7E)


def test_per_group_matches_torch_division_and_cast():
    """Independent route per group: torch amax, FP32 division, e4m3fn cast."""
    counts = [129, 0, 31, 250]
    offs = _groups(counts)
    x = workloads.bf16_normal((sum(counts), 64), 0.02, seed=12, name="pg2",
                              outlier_frac=0.005, outlier_scale=50.0)
    codes, s = per_tensor.pg_quantize(x, offs)
    xt = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).float()
    for e in range(len(counts)):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        amax = xt[lo:hi].abs().max()
        se = amax / torch.tensor(448.0)
        assert np.float32(se.item()) == s[e]
        ref = (xt[lo:hi] / se).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        assert np.array_equal(codes[lo:hi], ref.numpy())


def test_per_group_equivariance_and_isolation():
    """Scaling one group by 2^j scales only its scale and leaves every code
    unchanged; a NaN in one group affects that group only."""
    counts = [40, 60, 25]
    offs = _groups(counts)
    x = workloads.bf16_normal((sum(counts), 32), 1.0, seed=13, name="pg3")
    c0, s0 = per_tensor.pg_quantize(x, offs)
    v = codec.bf16_bits_to_f64(x)
    v2 = v.copy()
    v2[offs[1]:offs[2]] *= 2.0 ** -7
    c1, s1 = per_tensor.pg_quantize(bf16(v2), offs)
    assert np.array_equal(c0, c1)
    assert s1[0] == s0[0] and s1[2] == s0[2]
    assert s1[1] == np.float32(s0[1] * np.float32(2.0 ** -7))
    xn = x.copy()
    xn[offs[2] + 3, 5] = 0x7FC0                           # NaN in group 2
    c2, s2 = per_tensor.pg_quantize(xn, offs)
    assert s2[2] == 1.0 and s2[0] == s0[0] and s2[1] == s0[1]
    assert np.array_equal(c2[:offs[2]], c0[:offs[2]])
    assert c2[offs[2] + 3, 5] == 0x7F


def test_per_group_dequantize_exact():
    counts = [3, 0, 2]
    offs = _groups(counts)
    codes = np.array([[0x38, 0xC0], [0x7E, 0x00], [0x01, 0x80],
                      [0x30, 0x48], [0xB8, 0x08]], np.uint8)
    s = np.array([0.5, 3.0, 2.0 ** -3], np.float32)
    d = per_tensor.pg_dequantize(codes, s, offs)
    # E4M3: 0x38 = 1, 0xC0 = -2, 0x7E = 448, 0x01 = 2^-9, 0x30 = 0.5, 0x48 = 4,
    # 0xB8 = -1, 0x08 = 2^-6
    exp = np.array([[0.5, -1.0], [224.0, 0.0], [2.0 ** -10, -0.0],
                    [2.0 ** -4, 0.5], [-(2.0 ** -3), 2.0 ** -9]])
    assert np.array_equal(d, exp)


def test_per_group_colwise_layout_and_codes():
    """The transposed copy: group e's rows appear as columns starting at its
    padded offset (multiples of 32), padding columns are +0 codes, and every
    code equals the row-major copy's (direction does not change the data)."""
    counts = [33, 0, 1, 64, 5]
    offs = _groups(counts)
    x = workloads.bf16_normal((sum(counts), 40), 1.0, seed=14, name="pgc",
                              outlier_frac=0.02, outlier_scale=20.0)
    cT, sT, poff = per_tensor.pg_quantize_colwise(x, offs)
    c, s = per_tensor.pg_quantize(x, offs)
    assert poff.tolist() == [0, 64, 64, 96, 160, 192]
    assert cT.shape == (40, 192)
    assert np.array_equal(sT, s)
    for e in range(len(counts)):
        lo, hi, p = offs[e], offs[e + 1], poff[e]
        assert np.array_equal(cT[:, p:p + hi - lo], c[lo:hi].T)
        assert np.all(cT[:, p + hi - lo:poff[e + 1]] == 0)
    # dequantized transposed copy times its scales reproduces the row-major values
    d = per_tensor.pg_dequantize(c, s, offs)
    for e in range(len(counts)):
        lo, hi, p = offs[e], offs[e + 1], poff[e]
        assert np.array_equal(per_tensor.pt_dequantize(cT[:, p:p + hi - lo], s[e]), d[lo:hi].T)
