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
