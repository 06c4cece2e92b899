"""Pins of the blockwise (1x128 activation, 128x128 weight, FP32 scale)
oracle: torch's amax, FP32 division and float8_e4m3fn cast per block as an
independent encoder, a hand-worked exact block, outlier isolation (the
recipe's purpose), partial weight blocks, and the promoted sum of per-block
products against the dequantized matmul.  CPU only."""

import numpy as np
import torch

from block_quant_gemm_amd import workloads
from oracle import blockwise as bw
from oracle import codec, gemm


def _torch_block(vals32):
    """Codes of one block by torch: scale = amax/448 (FP32) or 1, then cast."""
    t = torch.from_numpy(vals32)
    amax = t.abs().max()
    s = amax / torch.tensor(448.0) if torch.isfinite(amax) and amax > 0 else torch.tensor(1.0)
    q = (t / s).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy(), np.float32(s.item())


def test_act_blocks_match_torch_per_block():
    x = workloads.bf16_normal((6, 512), 1.0, seed=1, name="bwx", outlier_frac=0.02,
                              outlier_scale=80.0)
    q, s = bw.bw_quantize_act(x)
    x32 = codec.bf16_bits_to_f64(x).astype(np.float32)
    for m in range(6):
        for b in range(4):
            tq, ts = _torch_block(x32[m, 128 * b:128 * b + 128].copy())
            assert s[m, b] == ts
            np.testing.assert_array_equal(q[m, 128 * b:128 * b + 128], tq)


def test_weight_blocks_match_torch_per_block_with_partial_rows():
    w = workloads.bf16_normal((200, 256), 0.02, seed=2, name="bww")
    q, s = bw.bw_quantize_weight(w)
    assert s.shape == (2, 2)
    w32 = codec.bf16_bits_to_f64(w).astype(np.float32)
    for r, rows in enumerate((slice(0, 128), slice(128, 200))):
        for b in range(2):
            blk = w32[rows, 128 * b:128 * b + 128].copy()
            tq, ts = _torch_block(blk)
            assert s[r, b] == ts
            np.testing.assert_array_equal(q[rows, 128 * b:128 * b + 128], tq)


def test_hand_worked_exact_block():
    """amax = 448 * 2^-4 = 28: scale 2^-4 exactly, so every value on the E4M3
    grid times 2^-4 encodes exactly and dequantizes to itself."""
    grid = codec.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))      # 0 .. 448
    vals = np.concatenate([grid[::-1][:64], -grid[:64]]) * 2.0 ** -4  # 128 values, max 28
    bits = codec.bf16_round_to_bits(vals)
    assert np.array_equal(codec.bf16_bits_to_f64(bits), vals)          # all BF16-exact
    q, s = bw.bw_quantize_act(bits[None, :])
    assert s[0, 0] == np.float32(2.0 ** -4)
    np.testing.assert_array_equal(bw.bw_dequantize_act(q, s)[0], vals)


def test_outlier_only_affects_its_block():
    x = workloads.bf16_normal((4, 1024), 1.0, seed=3, name="bwo")
    q0, s0 = bw.bw_quantize_act(x)
    xo = x.copy()
    xo[2, 300] = codec.bf16_round_to_bits(np.array([5000.0]))[0]         # block 2 of row 2
    q1, s1 = bw.bw_quantize_act(xo)
    changed = s1 != s0
    assert changed[2, 2] and changed.sum() == 1
    same = np.ones((4, 1024), bool)
    same[2, 256:384] = False
    np.testing.assert_array_equal(q1[same], q0[same])


def test_promoted_block_sum_equals_dequantized_matmul():
    """sum_b s_a[m,b] s_w[n/128,b] (Q_a Q_wᵀ over block b), each block product
    exact, equals the matmul of the dequantized operands."""
    a = workloads.bf16_normal((5, 384), 1.0, seed=4, name="bwa")
    w = workloads.bf16_normal((130, 384), 0.05, seed=4, name="bwb")
    qa, sa = bw.bw_quantize_act(a)
    qw, sw = bw.bw_quantize_weight(w)
    Y, _ = gemm.gemm_ref(bw.bw_dequantize_act(qa, sa), bw.bw_dequantize_weight(qw, sw))
    va, vw = codec.e4m3_decode(qa), codec.e4m3_decode(qw)
    P = np.zeros((5, 130))
    for b in range(3):
        ks = slice(128 * b, 128 * b + 128)
        blockprod = va[:, ks] @ vw[:, ks].T                           # exact in float64
        P += blockprod * sa[:, b:b + 1].astype(np.float64) * \
            np.repeat(sw[:, b].astype(np.float64), 128)[None, :130]
    np.testing.assert_allclose(P, Y, rtol=1e-12, atol=1e-12)
