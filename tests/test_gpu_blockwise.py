"""Parity of the blockwise FP8 comparison recipe (1x128 activation blocks,
128x128 weight blocks, FP32 scales, per-block promotion in the GEMM) with the
oracle, through the C ABI.  Quantizers bit-exact; GEMM outputs within the
oracle tolerance plus the matrix unit's truncation allowance of each block's
unit-scale product times the block's two scales."""

import numpy as np
import pytest
import torch

from block_quant_gemm_amd import mxq, workloads
from oracle import blockwise as bw
from oracle import codec, gemm
from tests import fp8_mode as f8
from tests.gpu_helpers import host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _strided_bf16(bits, pad):
    """Device BF16 view with row stride K + pad."""
    M, K = bits.shape
    buf = torch.zeros((M, K + pad), dtype=torch.bfloat16, device="cuda")
    buf[:, :K] = to_dev_bf16(bits)
    return buf[:, :K]


@pytest.mark.parametrize("M,K,pad", [(1, 128, 0), (37, 512, 0), (300, 2048, 0), (64, 384, 8),
                                     (5, 1408, 24)])
def test_act_quant_bit_exact(M, K, pad):
    say(f"blockwise act quant M={M} K={K} pad={pad}")
    x = workloads.bf16_normal((M, K), 1.0, seed=M + K, name="bwqa", outlier_frac=0.01,
                              outlier_scale=100.0)
    xd = _strided_bf16(x, pad) if pad else to_dev_bf16(x)
    q, s = mxq.fp8_quantize_blockwise_act(xd)
    rq, rs = bw.bw_quantize_act(x)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(q), rq)


def test_act_quant_special_blocks():
    vals = np.random.default_rng(3).normal(0, 1, (4, 512))
    vals[0, 5] = np.nan                    # NaN block
    vals[1, 200] = np.inf                  # Inf block
    vals[2, 256:384] = 0.0                 # zero block
    vals[3, 400] = 1e-38                   # tiny values: subnormal FP32 scale
    vals[3, 384:512] *= 1e-39
    bits = codec.bf16_round_to_bits(vals)
    q, s = mxq.fp8_quantize_blockwise_act(to_dev_bf16(bits))
    rq, rs = bw.bw_quantize_act(bits)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(q), rq)


@pytest.mark.parametrize("N,K,pad", [(128, 128, 0), (200, 256, 0), (1000, 512, 16),
                                     (10944, 2048, 0)])
def test_weight_quant_bit_exact(N, K, pad):
    say(f"blockwise weight quant N={N} K={K} pad={pad}")
    w = workloads.bf16_normal((N, K), 0.02, seed=N + K, name="bwqw")
    wd = _strided_bf16(w, pad) if pad else to_dev_bf16(w)
    q, s = mxq.fp8_quantize_blockwise_weight(wd)
    if N * K > 4_000_000:                  # full size: sampled block rows
        rows = np.r_[0:128, 5120:5248, 10880:N]
        rq, rs = bw.bw_quantize_weight(w[rows])
        sb = np.array([0, 40, 85])
        assert np.array_equal(host(s)[sb].view(np.uint32), rs.view(np.uint32))
        assert np.array_equal(host(q)[rows], rq)
        return
    rq, rs = bw.bw_quantize_weight(w)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(q), rq)


def _allowance(qa, sa, qw, sw, rows, cols):
    """Σ over 128-blocks of the unit-scale MFMA truncation allowance times
    the block's s_a * s_w, for entries (rows[i], cols[i])."""
    K = qa.shape[1]
    idx = np.arange(len(rows))
    ones = np.full((len(rows), 4), 127, np.uint8)
    T = np.zeros(len(rows))
    for b in range(K // 128):
        ks = slice(128 * b, 128 * b + 128)
        tb = f8.fp8_mfma_truncation_bound(qa[rows, ks], ones, qw[cols, ks], ones, idx, idx)
        T += tb * sa[rows, b].astype(np.float64) * sw[cols // 128, b].astype(np.float64)
    return T


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (200, 136, 256), (300, 1300, 384),
                                   (257, 520, 1408)])
@pytest.mark.parametrize("out", [mxq.OUT_BF16, mxq.OUT_FP32])
def test_blockwise_gemm(M, N, K, out):
    say(f"blockwise GEMM M={M} N={N} K={K} out={out}")
    a = workloads.bf16_normal((M, K), 1.0, seed=M * 3 + K, name="bga", outlier_frac=0.01,
                              outlier_scale=50.0)
    w = workloads.bf16_normal((N, K), 0.02, seed=N * 3 + K, name="bgw")
    qa, sa = bw.bw_quantize_act(a)
    qw, sw = bw.bw_quantize_weight(w)
    c = mxq.fp8_gemm_blockwise(to_dev(qa), to_dev(sa), to_dev(qw), to_dev(sw), out_dtype=out)
    Y, S = gemm.gemm_ref(bw.bw_dequantize_act(qa, sa), bw.bw_dequantize_weight(qw, sw))
    rows = np.repeat(np.arange(M), N)
    cols = np.tile(np.arange(N), M)
    T = _allowance(qa, sa, qw, sw, rows, cols).reshape(M, N)
    if out == mxq.OUT_FP32:
        ok = f8.check_fp32_extra(host(c).astype(np.float64), Y, S, T)
    else:
        ok = f8.check_bf16_extra(host(c), Y, S, T)
    say(f"  within tolerance: {ok.mean():.6f}")
    assert ok.all()


def test_blockwise_dense_ffn_forward_sampled():
    """The dense FFN gate/up forward 8192 x 10944 x 2048 (activations with 0.5 %
    outliers x50), quantized on the GPU; 3000 sampled outputs."""
    say("blockwise dense FFN forward 8192 x 10944 x 2048")
    d = workloads.dense_ffn(0)
    xq, xs = mxq.fp8_quantize_blockwise_act(to_dev_bf16(d["X"]))
    wq, ws = mxq.fp8_quantize_blockwise_weight(to_dev_bf16(d["W"]))
    c = mxq.fp8_gemm_blockwise(xq, xs, wq, ws)
    qa, sa, qw, sw = host(xq), host(xs), host(wq), host(ws)
    rng = np.random.default_rng(7)
    # the operands equal the oracle's on sampled rows / block rows
    r = np.sort(rng.choice(qa.shape[0], 8, replace=False))
    rq, rs = bw.bw_quantize_act(d["X"][r])
    assert np.array_equal(qa[r], rq) and np.array_equal(sa[r].view(np.uint32), rs.view(np.uint32))
    rq, rs = bw.bw_quantize_weight(d["W"][1280:1408])
    assert np.array_equal(qw[1280:1408], rq) and np.array_equal(sw[10:11].view(np.uint32),
                                                                rs.view(np.uint32))
    rows = rng.integers(0, qa.shape[0], 3000)
    cols = rng.integers(0, qw.shape[0], 3000)
    A = bw.bw_dequantize_act(qa[rows], sa[rows])
    sw_rows = sw[cols // 128]
    B = codec.e4m3_decode(qw[cols]) * np.repeat(sw_rows.astype(np.float64), 128, axis=1)
    idx = np.arange(3000)
    Y, S = gemm.gemm_ref_entries(A, B, idx, idx)
    T = _allowance(qa, sa, qw, sw, rows, cols)
    assert f8.check_bf16_extra(host(c)[rows, cols], Y, S, T).all()
