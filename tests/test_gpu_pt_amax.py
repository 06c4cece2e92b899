"""Per-tensor current scaling with the amax taken in the producing GEMM's
epilogue ("Transformer 与 LLM（06）：浮点格式、数值稳定性与混合精度" §七.2:
the amax pass is the extra read of current scaling, and the matmul that
produces the tensor can supply it).  Through the C ABI:

- fp8_gemm_per_tensor_amax writes the same C as fp8_gemm_per_tensor, bit for
  bit, and its amax is exactly max |C| over the outputs as stored (NaN when an
  output is NaN), on the 256-row and 128-row tile paths, with row and column
  tails, BF16 and FP32 outputs, both accumulation modes, and a strided C;
- fp8_quantize_per_tensor_amax equals the oracle's quantization with that
  amax (and the two-pass quantizer when it is the true amax);
- the chain GEMM -> quantize C with the epilogue's amax gives exactly the
  codes and scale of the two-pass quantization of C."""

import numpy as np
import pytest
import torch

from block_quant_gemm_amd import mxq, workloads
from oracle import codec, per_tensor
from tests.gpu_helpers import host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _host_amax(c, out):
    """max |C| of the stored outputs as float32 (NaN if any is NaN)."""
    v = codec.bf16_bits_to_f64(host(c)) if out == mxq.OUT_BF16 else host(c).astype(np.float64)
    a = np.abs(v)
    return np.float32(np.nan) if np.isnan(a).any() else np.float32(a.max(initial=0.0))


def _same(x, y):
    return (np.isnan(x) and np.isnan(y)) or x == y


def _operands(M, N, K, seed):
    a = workloads.bf16_normal((M, K), 1.0, seed=seed, name="pta", outlier_frac=0.01,
                              outlier_scale=40.0)
    b = workloads.bf16_normal((N, K), 0.02, seed=seed + 1, name="ptb")
    qa, sa = mxq.fp8_quantize_per_tensor(to_dev_bf16(a))
    qb, sb = mxq.fp8_quantize_per_tensor(to_dev_bf16(b))
    return qa, sa, qb, sb


@pytest.mark.parametrize("M,N,K", [(300, 260, 96), (4100, 2100, 64), (1024, 2048, 512),
                                   (33, 8, 32)])
@pytest.mark.parametrize("out", [mxq.OUT_BF16, mxq.OUT_FP32])
@pytest.mark.parametrize("accum", [mxq.ACC_FP32, mxq.ACC_MFMA_FP8])
def test_gemm_amax_is_max_of_output(M, N, K, out, accum):
    say(f"per-tensor gemm amax M={M} N={N} K={K} out={out} accum={accum}")
    qa, sa, qb, sb = _operands(M, N, K, seed=M + N)
    c0 = mxq.fp8_gemm_per_tensor(qa, sa, qb, sb, out_dtype=out, accum=accum)
    c, amax = mxq.fp8_gemm_per_tensor_amax(qa, sa, qb, sb, out_dtype=out, accum=accum)
    assert torch.equal(c.view(torch.uint8), c0.view(torch.uint8))
    got, want = host(amax)[0], _host_amax(c, out)
    assert _same(got, want), (got, want)
    assert want > 0


def test_gemm_amax_strided_output_and_reuse():
    """C in the first N columns of a wider buffer whose other columns hold
    larger values: only the outputs count.  A second call on the same amax
    buffer with smaller outputs clears it first."""
    say("per-tensor gemm amax, strided C, reused amax buffer")
    M, N, K = 520, 200, 128
    qa, sa, qb, sb = _operands(M, N, K, seed=7)
    buf = torch.full((M, N + 56), 1000.0, dtype=torch.bfloat16, device="cuda")
    c, amax = mxq.fp8_gemm_per_tensor_amax(qa, sa, qb, sb, c=buf[:, :N])
    assert _same(host(amax)[0], _host_amax(c, mxq.OUT_BF16))
    assert float(host(amax)[0]) < 1000.0
    qa2, sa2, qb2, sb2 = _operands(64, N, K, seed=9)
    small = torch.tensor([1e-6], dtype=torch.float32, device="cuda")
    c2, amax2 = mxq.fp8_gemm_per_tensor_amax(qa2, small, qb2, sb2, c_amax=amax)
    assert amax2.data_ptr() == amax.data_ptr()
    assert _same(host(amax2)[0], _host_amax(c2, mxq.OUT_BF16))


def test_gemm_amax_special_cases():
    """A NaN code in A makes its output row NaN and the amax NaN; K == 0
    writes zeros and amax 0; M == 0 only clears the amax."""
    say("per-tensor gemm amax: NaN row, K = 0, M = 0")
    M, N, K = 96, 64, 64
    qa, sa, qb, sb = _operands(M, N, K, seed=11)
    qa[5, 7] = 0x7F                                        # E4M3 NaN
    c, amax = mxq.fp8_gemm_per_tensor_amax(qa, sa, qb, sb)
    assert np.isnan(host(amax)[0]) and np.isnan(_host_amax(c, mxq.OUT_BF16))
    z = torch.empty((M, 0), dtype=torch.uint8, device="cuda")
    zb = torch.empty((N, 0), dtype=torch.uint8, device="cuda")
    c, amax = mxq.fp8_gemm_per_tensor_amax(z, sa, zb, sb)
    assert int(host(c.view(torch.int16)).max()) == 0 and host(amax)[0] == 0.0
    e = torch.empty((0, K), dtype=torch.uint8, device="cuda")
    amax.fill_(5.0)
    c, amax = mxq.fp8_gemm_per_tensor_amax(e, sa, qb, sb, c_amax=amax)
    assert c.shape == (0, N) and host(amax)[0] == 0.0


@pytest.mark.parametrize("n", [4099, 65536, 8])
def test_quantize_with_given_amax(n):
    say(f"per-tensor quant with given amax n={n}")
    x = workloads.bf16_normal((n,), 1.0, seed=n, name="ptq", outlier_frac=0.01,
                              outlier_scale=60.0)
    v = codec.bf16_bits_to_f64(x)
    xd = to_dev_bf16(x)
    true = np.float32(np.abs(v).max())
    q0, s0 = mxq.fp8_quantize_per_tensor(xd)
    for amax in (true, np.float32(true * 3.7), np.float32(448.0 * 2.0 ** -5), np.float32(0.0),
                 np.float32(np.nan), np.float32(np.inf)):
        q, s = mxq.fp8_quantize_per_tensor_amax(xd, to_dev(np.array([amax], np.float32)))
        rc, rs = per_tensor.pt_quantize_given_amax(x, amax)
        assert host(s)[0] == rs and np.array_equal(host(q), rc), f"amax {amax}"
        if amax == true:
            assert torch.equal(q, q0) and torch.equal(s, s0)


def test_quantize_given_amax_empty():
    s = torch.zeros(1, dtype=torch.float32, device="cuda")
    x = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    q, s = mxq.fp8_quantize_per_tensor_amax(x, to_dev(np.array([896.0], np.float32)), scale=s)
    assert q.numel() == 0 and host(s)[0] == 2.0


def test_chain_epilogue_amax_equals_two_pass():
    """The dense per-tensor chain: C = GEMM (BF16, amax from the epilogue),
    then C quantized with that amax, equals the two-pass quantization of C
    and the oracle's."""
    say("per-tensor chain 2048x2816x2048 with the epilogue's amax")
    M, N, K = 2048, 2816, 2048
    qa, sa, qb, sb = _operands(M, N, K, seed=21)
    c, amax = mxq.fp8_gemm_per_tensor_amax(qa, sa, qb, sb)
    q1, s1 = mxq.fp8_quantize_per_tensor_amax(c, amax)
    q0, s0 = mxq.fp8_quantize_per_tensor(c)
    assert torch.equal(q1, q0) and torch.equal(s1, s0)
    rows = np.random.default_rng(3).choice(M, 24, replace=False)
    ch = host(c)
    rc, rs = per_tensor.pt_quantize_given_amax(ch[rows], host(amax)[0])
    assert host(s1)[0] == rs and np.array_equal(host(q1)[rows], rc)
    assert host(s1)[0] == per_tensor.pt_scale(ch)
