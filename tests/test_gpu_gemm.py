"""Parity of the HIP MX / per-tensor GEMMs (dense, grouped variable-M,
grouped variable-K) with the FP64 oracle, through the C ABI.

Acceptance per element (oracle.gemm): |C - Y| <= 1e-5 * S + 1e-6, S = Σ|a_k b_k|,
plus, for the FP8 matrix-unit accumulation mode, the alignment-truncation
allowance of that instruction; BF16 outputs must be the BF16 rounding of a
value within that distance."""

import numpy as np
import pytest
import torch

from block_quant_gemm_amd import mxq, workloads
from oracle import gemm, mx, per_tensor
from tests.gpu_helpers import host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

OUTS = [mxq.OUT_BF16, mxq.OUT_FP32]


def _quant_rows(bits):
    q, s = mxq.mx_quantize_rowwise(to_dev_bf16(bits))
    return q, s, host(q), host(s)


def _sampled_ref(ah, ash, bh, bsh, rows, cols):
    """Oracle value, magnitude and MFMA allowance of entries (rows[i], cols[i])
    of A·Bᵀ, dequantizing only the rows involved."""
    a, sa, b, sb = ah[rows], ash[rows], bh[cols], bsh[cols]
    idx = np.arange(len(rows))
    Y, S = gemm.gemm_ref_entries(mx.mx_dequantize(a, sa), mx.mx_dequantize(b, sb), idx, idx)
    T = gemm.fp8_mfma_truncation_bound(a, sa, b, sb, idx, idx)
    return Y, S, T


def _check(c, Y, S, extra, out):
    extra = np.zeros_like(Y) if extra is None else extra
    if out == mxq.OUT_FP32:
        ok = gemm.check_fp32_extra(host(c).astype(np.float64), Y, S, extra)
        bare = gemm.check_fp32(host(c).astype(np.float64), Y, S)
    else:
        ok = gemm.check_bf16_extra(host(c), Y, S, extra)
        bare = gemm.check_bf16(host(c), Y, S)
    say(f"  elements {ok.size}: within 1e-5*S+1e-6: {bare.mean():.6f}; "
        f"within that + MFMA allowance: {ok.mean():.6f}")
    if not ok.all():
        bad = np.argwhere(~ok)[:12]
        say(f"  first failures (index, value, oracle): "
            f"{[(tuple(int(v) for v in i), float(host(c).astype(np.float64)[tuple(i)]) if out == mxq.OUT_FP32 else int(host(c)[tuple(i)]), float(Y[tuple(i)])) for i in bad]}")
    assert ok.all(), f"{(~ok).sum()} elements out of tolerance"
    return bare


@pytest.mark.parametrize("out", OUTS)
def test_tiny_linear_forward(out):
    say(f"tiny linear 256x256x512 out={out}")
    d = workloads.tiny_linear(0)
    aq, asc, ah, ash = _quant_rows(d["A"])
    bq, bsc, bh, bsh = _quant_rows(d["W"])
    c = mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=out)
    A, B = mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh)
    Y, S = gemm.gemm_ref(A, B)
    T = gemm.fp8_mfma_truncation_bound(ah, ash, bh, bsh)
    _check(c, Y, S, T, out)


def _relayout_scales(s, layout):
    """Copy of a [rows, nb] scale tensor with another row stride / base offset:
    'pad16' keeps the quantizer's (stride a multiple of 16: 16-byte windows),
    'odd' has an odd stride (byte-by-byte path), 'shift5' a stride multiple
    of 16 with the base 5 bytes past a 16-byte boundary (windows whose first
    block sits mid-window)."""
    if layout == "pad16":
        return s
    rows, nb = s.shape
    if layout == "odd":
        buf = torch.zeros((rows, nb + 1 + (nb % 2)), dtype=torch.uint8, device=s.device)
        v = buf[:, :nb]
    else:
        ld = (nb + 5 + 15) // 16 * 16
        buf = torch.zeros((rows, ld), dtype=torch.uint8, device=s.device)
        v = buf[:, 5:5 + nb]
    v.copy_(s)
    return v


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (200, 136, 96), (129, 257, 160), (64, 40, 1408),
                                   (3, 500, 2048), (300, 264, 1056), (300, 1024, 256),
                                   (257, 1300, 96)])
@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("layout", ["pad16", "odd", "shift5"])
def test_dense_ragged(M, N, K, out, layout):
    say(f"dense ragged M={M} N={N} K={K} out={out} scales={layout}")
    a = workloads.bf16_normal((M, K), 1.0, seed=M + K, name="ga")
    b = workloads.bf16_normal((N, K), 0.02, seed=N + K, name="gb")
    aq, asc, ah, ash = _quant_rows(a)
    bq, bsc, bh, bsh = _quant_rows(b)
    asc, bsc = _relayout_scales(asc, layout), _relayout_scales(bsc, layout)
    c = mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=out)
    Y, S = gemm.gemm_ref(mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh))
    _check(c, Y, S, gemm.fp8_mfma_truncation_bound(ah, ash, bh, bsh), out)


def test_dense_strided_output_and_k_zero():
    M, N, K = 70, 48, 64
    a = workloads.bf16_normal((M, K), 1.0, seed=1, name="sa")
    b = workloads.bf16_normal((N, K), 1.0, seed=1, name="sb")
    aq, asc, ah, ash = _quant_rows(a)
    bq, bsc, bh, bsh = _quant_rows(b)
    cbuf = torch.full((M, N + 8), 7.0, dtype=torch.float32, device="cuda")
    mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=mxq.OUT_FP32, c=cbuf[:, :N])
    Y, S = gemm.gemm_ref(mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh))
    _check(cbuf[:, :N], Y, S, gemm.fp8_mfma_truncation_bound(ah, ash, bh, bsh), mxq.OUT_FP32)
    assert torch.all(cbuf[:, N:] == 7.0)
    # K == 0: C = 0
    z = mxq.mx_gemm(aq[:, :0], asc[:, :0], bq[:, :0], bsc[:, :0], out_dtype=mxq.OUT_FP32)
    assert torch.all(z == 0)


def test_dense_ffn_forward_sampled():
    """X 8192x2048 (0.5% outliers x50) · W 10944x2048ᵀ, 4000 sampled entries."""
    say("dense FFN 8192x10944x2048 sampled")
    d = workloads.dense_ffn(0)
    aq, asc, ah, ash = _quant_rows(d["X"])
    bq, bsc, bh, bsh = _quant_rows(d["W"])
    c = mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=mxq.OUT_BF16)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, 8192, 4000)
    cols = rng.integers(0, 10944, 4000)
    Y, S, T = _sampled_ref(ah, ash, bh, bsh, rows, cols)
    ch = host(c)[rows, cols]
    ok = gemm.check_bf16_extra(ch, Y, S, T)
    say(f"  bare tolerance: {gemm.check_bf16(ch, Y, S).mean():.5f}")
    assert ok.all()


@pytest.mark.parametrize("out", OUTS)
def test_per_tensor_gemm(out):
    say(f"per-tensor gemm out={out}")
    a = workloads.bf16_normal((160, 512), 1.0, seed=5, name="pa", outlier_frac=0.005,
                              outlier_scale=50.0)
    b = workloads.bf16_normal((96, 512), 0.02, seed=5, name="pb")
    qa, sa = mxq.fp8_quantize_per_tensor(to_dev_bf16(a))
    qb, sb = mxq.fp8_quantize_per_tensor(to_dev_bf16(b))
    c = mxq.fp8_gemm_per_tensor(qa, sa, qb, sb, out_dtype=out)
    A = per_tensor.pt_dequantize(host(qa), host(sa)[0])
    B = per_tensor.pt_dequantize(host(qb), host(sb)[0])
    Y, S = gemm.gemm_ref(A, B)
    ones_a = np.full((160, 16), 127, np.uint8)
    ones_b = np.full((96, 16), 127, np.uint8)
    T = gemm.fp8_mfma_truncation_bound(host(qa), ones_a, host(qb), ones_b) * \
        float(host(sa)[0]) * float(host(sb)[0])
    # the two FP32 scales are multiplied into the FP32 sum: two more roundings
    T = T + 2.0 ** -23 * np.abs(Y)
    _check(c, Y, S, T, out)


# ---------------------------------------------------------------------------
# grouped, variable M
# ---------------------------------------------------------------------------

def _grouped_case(counts, N, K, seed):
    counts = np.array(counts, np.int64)
    offs = workloads.offsets_from_counts(counts)
    E, M = len(counts), int(counts.sum())
    a = workloads.bf16_normal((M, K), 1.0, seed=seed, name="xa")
    w = workloads.bf16_normal((E * N, K), 0.02, seed=seed, name="xw")
    return offs, a, w


@pytest.mark.parametrize("counts,N,K", [
    ([40, 0, 1, 130, 0, 300, 0], 160, 256),
    ([0, 0, 257], 96, 64),
    ([5], 32, 32),
    ([128, 128, 0, 1, 127, 129], 136, 1408),
    ([300, 0, 45, 513], 768, 192),
    ([300, 0, 45, 513], 700, 128),
])
@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("layout", ["pad16", "odd", "shift5"])
def test_grouped_var_m(counts, N, K, out, layout):
    say(f"grouped var-M counts={counts} N={N} K={K} out={out} scales={layout}")
    offs, a, w = _grouped_case(counts, N, K, seed=len(counts) + K)
    E = len(counts)
    aq, asc, ah, ash = _quant_rows(a)
    bq, bsc, bh, bsh = _quant_rows(w)                       # [E*N, K]
    asc, bsc = _relayout_scales(asc, layout), _relayout_scales(bsc, layout)
    c = mxq.mx_grouped_gemm(aq, asc, bq.view(E, N, K), bsc.view(E, N, K // 32),
                            to_dev(offs), out_dtype=out)
    A, B = mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh)
    Y, S = gemm.grouped_gemm_ref(A, B.reshape(E, N, K), offs)
    M = a.shape[0]
    rows = np.repeat(np.arange(M), N)
    expert = np.searchsorted(offs, np.arange(M), side="right") - 1
    cols = (np.repeat(expert, N) * N + np.tile(np.arange(N), M))
    T = gemm.fp8_mfma_truncation_bound(ah, ash, bh, bsh, rows, cols).reshape(M, N)
    _check(c, Y, S, T, out)


def test_grouped_var_m_equals_dense_for_one_group():
    a = workloads.bf16_normal((300, 256), 1.0, seed=9, name="oa")
    w = workloads.bf16_normal((72, 256), 0.02, seed=9, name="ow")
    aq, asc, _, _ = _quant_rows(a)
    bq, bsc, _, _ = _quant_rows(w)
    cg = mxq.mx_grouped_gemm(aq, asc, bq.view(1, 72, 256), bsc.view(1, 72, 8),
                             to_dev(np.array([0, 300], np.int64)), out_dtype=mxq.OUT_FP32)
    cd = mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=mxq.OUT_FP32)
    assert torch.equal(cg, cd)


def test_grouped_moe_gate_up_sampled():
    """MoE gate_up forward at full size: 49152 rows, 64 experts (Zipf), W_gu
    [64, 2816, 2048]; 3000 sampled outputs."""
    say("grouped gate_up 49152 x 2816 x 2048, 64 experts")
    d = workloads.moe_forward(0)
    offs, E = d["offsets"], 64
    aq, asc, ah, ash = _quant_rows(d["X"])
    wq, wsc, wh, wsh = _quant_rows(d["W_gu"].reshape(E * 2816, 2048))
    c = mxq.mx_grouped_gemm(aq, asc, wq.view(E, 2816, 2048), wsc.view(E, 2816, 64),
                            to_dev(offs), out_dtype=mxq.OUT_BF16)
    rng = np.random.default_rng(1)
    rows = rng.integers(0, 49152, 3000)
    n = rng.integers(0, 2816, 3000)
    e = np.searchsorted(offs, rows, side="right") - 1
    cols = e * 2816 + n
    Y, S, T = _sampled_ref(ah, ash, wh, wsh, rows, cols)
    ch = host(c)[rows, n]
    bare = gemm.check_bf16(ch, Y, S)
    say(f"  bare tolerance: {bare.mean():.5f}")
    assert gemm.check_bf16_extra(ch, Y, S, T).all()
    assert bare.all()


# ---------------------------------------------------------------------------
# grouped, variable K (weight gradient)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("counts,N,K", [
    ([40, 0, 1, 130, 0, 300, 0], 160, 96),
    ([0, 64], 32, 32),
    ([333, 12, 0, 77], 136, 200),
    ([700, 33, 1100, 0, 517], 288, 160),
    ([300, 0, 45, 513], 296, 768),
    ([300, 0, 45, 513], 264, 600),
])
@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("layout", ["pad16", "odd", "shift5"])
def test_grouped_wgrad(counts, N, K, out, layout):
    say(f"grouped wgrad counts={counts} N={N} K={K} out={out} scales={layout}")
    counts = np.array(counts, np.int64)
    offs = workloads.offsets_from_counts(counts)
    E, T = len(counts), int(counts.sum())
    dy = workloads.bf16_normal((T, N), 1e-3, seed=T, name="wdy")
    x = workloads.bf16_normal((T, K), 1.0, seed=T, name="wx")
    dyT, dysT, poff = mxq.mx_quantize_colwise(to_dev_bf16(dy), to_dev(offs))
    xT, xsT, _ = mxq.mx_quantize_colwise(to_dev_bf16(x), to_dev(offs))
    dysT, xsT = _relayout_scales(dysT, layout), _relayout_scales(xsT, layout)
    c = mxq.mx_grouped_gemm_wgrad(dyT, dysT, xT, xsT, poff, out_dtype=out)
    ah, ash, bh, bsh, ph = host(dyT), host(dysT), host(xT), host(xsT), host(poff)
    A, B = mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh)
    Y, S = gemm.grouped_wgrad_ref(A, B, ph)
    Tb = np.zeros_like(Y)
    for e in range(E):
        lo, hi = int(ph[e]), int(ph[e + 1])
        if hi > lo:
            Tb[e] = gemm.fp8_mfma_truncation_bound(ah[:, lo:hi], ash[:, lo // 32:hi // 32],
                                                   bh[:, lo:hi], bsh[:, lo // 32:hi // 32])
    _check(c, Y, S, Tb, out)
    for e in np.nonzero(counts == 0)[0]:
        assert torch.all(c[e] == 0)


def test_determinism():
    d = workloads.tiny_linear(1)
    aq, asc, _, _ = _quant_rows(d["A"])
    bq, bsc, _, _ = _quant_rows(d["W"])
    c1 = mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=mxq.OUT_FP32)
    c2 = mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=mxq.OUT_FP32)
    assert torch.equal(c1, c2)
