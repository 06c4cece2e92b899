"""Full block step at sequence 4096 x batch 4 (16384 tokens): the MLA
projection and shared-expert Linears, forward, dgrad and wgrad, and the
64-expert routed products at 98304 rows, every operand MX-quantized in both
directions by the dual-axis quantizer.  Sizes are the real ones; the oracle
checks sampled codes and sampled GEMM outputs (each output is one dot
product of dequantized rows), with the tolerance of oracle.gemm."""

import numpy as np
import pytest
import torch

from block_quant_gemm_amd import mxq, workloads
from oracle import gemm, mx
from tests import fp8_mode as f8
from tests.gpu_helpers import host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

T = workloads.BLOCK_TOKENS
NS = 600                                    # sampled outputs per product


def _rows_equal(x, q, s, rows):
    rc, rs = mx.mx_quantize_rowwise(np.ascontiguousarray(x[rows]))
    ri = torch.from_numpy(rows).cuda()
    assert np.array_equal(host(q[ri]), rc) and np.array_equal(host(s[ri]), rs)


def _cols_equal(x, qT, sT, cols, offs):
    cc, cs, rpoff = mx.mx_quantize_grouped_colwise(np.ascontiguousarray(x[:, cols]), offs)
    ci = torch.from_numpy(cols).cuda()
    Mp = int(rpoff[-1])
    assert np.array_equal(host(qT[ci])[:, :Mp], cc)
    assert np.array_equal(host(sT[ci])[:, :Mp // 32], cs)


def _check_sampled(c, aq, asc, bq, bsc, rows, cols, crows=None, ccols=None):
    """C[crows, ccols] against the oracle dot products of operand rows
    (rows of A, rows of B) from the GPU's own codes and scales."""
    crows = rows if crows is None else crows
    ccols = cols if ccols is None else ccols
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    ah, ash = host(aq[ri]), host(asc[ri])
    bh, bsh = host(bq[ci]), host(bsc[ci])
    idx = np.arange(len(rows))
    Y, S = gemm.gemm_ref_entries(mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh), idx, idx)
    Tb = f8.fp8_mfma_truncation_bound(ah, ash, bh, bsh, idx, idx)
    ch = host(c)[crows, ccols]
    ok = f8.check_bf16_extra(ch, Y, S, Tb)
    if not ok.all():
        bad = np.nonzero(~ok)[0][:8]
        raise AssertionError(f"outputs {list(zip(crows[bad], ccols[bad]))}: "
                             f"{ch[bad]} vs {Y[bad]}")


@pytest.mark.parametrize("name,fin,fout", workloads.BLOCK_DENSE_LINEARS)
def test_block_dense_linear_fwd_dgrad_wgrad(name, fin, fout):
    say(f"block linear {name}: {T} tokens, {fin} -> {fout}")
    d = workloads.block_linear(name, fin, fout)
    rng = np.random.default_rng(fin * 7 + fout)
    one = to_dev(np.array([0, T], np.int64))
    w_one = to_dev(np.array([0, fout], np.int64))
    xq, xs, xT, xTs, _ = mxq.mx_quantize_dual(to_dev_bf16(d["X"]), one)
    wq, ws, wT, wTs, _ = mxq.mx_quantize_dual(to_dev_bf16(d["W"]), w_one)
    gq, gs, gT, gTs, _ = mxq.mx_quantize_dual(to_dev_bf16(d["dY"]), one)
    # sampled codes of each copy against the oracle
    _rows_equal(d["X"], xq, xs, np.sort(rng.choice(T, 16, replace=False)))
    _cols_equal(d["X"], xT, xTs, rng.choice(fin, 4, replace=False), np.array([0, T]))
    _rows_equal(d["W"], wq, ws, np.sort(rng.choice(fout, 16, replace=False)))
    _cols_equal(d["W"], wT, wTs, rng.choice(fin, 4, replace=False), np.array([0, fout]))
    _cols_equal(d["dY"], gT, gTs, rng.choice(fout, 4, replace=False), np.array([0, T]))
    # forward Y = X Wᵀ [T, out]
    y = mxq.mx_gemm(xq, xs, wq, ws)
    r, n = rng.integers(0, T, NS), rng.integers(0, fout, NS)
    _check_sampled(y, xq, xs, wq, ws, r, n)
    # dgrad dX = dY W [T, in]: B = the column copy of W (blocks along out)
    wTv, wTsv = wT[:, :fout], wTs[:, :fout // 32]
    dx = mxq.mx_gemm(gq, gs, wTv, wTsv)
    r, k = rng.integers(0, T, NS), rng.integers(0, fin, NS)
    _check_sampled(dx, gq, gs, wTv, wTsv, r, k)
    # wgrad dW = dYᵀ X [out, in]: both column copies (blocks along tokens)
    gTv, gTsv, xTv, xTsv = gT[:, :T], gTs[:, :T // 32], xT[:, :T], xTs[:, :T // 32]
    dw = mxq.mx_gemm(gTv, gTsv, xTv, xTsv)
    n, k = rng.integers(0, fout, NS), rng.integers(0, fin, NS)
    _check_sampled(dw, gTv, gTsv, xTv, xTsv, n, k)


def test_block_routed_experts_98304_rows():
    """Routed experts at 16384 tokens x top-6: gate/up forward and its weight
    gradient over the Zipf expert groups (98304 rows)."""
    say("block routed experts: 98304 rows, 64 experts")
    fw = workloads.moe_forward(0, tokens=T)
    bw = workloads.moe_backward(0, tokens=T)
    offs, E, F2 = fw["offsets"], 64, 2 * workloads.MOE_FFN
    M = int(offs[-1])
    assert M == 6 * T
    od = to_dev(offs)
    rng = np.random.default_rng(5)
    xq, xs, xT, xTs, poff = mxq.mx_quantize_dual(to_dev_bf16(fw["X"]), od)
    w = fw["W_gu"].reshape(E * F2, workloads.HIDDEN)
    wq, ws = mxq.mx_quantize_rowwise(to_dev_bf16(w))
    _rows_equal(fw["X"], xq, xs, np.sort(rng.choice(M, 16, replace=False)))
    _cols_equal(fw["X"], xT, xTs, rng.choice(workloads.HIDDEN, 3, replace=False), offs)
    gu = mxq.mx_grouped_gemm(xq, xs, wq.view(E, F2, workloads.HIDDEN),
                             ws.view(E, F2, workloads.HIDDEN // 32), od)
    r, n = rng.integers(0, M, NS), rng.integers(0, F2, NS)
    e = np.searchsorted(offs, r, side="right") - 1
    _check_sampled(gu, xq, xs, wq, ws, r, e * F2 + n, r, n)
    uq, us, uT, uTs, _ = mxq.mx_quantize_dual(to_dev_bf16(bw["dGU"]), od)
    dw = mxq.mx_grouped_gemm_wgrad(uT, uTs, xT, xTs, poff)
    ph = host(poff)
    e = rng.integers(0, E, NS)
    n, k = rng.integers(0, F2, NS), rng.integers(0, workloads.HIDDEN, NS)
    # dW[e, n, k] = Σ over expert e's padded token range of uT[n, t] xT[k, t]
    Y = np.zeros(NS); S = np.zeros(NS); Tb = np.zeros(NS)
    uh, ush, xh, xsh = host(uT), host(uTs), host(xT), host(xTs)
    for i in range(NS):
        lo, hi = int(ph[e[i]]), int(ph[e[i] + 1])
        a = mx.mx_dequantize(uh[n[i]:n[i] + 1, lo:hi], ush[n[i]:n[i] + 1, lo // 32:hi // 32])
        b = mx.mx_dequantize(xh[k[i]:k[i] + 1, lo:hi], xsh[k[i]:k[i] + 1, lo // 32:hi // 32])
        y, s = gemm.gemm_ref(a, b)
        Y[i], S[i] = y[0, 0], s[0, 0]
        Tb[i] = f8.fp8_mfma_truncation_bound(uh[n[i]:n[i] + 1, lo:hi],
                                               ush[n[i]:n[i] + 1, lo // 32:hi // 32],
                                               xh[k[i]:k[i] + 1, lo:hi],
                                               xsh[k[i]:k[i] + 1, lo // 32:hi // 32])[0, 0]
    ch = host(dw)[e, n, k]
    assert f8.check_bf16_extra(ch, Y, S, Tb).all()
