"""Per-expert current scaling with the amax taken in the producing matmul's
epilogue: the per-group-scaled gate/up product with SwiGLU (h in BF16 and
each group's max |h|), and the per-group quantizers that take the group
amaxes instead of finding them.  Through the C ABI, against the oracle.

The quantizers with given amaxes must equal the oracle's per-group
quantization bit for bit when the amaxes are the groups' true max |x|.  The
product's h is checked like the MX SwiGLU product's (tests/test_gpu_swiglu.py
intervals), its BF16 rounding included; h_amax must be the max |h| of what
the kernel wrote and lie within the oracle's interval."""

import numpy as np
import pytest

from block_quant_gemm_amd import mxq, workloads
from oracle import codec, gemm, per_tensor
from tests import fp8_mode as f8
from tests.gpu_helpers import host, say, to_dev, to_dev_bf16
from tests.test_gpu_per_group import _gemm_allowance
from tests.test_gpu_swiglu import h_bounds

pytestmark = pytest.mark.gpu


def _group_amax(bits, offs):
    """max |x| of each row group of a BF16 matrix (NaN if the group has one)."""
    x = codec.bf16_bits_to_f64(bits)
    out = np.zeros(len(offs) - 1, np.float32)
    for e in range(len(offs) - 1):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi > lo:
            out[e] = np.max(np.abs(x[lo:hi]))
    return out


@pytest.mark.parametrize("counts,K", [
    ([40, 0, 1, 130, 0, 300, 0], 64),
    ([1000, 17, 0, 2, 511], 2048),
    ([5], 8),
])
def test_quantize_with_given_amax_bit_exact(counts, K):
    say(f"per-group quant with given amax counts={counts} K={K}")
    offs = workloads.offsets_from_counts(np.array(counts, np.int64))
    M = int(offs[-1])
    x = workloads.bf16_normal((M, K), 1.0, seed=M + K, name="pgx", outlier_frac=0.01,
                              outlier_scale=30.0)
    amax = to_dev(_group_amax(x, offs))
    q, s = mxq.fp8_quantize_per_group_amax(to_dev_bf16(x), to_dev(offs), amax)
    rq, rs = per_tensor.pg_quantize(x, offs)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(q), rq)
    if K % 8 == 0:
        qT, sT, poff = mxq.fp8_quantize_per_group_colwise_amax(to_dev_bf16(x), to_dev(offs),
                                                               amax)
        cq, cs, cp = per_tensor.pg_quantize_colwise(x, offs)
        assert np.array_equal(host(sT).view(np.uint32), cs.view(np.uint32))
        assert np.array_equal(host(poff), cp)
        assert np.array_equal(host(qT)[:, :int(cp[-1])], cq)


def test_quantize_with_given_amax_special_groups():
    """Groups holding NaN, Inf, only zeros, and an empty group: the same codes
    and scales as the oracle (which finds the amaxes itself)."""
    K = 32
    offs = np.array([0, 3, 3, 7, 9, 12], np.int64)
    vals = np.random.default_rng(2).normal(0, 1, (12, K)).astype(np.float32)
    vals[1, 5] = np.nan
    vals[4, 0] = np.inf
    vals[7:9] = 0.0
    bits = codec.bf16_round_to_bits(vals.astype(np.float64))
    amax = to_dev(_group_amax(bits, offs))
    q, s = mxq.fp8_quantize_per_group_amax(to_dev_bf16(bits), to_dev(offs), amax)
    rq, rs = per_tensor.pg_quantize(bits, offs)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(q), rq)


def _pg_operands(counts, F, K, seed):
    offs = workloads.offsets_from_counts(np.array(counts, np.int64))
    E, M = len(counts), int(offs[-1])
    a = workloads.bf16_normal((M, K), 1.0, seed=seed, name="pga")
    w = workloads.bf16_normal((E * 2 * F, K), 0.02, seed=seed, name="pgw")
    woffs = np.arange(E + 1, dtype=np.int64) * 2 * F
    aq, sa = per_tensor.pg_quantize(a, offs)
    wq, swt = per_tensor.pg_quantize(w, woffs)
    return offs, woffs, aq, sa, wq, swt


@pytest.mark.parametrize("counts,F,K", [
    ([300, 0, 1, 257, 31, 600], 320, 256),
    ([0, 0, 513], 1408, 128),
    ([5], 32, 64),
])
def test_per_group_swiglu_product(counts, F, K):
    say(f"per-group SwiGLU product counts={counts} F={F} K={K}")
    offs, woffs, aq, sa, wq, swt = _pg_operands(counts, F, K, seed=F + K + len(counts))
    E, M = len(counts), aq.shape[0]
    offs_d = to_dev(offs)
    gu, h, h_amax = mxq.fp8_grouped_gemm_per_group_swiglu(
        to_dev(aq), to_dev(sa), to_dev(wq).view(E, 2 * F, K), to_dev(swt), offs_d)
    guh, hh, amh = host(gu), host(h), host(h_amax)
    A = per_tensor.pg_dequantize(aq, sa, offs)
    B = per_tensor.pg_dequantize(wq, swt, woffs).reshape(E, 2 * F, K)
    Y, S = gemm.grouped_gemm_ref(A, B, offs)
    T = _gemm_allowance(aq, wq, sa, swt, offs, 2 * F) + 2.0 ** -23 * np.abs(Y)
    assert f8.check_bf16_extra(guh, Y, S, T).all()
    dY = gemm.tolerance(S) + T
    lo, hi = h_bounds(Y[:, :F], Y[:, F:], dY[:, :F], dY[:, F:])
    hv = codec.bf16_bits_to_f64(hh)
    blo, bhi = codec.bf16_round(lo), codec.bf16_round(hi)
    ok = (hv >= blo) & (hv <= bhi)
    say(f"  h within its interval: {ok.mean():.6f}; fixed by it: {(blo == bhi).mean():.5f}")
    assert ok.all()
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if b == a:
            assert amh[e] == 0.0
            continue
        assert amh[e] == np.max(np.abs(hv[a:b]))            # the max of what was written
        mag_lo = np.where((blo[a:b] <= 0) & (bhi[a:b] >= 0), 0.0,
                          np.minimum(np.abs(blo[a:b]), np.abs(bhi[a:b])))
        mag_hi = np.maximum(np.abs(blo[a:b]), np.abs(bhi[a:b]))
        assert mag_lo.max() <= amh[e] <= mag_hi.max()
    # h's per-group copies from the epilogue's amax equal those of the
    # quantizers that find the amax themselves
    q1, s1 = mxq.fp8_quantize_per_group_amax(h, offs_d, h_amax)
    q2, s2 = mxq.fp8_quantize_per_group(h, offs_d)
    assert np.array_equal(host(s1).view(np.uint32), host(s2).view(np.uint32))
    assert np.array_equal(host(q1), host(q2))
    t1 = mxq.fp8_quantize_per_group_colwise_amax(h, offs_d, h_amax)
    t2 = mxq.fp8_quantize_per_group_colwise(h, offs_d)
    for x1, x2 in zip(t1, t2):
        assert np.array_equal(host(x1), host(x2))
    d1 = mxq.fp8_quantize_per_group_dual(h, offs_d, amax=h_amax)
    d2 = mxq.fp8_quantize_per_group_dual(h, offs_d)
    Mp = int(host(d2[3])[-1])
    assert np.array_equal(host(d1[0]), host(d2[0]))
    assert np.array_equal(host(d1[1])[:, :Mp], host(d2[1])[:, :Mp])
    assert np.array_equal(host(d1[2]).view(np.uint32), host(d2[2]).view(np.uint32))
    assert np.array_equal(host(d1[3]), host(d2[3]))


def test_per_group_swiglu_full_size_sampled():
    """The per-group-scaled gate/up product with SwiGLU at full size (49152
    rows, 64 Zipf experts, F 1408, K 2048; operands from the per-group
    quantizer, whose codes and scales are pinned bit-exact to the oracle in
    tests/test_gpu_per_group.py): 1500 sampled h values within their intervals,
    600 sampled gate/up outputs, and every group's amax equal to the max |h|
    the kernel wrote."""
    say("per-group SwiGLU product 49152 x (2 x 1408) x 2048, 64 experts")
    d = workloads.moe_forward(0)
    offs, E, F, K = d["offsets"], 64, workloads.MOE_FFN, workloads.HIDDEN
    woffs = np.arange(E + 1, dtype=np.int64) * 2 * F
    offs_d = to_dev(offs)
    aq, sa = mxq.fp8_quantize_per_group(to_dev_bf16(d["X"]), offs_d)
    wq, wsc = mxq.fp8_quantize_per_group(to_dev_bf16(d["W_gu"].reshape(E * 2 * F, K)),
                                         to_dev(woffs))
    gu, h, h_amax = mxq.fp8_grouped_gemm_per_group_swiglu(aq, sa, wq.view(E, 2 * F, K), wsc,
                                                          offs_d)
    ah, sah, wh, swh = host(aq), host(sa), host(wq), host(wsc)
    guh, hv, amh = host(gu), codec.bf16_bits_to_f64(host(h)), host(h_amax)
    rng = np.random.default_rng(13)
    M = ah.shape[0]

    def ref(rows, wrows):
        e = np.searchsorted(offs, rows, side="right") - 1
        idx = np.arange(len(rows))
        A = per_tensor.pt_dequantize(ah[rows], np.float32(1.0)) * sah[e].astype(np.float64)[:, None]
        B = per_tensor.pt_dequantize(wh[wrows], np.float32(1.0)) * swh[e].astype(np.float64)[:, None]
        Y, S = gemm.gemm_ref_entries(A, B, idx, idx)
        ones = np.full((len(rows), K // 32), 127, np.uint8)
        T = f8.fp8_mfma_truncation_bound(ah[rows], ones, wh[wrows], ones, idx, idx) * \
            sah[e].astype(np.float64) * swh[e].astype(np.float64) + 2.0 ** -23 * np.abs(Y)
        return Y, gemm.tolerance(S) + T, S, T

    r, n = rng.integers(0, M, 600), rng.integers(0, 2 * F, 600)
    e = np.searchsorted(offs, r, side="right") - 1
    Y, _, S, T = ref(r, e * 2 * F + n)
    assert f8.check_bf16_extra(guh[r, n], Y, S, T).all()
    r, c = rng.integers(0, M, 1500), rng.integers(0, F, 1500)
    e = np.searchsorted(offs, r, side="right") - 1
    g, dg, _, _ = ref(r, e * 2 * F + c)
    u, du, _, _ = ref(r, e * 2 * F + F + c)
    lo, hi = h_bounds(g, u, dg, du)
    ok = (hv[r, c] >= codec.bf16_round(lo)) & (hv[r, c] <= codec.bf16_round(hi))
    assert ok.all()
    for k in range(E):
        a, b = int(offs[k]), int(offs[k + 1])
        assert amh[k] == (np.max(np.abs(hv[a:b])) if b > a else 0.0)
