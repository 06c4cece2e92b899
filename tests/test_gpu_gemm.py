"""Parity of the HIP MX / per-tensor GEMMs (dense, grouped variable-M,
grouped variable-K) with the FP64 oracle, through the C ABI.

Every case runs in both accumulation modes:
- MXQ_ACC_FP32 (exact products, FP32 sums): every element must satisfy the
  contract's rule |C - Y| <= 1e-5 * S + 1e-6 (oracle.gemm), S = Σ|a_k b_k|;
  BF16 outputs must be the BF16 rounding of a value within that distance.
- MXQ_ACC_MFMA_FP8 (the FP8 matrix unit): the rule plus the unit's truncation
  allowance (tests/fp8_mode.py); the fraction inside the bare rule is printed.
Before outputs are compared, the operand codes and scales the library
produced are checked bit for bit against the oracle's quantization."""

import numpy as np
import pytest
import torch

from block_quant_gemm_amd import mxq, workloads
from oracle import gemm, mx, per_tensor
from tests.fp8_mode import accept, fp8_mfma_truncation_bound
from tests.gpu_helpers import host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

OUTS = [mxq.OUT_BF16, mxq.OUT_FP32]
ACCS = [mxq.ACC_FP32, mxq.ACC_MFMA_FP8]


def _quant_rows(bits):
    """Row quantization on the GPU, checked against the oracle's codes."""
    q, s = mxq.mx_quantize_rowwise(to_dev_bf16(bits))
    qh, sh = host(q), host(s)
    rq, rs = mx.mx_quantize_rowwise(bits)
    assert np.array_equal(qh, rq) and np.array_equal(sh, rs), "operand codes differ from the oracle"
    return q, s, qh, sh


def _check(c, Y, S, out, accum, extra=None, label=""):
    return accept(host(c), Y, S, out == mxq.OUT_FP32, accum == mxq.ACC_FP32, extra, label)


# Poisoned, guarded outputs: the result is a view of a larger buffer filled with
# a NaN sentinel, so an output element the kernel does not write fails the
# comparison, and the bands past its last row and column must stay intact.
_SENTINEL = {mxq.OUT_BF16: (torch.bfloat16, 0x7FA5), mxq.OUT_FP32: (torch.float32, 0x7FC0A5A5)}


def _guarded(rows, cols, out, lead=None, pad_rows=3, pad_cols=24):
    """(view [rows, cols] or [lead, rows//lead, cols], buffer): the view's row
    stride is cols + pad_cols and pad_rows sentinel rows follow it."""
    dt, bits = _SENTINEL[out]
    ld = cols + pad_cols
    buf = torch.empty((rows + pad_rows, ld), dtype=dt, device="cuda")
    ib = torch.int16 if dt == torch.bfloat16 else torch.int32
    buf.view(ib).fill_(bits if dt == torch.float32 else bits - 0x10000 * (bits >= 0x8000))
    v = buf[:rows, :cols]
    if lead is not None:
        v = buf[:rows].view(lead, rows // lead, ld)[:, :, :cols]
    return v, buf


def _guard_intact(buf, rows, cols, out):
    dt, bits = _SENTINEL[out]
    ib = torch.int16 if dt == torch.bfloat16 else torch.int32
    b = buf.view(ib)
    want = bits if dt == torch.float32 else bits - 0x10000 * (bits >= 0x8000)
    assert torch.all(b[:, cols:] == want), "write past the last column"
    assert torch.all(b[rows:] == want), "write past the last row"


@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("accum", ACCS)
def test_tiny_linear_forward(out, accum):
    """A, W 256x512 with 1% outliers x100: all 65536 outputs."""
    say(f"tiny linear 256x256x512 out={out} accum={accum}")
    d = workloads.tiny_linear(0)
    aq, asc, ah, ash = _quant_rows(d["A"])
    bq, bsc, bh, bsh = _quant_rows(d["W"])
    c, buf = _guarded(256, 256, out)
    mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=out, accum=accum, c=c)
    Y, S = gemm.gemm_ref(mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh))
    _check(c, Y, S, out, accum, lambda: fp8_mfma_truncation_bound(ah, ash, bh, bsh))
    _guard_intact(buf, 256, 256, out)


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


# Up to 128 tiles of 256 rows the dense GEMM runs on 128-row tiles; the last
# two shapes (81 and 289 tiles of 256 rows) take the 128-row and the 256-row
# path with a ragged last row and column of tiles.
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (200, 136, 96), (129, 257, 160), (64, 40, 1408),
                                   (3, 500, 2048), (300, 264, 1056), (300, 1024, 256),
                                   (257, 1300, 96), (2050, 2100, 64), (4100, 4130, 96)])
@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("layout", ["pad16", "odd", "shift5"])
@pytest.mark.parametrize("accum", ACCS)
def test_dense_ragged(M, N, K, out, layout, accum):
    say(f"dense ragged M={M} N={N} K={K} out={out} scales={layout} accum={accum}")
    a = workloads.bf16_normal((M, K), 1.0, seed=M + K, name="ga", outlier_frac=0.01,
                              outlier_scale=100.0)
    b = workloads.bf16_normal((N, K), 0.02, seed=N + K, name="gb")
    aq, asc, ah, ash = _quant_rows(a)
    bq, bsc, bh, bsh = _quant_rows(b)
    asc, bsc = _relayout_scales(asc, layout), _relayout_scales(bsc, layout)
    c, buf = _guarded(M, N, out)
    mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=out, accum=accum, c=c)
    Y, S = gemm.gemm_ref(mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh))
    _check(c, Y, S, out, accum, lambda: fp8_mfma_truncation_bound(ah, ash, bh, bsh))
    _guard_intact(buf, M, N, out)


@pytest.mark.parametrize("accum", ACCS)
def test_dense_strided_output_and_k_zero(accum):
    M, N, K = 70, 48, 64
    a = workloads.bf16_normal((M, K), 1.0, seed=1, name="sa")
    b = workloads.bf16_normal((N, K), 1.0, seed=1, name="sb")
    aq, asc, ah, ash = _quant_rows(a)
    bq, bsc, bh, bsh = _quant_rows(b)
    cbuf = torch.full((M, N + 8), 7.0, dtype=torch.float32, device="cuda")
    mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=mxq.OUT_FP32, accum=accum, c=cbuf[:, :N])
    Y, S = gemm.gemm_ref(mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh))
    _check(cbuf[:, :N], Y, S, mxq.OUT_FP32, accum,
           lambda: fp8_mfma_truncation_bound(ah, ash, bh, bsh))
    assert torch.all(cbuf[:, N:] == 7.0)
    # K == 0: C = 0
    z = mxq.mx_gemm(aq[:, :0], asc[:, :0], bq[:, :0], bsc[:, :0], out_dtype=mxq.OUT_FP32,
                    accum=accum)
    assert torch.all(z == 0)


def test_exact_mode_special_blocks():
    """Exact mode on blocks the FP8 unit truncates or the widening must keep:
    one large product beside small ones in every 8-run, NaN and Inf blocks
    (NaN rows/columns out), all-zero blocks (scale code 0), tiny blocks whose
    scale codes sit at the low end of the exact range (2^-116 and up)."""
    rng = np.random.default_rng(3)
    M, N, K = 64, 48, 256
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32)
    a[:, ::8] *= 3000.0                                 # a large product leads each run
    a[5, 32:64] = 0.0                                   # all-zero block
    a[7, 64:96] *= 2.0 ** -100                          # a tiny block (scale code about 20)
    b[3, 96:128] *= 2.0 ** -110
    a[9, 0] = np.inf                                    # Inf block -> row 9 is NaN
    b[11, 200] = np.nan                                 # NaN block -> column 11 is NaN
    to_bits = lambda x: torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    aq, asc, ah, ash = _quant_rows(to_bits(a))
    bq, bsc, bh, bsh = _quant_rows(to_bits(b))
    assert ash.min() >= 3 or (ash[ash < 3] == 0).all()
    for out in OUTS:
        c = mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=out, accum=mxq.ACC_FP32)
        Y, S = gemm.gemm_ref(mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh))
        assert np.isnan(Y[9]).all() and np.isnan(Y[:, 11]).all()
        _check(c, Y, S, out, mxq.ACC_FP32, label="special blocks")
        ch = host(c).astype(np.float64) if out == mxq.OUT_FP32 else None
        if ch is not None:
            assert np.isnan(ch[9]).all() and np.isnan(ch[:, 11]).all()
    # the FP8 unit loses the small products of these runs: the rule alone fails
    c8 = mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=mxq.OUT_FP32, accum=mxq.ACC_MFMA_FP8)
    fin = np.isfinite(Y)
    bare8 = gemm.check_fp32(host(c8).astype(np.float64), Y, S)
    say(f"  fp8 mode inside the bare rule on these runs: {bare8[fin].mean():.4f}")
    assert not bare8[fin].all()


@pytest.mark.parametrize("accum", ACCS)
def test_dense_ffn_forward_sampled(accum):
    """X 8192x2048 (0.5% outliers x50) · W 10944x2048ᵀ, 4000 sampled entries;
    the sampled rows' codes checked against the oracle."""
    say(f"dense FFN 8192x10944x2048 sampled accum={accum}")
    d = workloads.dense_ffn(0)
    aq, asc = mxq.mx_quantize_rowwise(to_dev_bf16(d["X"]))
    bq, bsc = mxq.mx_quantize_rowwise(to_dev_bf16(d["W"]))
    c = mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=mxq.OUT_BF16, accum=accum)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, 8192, 4000)
    cols = rng.integers(0, 10944, 4000)
    ah, ash = host(aq[to_dev(rows)]), host(asc[to_dev(rows)])
    bh, bsh = host(bq[to_dev(cols)]), host(bsc[to_dev(cols)])
    ra, rsa = mx.mx_quantize_rowwise(d["X"][rows])
    rb, rsb = mx.mx_quantize_rowwise(d["W"][cols])
    assert np.array_equal(ah, ra) and np.array_equal(ash, rsa)
    assert np.array_equal(bh, rb) and np.array_equal(bsh, rsb)
    idx = np.arange(len(rows))
    Y, S = gemm.gemm_ref_entries(mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh), idx, idx)
    _check(c[to_dev(rows), to_dev(cols)], Y, S, mxq.OUT_BF16, accum,
           lambda: fp8_mfma_truncation_bound(ah, ash, bh, bsh, idx, idx))


def _pt_quant(bits):
    q, s = mxq.fp8_quantize_per_tensor(to_dev_bf16(bits))
    rq, rs = per_tensor.pt_quantize(bits)
    assert np.array_equal(host(q), rq) and host(s)[0] == np.float32(rs), "per-tensor codes"
    return q, s


def _pt_extra(qa, sa, qb, sb, rows=None, cols=None):
    """FP8-mode allowance of a per-tensor product: the unit-scale truncation
    bound times the two FP32 scales."""
    ka, kb = qa.shape[1], qb.shape[1]
    ones_a = np.full((qa.shape[0], ka // 32), 127, np.uint8)
    ones_b = np.full((qb.shape[0], kb // 32), 127, np.uint8)
    return fp8_mfma_truncation_bound(qa, ones_a, qb, ones_b, rows, cols) * float(sa) * float(sb)


@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("accum", ACCS)
def test_per_tensor_gemm(out, accum):
    say(f"per-tensor gemm out={out} accum={accum}")
    a = workloads.bf16_normal((160, 512), 1.0, seed=5, name="pa", outlier_frac=0.005,
                              outlier_scale=50.0)
    b = workloads.bf16_normal((96, 512), 0.02, seed=5, name="pb")
    qa, sa = _pt_quant(a)
    qb, sb = _pt_quant(b)
    c, buf = _guarded(160, 96, out)
    mxq.fp8_gemm_per_tensor(qa, sa, qb, sb, out_dtype=out, accum=accum, c=c)
    A = per_tensor.pt_dequantize(host(qa), host(sa)[0])
    B = per_tensor.pt_dequantize(host(qb), host(sb)[0])
    Y, S = gemm.gemm_ref(A, B)
    _check(c, Y, S, out, accum,
           lambda: _pt_extra(host(qa), host(sa)[0], host(qb), host(sb)[0]))
    _guard_intact(buf, 160, 96, out)


@pytest.mark.parametrize("accum", ACCS)
def test_per_tensor_gemm_dense_ffn_sampled(accum):
    """The dense FFN shape (8192x10944x2048, 43x43 tiles) in the per-tensor
    format: 3000 sampled outputs against the oracle."""
    say(f"per-tensor dense FFN 8192x10944x2048 sampled accum={accum}")
    d = workloads.dense_ffn(0)
    qa, sa = _pt_quant(d["X"])
    qb, sb = _pt_quant(d["W"])
    c = mxq.fp8_gemm_per_tensor(qa, sa, qb, sb, out_dtype=mxq.OUT_BF16, accum=accum)
    rng = np.random.default_rng(7)
    rows = rng.integers(0, 8192, 3000)
    cols = rng.integers(0, 10944, 3000)
    sah, sbh = host(sa)[0], host(sb)[0]
    ah, bh = host(qa[to_dev(rows)]), host(qb[to_dev(cols)])
    idx = np.arange(len(rows))
    Y, S = gemm.gemm_ref_entries(per_tensor.pt_dequantize(ah, sah),
                                 per_tensor.pt_dequantize(bh, sbh), idx, idx)
    _check(c[to_dev(rows), to_dev(cols)], Y, S, mxq.OUT_BF16, accum,
           lambda: _pt_extra(ah, sah, bh, sbh, idx, idx))


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


def _grouped_extra(ah, ash, bh, bsh, offs, N):
    M = ah.shape[0]
    rows = np.repeat(np.arange(M), N)
    expert = np.searchsorted(offs, np.arange(M), side="right") - 1
    cols = np.repeat(expert, N) * N + np.tile(np.arange(N), M)
    return fp8_mfma_truncation_bound(ah, ash, bh, bsh, rows, cols).reshape(M, N)


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
@pytest.mark.parametrize("accum", ACCS)
def test_grouped_var_m(counts, N, K, out, layout, accum):
    say(f"grouped var-M counts={counts} N={N} K={K} out={out} scales={layout} accum={accum}")
    offs, a, w = _grouped_case(counts, N, K, seed=len(counts) + K)
    E = len(counts)
    aq, asc, ah, ash = _quant_rows(a)
    bq, bsc, bh, bsh = _quant_rows(w)                       # [E*N, K]
    asc, bsc = _relayout_scales(asc, layout), _relayout_scales(bsc, layout)
    M = a.shape[0]
    c, buf = _guarded(M, N, out)
    mxq.mx_grouped_gemm(aq, asc, bq.view(E, N, K), bsc.view(E, N, K // 32),
                        to_dev(offs), out_dtype=out, accum=accum, c=c)
    A, B = mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh)
    Y, S = gemm.grouped_gemm_ref(A, B.reshape(E, N, K), offs)
    _check(c, Y, S, out, accum, lambda: _grouped_extra(ah, ash, bh, bsh, offs, N))
    _guard_intact(buf, M, N, out)


@pytest.mark.parametrize("counts,R,K,M_cap_extra", [
    ([40, 0, 1, 130, 300], 256, 96, 0),       # 5 experts, R/32 = 8: odd experts 8 B into a window
    ([7, 300, 0, 33, 64, 1, 90], 256, 160, 64),  # 7 experts, spare capacity
    ([120, 5, 77], 2816, 64, 0),              # the gate/up weight's 88-byte scale stride
    ([64, 0, 200], 1408, 96, 32),             # the down weight's transposed copy (44 B)
])
@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("accum", ACCS)
def test_grouped_dgrad_on_weight_column_copies(counts, R, K, M_cap_extra, out, accum):
    """dgrad dX[rows of e] = dY[rows of e] · W_e, with W [E, R, K] column-
    quantized per expert (one group of R rows each) and read in place through
    expert_view: expert e's copy starts at column e*R of the transposed codes
    and at byte e*R/32 of each scale row, so with R/32 = 8 mod 16 every odd
    expert's first block sits 8 bytes into a 16-byte scale window."""
    say(f"dgrad on column copies counts={counts} R={R} K={K} out={out} accum={accum}")
    counts = np.array(counts, np.int64)
    offs = workloads.offsets_from_counts(counts)
    E, M = len(counts), int(counts.sum())
    dy = workloads.bf16_normal((M, R), 1e-3, seed=R + K, name="dg.dy", outlier_frac=0.01,
                               outlier_scale=30.0)
    w = workloads.bf16_normal((E * R, K), 0.02, seed=R + K, name="dg.w")
    woff = np.arange(E + 1, dtype=np.int64) * R
    qT, sT, poffw = mxq.mx_quantize_colwise(to_dev_bf16(w), to_dev(woff),
                                            M_cap=mxq.colwise_capacity(E * R, E) + M_cap_extra)
    rqT, rsT, rpoff = mx.mx_quantize_grouped_colwise(w, woff)
    assert np.array_equal(host(poffw), rpoff)
    assert np.array_equal(host(qT)[:, :E * R], rqT) and np.array_equal(host(sT)[:, :E * R // 32], rsT)
    bq, bs = mxq.expert_view(qT, sT, E, R)                   # [E, K, R]
    gq, gs, gh, gsh = _quant_rows(dy)
    c, buf = _guarded(M, K, out)
    mxq.mx_grouped_gemm(gq, gs, bq, bs, to_dev(offs), out_dtype=out, accum=accum, c=c)
    # oracle: expert e's B operand is rows of W_eᵀ, i.e. its column copy
    Bv = mx.mx_dequantize(rqT, rsT).reshape(K, E, R).transpose(1, 0, 2)   # [E, K, R]
    Y, S = gemm.grouped_gemm_ref(mx.mx_dequantize(gh, gsh), Bv, offs)
    bh = rqT.reshape(K, E, R).transpose(1, 0, 2).reshape(E * K, R)
    bsh = rsT.reshape(K, E, R // 32).transpose(1, 0, 2).reshape(E * K, R // 32)
    _check(c, Y, S, out, accum, lambda: _grouped_extra(gh, gsh, bh, bsh, offs, K))
    _guard_intact(buf, M, K, out)


@pytest.mark.parametrize("accum", ACCS)
def test_grouped_var_m_equals_dense_for_one_group(accum):
    a = workloads.bf16_normal((300, 256), 1.0, seed=9, name="oa")
    w = workloads.bf16_normal((72, 256), 0.02, seed=9, name="ow")
    aq, asc, _, _ = _quant_rows(a)
    bq, bsc, _, _ = _quant_rows(w)
    cg = mxq.mx_grouped_gemm(aq, asc, bq.view(1, 72, 256), bsc.view(1, 72, 8),
                             to_dev(np.array([0, 300], np.int64)), out_dtype=mxq.OUT_FP32,
                             accum=accum)
    cd = mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=mxq.OUT_FP32, accum=accum)
    assert torch.equal(cg, cd)


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
    # more experts than one wavefront ranks at once: unordered sizes with empty
    # experts (ranked largest first), and sizes already in order (kept)
    (np.random.default_rng(7).integers(0, 40, 130).tolist(), 64, 64),
    (sorted(np.random.default_rng(8).integers(0, 90, 100).tolist(), reverse=True), 72, 96),
])
@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("layout", ["pad16", "odd", "shift5"])
@pytest.mark.parametrize("accum", ACCS)
def test_grouped_wgrad(counts, N, K, out, layout, accum):
    say(f"grouped wgrad counts={counts} N={N} K={K} out={out} scales={layout} accum={accum}")
    counts = np.array(counts, np.int64)
    offs = workloads.offsets_from_counts(counts)
    E, T = len(counts), int(counts.sum())
    dy = workloads.bf16_normal((T, N), 1e-3, seed=T, name="wdy")
    x = workloads.bf16_normal((T, K), 1.0, seed=T, name="wx", outlier_frac=0.01,
                              outlier_scale=50.0)
    dyT, dysT, poff = mxq.mx_quantize_colwise(to_dev_bf16(dy), to_dev(offs))
    xT, xsT, _ = mxq.mx_quantize_colwise(to_dev_bf16(x), to_dev(offs))
    ah, ash, bh, bsh, ph = host(dyT), host(dysT), host(xT), host(xsT), host(poff)
    Mp = int(ph[-1])
    ra, rsa, rp = mx.mx_quantize_grouped_colwise(dy, offs)
    rb, rsb, _ = mx.mx_quantize_grouped_colwise(x, offs)
    assert np.array_equal(ph, rp)
    assert np.array_equal(ah[:, :Mp], ra) and np.array_equal(ash[:, :Mp // 32], rsa)
    assert np.array_equal(bh[:, :Mp], rb) and np.array_equal(bsh[:, :Mp // 32], rsb)
    dysT, xsT = _relayout_scales(dysT, layout), _relayout_scales(xsT, layout)
    c, buf = _guarded(E * N, K, out, lead=E)
    mxq.mx_grouped_gemm_wgrad(dyT, dysT, xT, xsT, poff, out_dtype=out, accum=accum, c=c)
    A, B = mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh)
    Y, S = gemm.grouped_wgrad_ref(A, B, ph)

    def extra():
        Tb = np.zeros_like(Y)
        for e in range(E):
            lo, hi = int(ph[e]), int(ph[e + 1])
            if hi > lo:
                Tb[e] = fp8_mfma_truncation_bound(ah[:, lo:hi], ash[:, lo // 32:hi // 32],
                                                  bh[:, lo:hi], bsh[:, lo // 32:hi // 32])
        return Tb
    _check(c, Y, S, out, accum, extra)
    _guard_intact(buf, E * N, K, out)
    for e in np.nonzero(counts == 0)[0]:
        assert torch.all(c[e] == 0)


@pytest.mark.parametrize("accum", ACCS)
def test_determinism(accum):
    d = workloads.tiny_linear(1)
    aq, asc, _, _ = _quant_rows(d["A"])
    bq, bsc, _, _ = _quant_rows(d["W"])
    c1 = mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=mxq.OUT_FP32, accum=accum)
    c2 = mxq.mx_gemm(aq, asc, bq, bsc, out_dtype=mxq.OUT_FP32, accum=accum)
    assert torch.equal(c1, c2)
