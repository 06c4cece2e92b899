"""Parity of the HIP per-group (per-expert) current-scaling quantizer and of
the grouped FP8 GEMM with per-group scales against the oracle, through the C
ABI.  Codes and scales must be bit-exact; GEMM outputs within the tolerance
of oracle.gemm (1e-5 * S + 1e-6 plus the FP8 matrix-unit allowance)."""

import numpy as np
import pytest
import torch

from block_quant_gemm_amd import mxq, workloads
from oracle import codec, gemm, per_tensor
from tests import fp8_mode as f8
from tests.gpu_helpers import host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

ACCS = [mxq.ACC_FP32, mxq.ACC_MFMA_FP8]


def _quant(bits, offs):
    q, s = mxq.fp8_quantize_per_group(to_dev_bf16(bits), to_dev(offs))
    return q, s, host(q), host(s)


def _assert_quant_equal(bits, offs, qh, sh):
    rq, rs = per_tensor.pg_quantize(bits, offs)
    assert np.array_equal(sh.view(np.uint32), rs.view(np.uint32)), (sh, rs)
    if not np.array_equal(qh, rq):
        bad = np.argwhere(qh != rq)[:8]
        raise AssertionError(f"codes differ at {bad.tolist()}: "
                             f"{qh[tuple(bad.T)].tolist()} vs {rq[tuple(bad.T)].tolist()}")


@pytest.mark.parametrize("counts,K", [
    ([40, 0, 1, 130, 0, 300, 0], 64),
    ([0, 0, 257], 136),
    ([5], 8),
    ([1000, 17, 0, 2, 511], 2048),
    ([0], 32),
])
def test_per_group_quant_bit_exact(counts, K):
    say(f"per-group quant counts={counts} K={K}")
    counts = np.array(counts, np.int64)
    offs = workloads.offsets_from_counts(counts)
    x = workloads.bf16_normal((int(counts.sum()), K), 1.0, seed=K, name="pgx",
                              outlier_frac=0.01, outlier_scale=100.0)
    _, _, qh, sh = _quant(x, offs)
    _assert_quant_equal(x, offs, qh, sh)


def test_per_group_quant_special_groups():
    """NaN, Inf, all-zero, subnormal-scale, amax = 448 (s = 1) and empty
    groups side by side; a group's special values affect that group only."""
    say("per-group quant special groups")
    counts = np.array([8, 8, 8, 0, 8, 8, 8], np.int64)
    offs = workloads.offsets_from_counts(counts)
    K = 64
    x = workloads.bf16_normal((48, K), 1.0, seed=3, name="pgs")
    x[offs[0] + 2, 7] = 0x7FC0                       # NaN in group 0
    x[offs[1] + 5, 1] = 0xFF80                       # -Inf in group 1
    x[offs[2]:offs[3]] = 0                           # zeros in group 2 (+0 and -0)
    x[offs[2] + 1, ::2] = 0x8000
    tiny = workloads.bf16_normal((8, K), 1.0, seed=4, name="pgt")
    v = codec.bf16_bits_to_f64(tiny) * 2.0 ** -122   # amax / 448 is FP32-subnormal
    t32 = torch.tensor(v, dtype=torch.float32).to(torch.bfloat16)
    x[offs[4]:offs[5]] = t32.view(torch.int16).numpy().view(np.uint16)
    x[offs[5] + 3, 9] = 0x43E0                       # 448 in group 5
    x[offs[5]:offs[6]] &= 0xBFFF                     # keep the rest small: |v| < 2
    x[offs[5] + 3, 9] = 0x43E0
    _, _, qh, sh = _quant(x, offs)
    _assert_quant_equal(x, offs, qh, sh)
    assert sh[0] == 1.0 and sh[1] == 1.0 and sh[2] == 1.0 and sh[3] == 1.0
    assert sh[4] < np.float32(1.17549435e-38)
    assert sh[5] == 1.0


def test_per_group_quant_strided_and_weights():
    """Row strides beyond K and a 3-D weight stack with offsets e*N."""
    say("per-group quant strided / weight stack")
    E, N, K = 6, 96, 160
    w = workloads.bf16_normal((E * N, K), 0.02, seed=5, name="pgw")
    offs = np.arange(E + 1, dtype=np.int64) * N
    xs = torch.zeros((E * N, K + 24), dtype=torch.bfloat16, device="cuda")
    xs[:, :K] = to_dev_bf16(w)
    q = torch.full((E * N, K + 16), 0xA5, dtype=torch.uint8, device="cuda")
    qv, sc = mxq.fp8_quantize_per_group(xs[:, :K], to_dev(offs), q=q[:, :K])
    torch.cuda.synchronize()
    _assert_quant_equal(w, offs, host(qv), host(sc))
    assert torch.all(q[:, K:] == 0xA5)


def test_per_group_quant_full_size_moe():
    """X [49152, 2048] over the 64 Zipf expert groups and W_gu [64*2816, 2048]
    per expert, bit-exact against the oracle."""
    say("per-group quant X 49152x2048 and W_gu 180224x2048")
    d = workloads.moe_forward(0)
    offs = d["offsets"]
    _, _, qh, sh = _quant(d["X"], offs)
    _assert_quant_equal(d["X"], offs, qh, sh)
    w = d["W_gu"].reshape(64 * 2816, 2048)
    woffs = np.arange(65, dtype=np.int64) * 2816
    _, _, qh, sh = _quant(w, woffs)
    _assert_quant_equal(w, woffs, qh, sh)


def _gemm_allowance(ah, bh, sa, sb, offs, N):
    """MFMA allowance (unit block scales) times the group's two scales, plus
    the two FP32 roundings of multiplying the scales into the sum."""
    E = len(offs) - 1
    K = ah.shape[1]
    T = np.zeros((ah.shape[0], N))
    ones_a = np.full((ah.shape[0], K // 32), 127, np.uint8)
    ones_b = np.full((N, K // 32), 127, np.uint8)
    for e in range(E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi > lo:
            T[lo:hi] = f8.fp8_mfma_truncation_bound(
                ah[lo:hi], ones_a[lo:hi], bh[e * N:(e + 1) * N], ones_b) * \
                float(sa[e]) * float(sb[e])
    return T


@pytest.mark.parametrize("counts,N,K", [
    ([40, 0, 1, 130, 0, 300, 0], 160, 256),
    ([300, 0, 45, 513], 768, 192),
    ([5], 32, 32),
])
@pytest.mark.parametrize("out", [mxq.OUT_BF16, mxq.OUT_FP32])
@pytest.mark.parametrize("accum", ACCS)
def test_per_group_grouped_gemm(counts, N, K, out, accum):
    say(f"per-group grouped gemm counts={counts} N={N} K={K} out={out} accum={accum}")
    counts = np.array(counts, np.int64)
    offs = workloads.offsets_from_counts(counts)
    E, M = len(counts), int(counts.sum())
    a = workloads.bf16_normal((M, K), 1.0, seed=M + K, name="pga", outlier_frac=0.005,
                              outlier_scale=50.0)
    w = workloads.bf16_normal((E * N, K), 0.02, seed=N + K, name="pgb")
    woffs = np.arange(E + 1, dtype=np.int64) * N
    aq, sa, ah, sah = _quant(a, offs)
    wq, sw, wh, swh = _quant(w, woffs)
    c = mxq.fp8_grouped_gemm_per_group(aq, sa, wq.view(E, N, K), sw, to_dev(offs),
                                       out_dtype=out, accum=accum)
    A = per_tensor.pg_dequantize(ah, sah, offs)
    B = per_tensor.pg_dequantize(wh, swh, woffs).reshape(E, N, K)
    Y, S = gemm.grouped_gemm_ref(A, B, offs)
    f8.accept(host(c), Y, S, out == mxq.OUT_FP32, accum == mxq.ACC_FP32,
              lambda: _gemm_allowance(ah, wh, sah, swh, offs, N) + 2.0 ** -23 * np.abs(Y))


def test_per_group_one_group_equals_per_tensor():
    """One group spanning all rows is the per-tensor recipe: same codes,
    same scale, same GEMM output bit for bit."""
    say("per-group with one group == per-tensor")
    a = workloads.bf16_normal((300, 256), 1.0, seed=9, name="pgo")
    w = workloads.bf16_normal((72, 256), 0.02, seed=9, name="pgw2")
    one = to_dev(np.array([0, 300], np.int64))
    aq, sa = mxq.fp8_quantize_per_group(to_dev_bf16(a), one)
    wq, sw = mxq.fp8_quantize_per_group(to_dev_bf16(w), to_dev(np.array([0, 72], np.int64)))
    pq, ps = mxq.fp8_quantize_per_tensor(to_dev_bf16(a))
    assert torch.equal(aq, pq) and torch.equal(sa, ps)
    cg = mxq.fp8_grouped_gemm_per_group(aq, sa, wq.view(1, 72, 256), sw, one,
                                        out_dtype=mxq.OUT_FP32)
    cd = mxq.fp8_gemm_per_tensor(aq, sa, wq, sw, out_dtype=mxq.OUT_FP32)
    assert torch.equal(cg, cd)


@pytest.mark.parametrize("accum", ACCS)
def test_per_group_gate_up_full_size_sampled(accum):
    """MoE gate_up forward at full size with per-expert scales: 49152 rows,
    64 experts, W_gu [64, 2816, 2048]; 2000 sampled outputs."""
    say(f"per-group grouped gate_up 49152 x 2816 x 2048 accum={accum}")
    d = workloads.moe_forward(0)
    offs, E = d["offsets"], 64
    w = d["W_gu"].reshape(E * 2816, 2048)
    woffs = np.arange(E + 1, dtype=np.int64) * 2816
    aq, sa, ah, sah = _quant(d["X"], offs)
    wq, sw, wh, swh = _quant(w, woffs)
    c = mxq.fp8_grouped_gemm_per_group(aq, sa, wq.view(E, 2816, 2048), sw, to_dev(offs),
                                       accum=accum)
    rng = np.random.default_rng(2)
    rows = rng.integers(0, 49152, 2000)
    n = rng.integers(0, 2816, 2000)
    e = np.searchsorted(offs, rows, side="right") - 1
    cols = e * 2816 + n
    idx = np.arange(len(rows))
    A = per_tensor.pt_dequantize(ah[rows], np.float32(1.0)) * sah[e].astype(np.float64)[:, None]
    B = per_tensor.pt_dequantize(wh[cols], np.float32(1.0)) * swh[e].astype(np.float64)[:, None]
    Y, S = gemm.gemm_ref_entries(A, B, idx, idx)
    ones = np.full((len(rows), 64), 127, np.uint8)
    ch = host(c)[rows, n]
    f8.accept(ch, Y, S, False, accum == mxq.ACC_FP32,
              lambda: f8.fp8_mfma_truncation_bound(ah[rows], ones, wh[cols], ones, idx, idx) *
              sah[e].astype(np.float64) * swh[e].astype(np.float64) + 2.0 ** -23 * np.abs(Y))


# ---------------------------------------------------------------------------
# transposed copy (dgrad / wgrad operands)
# ---------------------------------------------------------------------------

def _colwise(bits, offs, M_cap=None):
    qT, s, poff = mxq.fp8_quantize_per_group_colwise(to_dev_bf16(bits), to_dev(offs),
                                                     M_cap=M_cap)
    return qT, s, poff, host(qT), host(s), host(poff)


def _assert_colwise_equal(bits, offs, qTh, sh, ph):
    rq, rs, rp = per_tensor.pg_quantize_colwise(bits, offs)
    assert np.array_equal(ph, rp)
    assert np.array_equal(sh.view(np.uint32), rs.view(np.uint32))
    Mp = int(rp[-1])
    if not np.array_equal(qTh[:, :Mp], rq):
        bad = np.argwhere(qTh[:, :Mp] != rq)[:8]
        raise AssertionError(f"codes differ at {bad.tolist()}")
    assert np.all(qTh[:, Mp:] == 0), "columns past the padded total"


@pytest.mark.parametrize("counts,K", [
    ([40, 0, 1, 130, 0, 300, 0], 64),
    ([0, 0, 257], 136),
    ([5], 8),
    ([1000, 17, 0, 2, 511], 2048),
])
def test_per_group_colwise_bit_exact(counts, K):
    say(f"per-group colwise counts={counts} K={K}")
    counts = np.array(counts, np.int64)
    offs = workloads.offsets_from_counts(counts)
    x = workloads.bf16_normal((int(counts.sum()), K), 1.0, seed=K + 1, name="pgcx",
                              outlier_frac=0.01, outlier_scale=100.0)
    _, _, _, qTh, sh, ph = _colwise(x, offs)
    _assert_colwise_equal(x, offs, qTh, sh, ph)


def test_per_group_colwise_special_groups_and_capacity():
    """NaN / Inf / zero / subnormal-scale groups, and a capacity well past the
    padded total (zero-filled)."""
    say("per-group colwise special groups")
    counts = np.array([8, 40, 8, 0, 33, 8], np.int64)
    offs = workloads.offsets_from_counts(counts)
    K = 96
    x = workloads.bf16_normal((int(counts.sum()), K), 1.0, seed=6, name="pgcs")
    x[offs[0] + 2, 7] = 0xFFC0                        # -NaN in group 0
    x[offs[1] + 5, 1] = 0x7F80                        # +Inf in group 1
    x[offs[1] + 9, 3] = 0xFFC0                        # and a NaN
    x[offs[2]:offs[3]] = 0x8000                       # -0 in group 2
    tiny = workloads.bf16_normal((33, K), 1.0, seed=7, name="pgct")
    v = codec.bf16_bits_to_f64(tiny) * 2.0 ** -122
    x[offs[4]:offs[5]] = torch.tensor(v, dtype=torch.float32).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)
    _, _, _, qTh, sh, ph = _colwise(x, offs, M_cap=512)
    _assert_colwise_equal(x, offs, qTh, sh, ph)


def test_per_group_colwise_full_size_sampled_columns():
    """dGU [49152, 2816] over the 64 Zipf groups: 32 sampled columns."""
    say("per-group colwise dGU 49152x2816")
    counts = workloads.moe_counts(0)
    offs = workloads.offsets_from_counts(counts)
    dGU = workloads.moe_backward(0)["dGU"]
    qT, s, poff, _, sh, ph = _colwise(dGU, offs)
    # the group scales depend on every column: take them from the full tensor
    rq, rs = per_tensor.pg_quantize(dGU, offs)
    assert np.array_equal(sh.view(np.uint32), rs.view(np.uint32))
    cols = np.random.default_rng(3).choice(dGU.shape[1], 32, replace=False)
    rp = np.concatenate([[0], np.cumsum((np.diff(offs) + 31) // 32 * 32)])
    assert np.array_equal(ph, rp)
    qh = host(qT[torch.from_numpy(cols).cuda()])
    for e in range(len(offs) - 1):
        lo, hi, p = int(offs[e]), int(offs[e + 1]), int(rp[e])
        assert np.array_equal(qh[:, p:p + hi - lo], rq[lo:hi, cols].T)
        assert np.all(qh[:, p + hi - lo:int(rp[e + 1])] == 0)


def _dequant_colwise(qTh, sh, ph):
    """Exact values of a transposed per-group copy: group columns times their scale."""
    out = np.zeros(qTh.shape)
    for e in range(len(ph) - 1):
        lo, hi = int(ph[e]), int(ph[e + 1])
        if hi > lo:
            out[:, lo:hi] = per_tensor.pt_dequantize(qTh[:, lo:hi], sh[e])
    return out


@pytest.mark.parametrize("counts,N,K", [
    ([40, 0, 1, 130, 0, 300, 0], 160, 96),
    ([300, 0, 45, 513], 296, 768),
])
@pytest.mark.parametrize("out", [mxq.OUT_BF16, mxq.OUT_FP32])
@pytest.mark.parametrize("accum", ACCS)
def test_per_group_wgrad(counts, N, K, out, accum):
    say(f"per-group wgrad counts={counts} N={N} K={K} out={out} accum={accum}")
    counts = np.array(counts, np.int64)
    offs = workloads.offsets_from_counts(counts)
    E, T = len(counts), int(counts.sum())
    dy = workloads.bf16_normal((T, N), 1e-3, seed=T + N, name="pgwd", outlier_frac=0.005,
                               outlier_scale=30.0)
    x = workloads.bf16_normal((T, K), 1.0, seed=T + K, name="pgwx")
    aT, sa, poff, aTh, sah, ph = _colwise(dy, offs)
    bT, sb, _, bTh, sbh, _ = _colwise(x, offs)
    c = mxq.fp8_grouped_gemm_wgrad_per_group(aT, sa, bT, sb, poff, out_dtype=out, accum=accum)
    A, B = _dequant_colwise(aTh, sah, ph), _dequant_colwise(bTh, sbh, ph)
    Y, S = gemm.grouped_wgrad_ref(A[:, :int(ph[-1])], B[:, :int(ph[-1])], ph)
    Tb = np.zeros_like(Y)
    for e in range(E):
        lo, hi = int(ph[e]), int(ph[e + 1])
        if hi > lo:
            ones_a = np.full((N, (hi - lo) // 32), 127, np.uint8)
            ones_b = np.full((K, (hi - lo) // 32), 127, np.uint8)
            Tb[e] = f8.fp8_mfma_truncation_bound(aTh[:, lo:hi], ones_a, bTh[:, lo:hi],
                                                   ones_b) * float(sah[e]) * float(sbh[e])
    Tb = Tb + 2.0 ** -23 * np.abs(Y)
    f8.accept(host(c), Y, S, out == mxq.OUT_FP32, accum == mxq.ACC_FP32, Tb)
    for e in np.nonzero(counts == 0)[0]:
        assert torch.all(c[e] == 0)


@pytest.mark.parametrize("accum", ACCS)
def test_per_group_dgrad_with_transposed_weights(accum):
    """Data gradient dX = dY · W_e per expert: the weights' transposed
    per-expert copy read in place through per-expert strides."""
    say(f"per-group dgrad accum={accum}")
    counts = np.array([40, 0, 130, 77], np.int64)
    offs = workloads.offsets_from_counts(counts)
    E, M, N, K = 4, int(counts.sum()), 192, 320     # W_e [N, K]; dY [M, N]; dX [M, K]
    w = workloads.bf16_normal((E * N, K), 0.02, seed=21, name="pgdw")
    dy = workloads.bf16_normal((M, N), 1e-3, seed=21, name="pgdy")
    woffs = np.arange(E + 1, dtype=np.int64) * N
    wT, sw, _, wTh, swh, wph = _colwise(w, woffs)    # [K, E*N]
    gq, sg, gh, sgh = _quant(dy, offs)
    bview = wT[:, :E * N].view(K, E, N).permute(1, 0, 2)  # [E, K, N], expert stride N
    c = mxq.fp8_grouped_gemm_per_group(gq, sg, bview, sw, to_dev(offs), out_dtype=mxq.OUT_FP32,
                                       accum=accum)
    A = per_tensor.pg_dequantize(gh, sgh, offs)
    Bt = _dequant_colwise(wTh, swh, wph)             # [K, E*N]
    B = np.stack([Bt[:, e * N:(e + 1) * N] for e in range(E)])   # [E, K, N]
    Y, S = gemm.grouped_gemm_ref(A, B, offs)
    T = np.zeros_like(Y)
    onesa = np.full((M, N // 32), 127, np.uint8)
    onesb = np.full((K, N // 32), 127, np.uint8)
    for e in range(E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi > lo:
            T[lo:hi] = f8.fp8_mfma_truncation_bound(gh[lo:hi], onesa[lo:hi],
                                                      wTh[:, e * N:(e + 1) * N], onesb) * \
                float(sgh[e]) * float(swh[e])
    T = T + 2.0 ** -23 * np.abs(Y)
    f8.accept(host(c), Y, S, True, accum == mxq.ACC_FP32, T)


# ---------------------------------------------------------------------------
# both copies in one pass
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("counts,K", [
    ([40, 0, 1, 130, 0, 300, 0], 64),
    ([1000, 17, 0, 2, 511], 2048),
    ([5], 8),
    ([0, 0, 257], 136),
])
def test_per_group_dual_bit_exact(counts, K):
    say(f"per-group dual quant counts={counts} K={K}")
    offs = workloads.offsets_from_counts(np.array(counts, np.int64))
    M = int(offs[-1])
    x = workloads.bf16_normal((M, K), 1.0, seed=M + 3 * K, name="pgd", outlier_frac=0.01,
                              outlier_scale=40.0)
    q, qT, s, poff = mxq.fp8_quantize_per_group_dual(to_dev_bf16(x), to_dev(offs))
    rq, rs = per_tensor.pg_quantize(x, offs)
    cq, cs, cp = per_tensor.pg_quantize_colwise(x, offs)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(cs.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(poff), cp)
    assert np.array_equal(host(qT)[:, :int(cp[-1])], cq)


def test_per_group_dual_special_groups():
    """NaN, Inf, zero and empty groups, as the oracle."""
    K = 64
    offs = np.array([0, 3, 3, 40, 41, 90], np.int64)
    vals = np.random.default_rng(8).normal(0, 1, (90, K))
    vals[1, 5] = np.nan
    vals[20, 0] = np.inf
    vals[40] = 0.0
    bits = codec.bf16_round_to_bits(vals)
    q, qT, s, poff = mxq.fp8_quantize_per_group_dual(to_dev_bf16(bits), to_dev(offs))
    rq, rs = per_tensor.pg_quantize(bits, offs)
    cq, _, cp = per_tensor.pg_quantize_colwise(bits, offs)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(qT)[:, :int(cp[-1])], cq)


def test_per_group_dual_equals_single_copies_full_size():
    """dGU [49152, 2816] over the 64 expert groups, and W_gu [64 x 2816, 2048]
    with one group per expert: byte-equal to the row-major and transposed
    single-copy quantizers (each pinned to the oracle above)."""
    say("per-group dual quant, full-size dGU and W_gu")
    bw = workloads.moe_backward(0)
    fw = workloads.moe_forward(0)
    cases = [(bw["dGU"], fw["offsets"]),
             (fw["W_gu"].reshape(64 * 2816, 2048), np.arange(65, dtype=np.int64) * 2816)]
    for bits, offs in cases:
        xd, od = to_dev_bf16(bits), to_dev(offs)
        q, qT, s, poff = mxq.fp8_quantize_per_group_dual(xd, od)
        q1, s1 = mxq.fp8_quantize_per_group(xd, od)
        qT2, s2, p2 = mxq.fp8_quantize_per_group_colwise(xd, od)
        Mp = int(host(p2)[-1])
        assert torch.equal(q, q1) and torch.equal(s, s1) and torch.equal(s, s2)
        assert torch.equal(poff, p2) and torch.equal(qT[:, :Mp], qT2[:, :Mp])


def test_per_group_dual_with_given_amax():
    """With the groups' amaxes given, the same codes and scales as the oracle."""
    offs = workloads.offsets_from_counts(np.array([300, 0, 1, 77], np.int64))
    x = workloads.bf16_normal((378, 256), 1.0, seed=4, name="pgda", outlier_frac=0.02,
                              outlier_scale=20.0)
    xv = codec.bf16_bits_to_f64(x)
    amax = np.array([np.abs(xv[offs[e]:offs[e + 1]]).max() if offs[e + 1] > offs[e] else 0.0
                     for e in range(4)], np.float32)
    q, qT, s, poff = mxq.fp8_quantize_per_group_dual(to_dev_bf16(x), to_dev(offs),
                                                     amax=to_dev(amax))
    rq, rs = per_tensor.pg_quantize(x, offs)
    cq, _, cp = per_tensor.pg_quantize_colwise(x, offs)
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(qT)[:, :int(cp[-1])], cq)
