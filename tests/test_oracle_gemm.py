"""Pins of the GEMM oracle: exact brute force with Fractions, the integer
special case, reductions between grouped and dense forms, and the acceptance
check itself.  CPU only."""

from fractions import Fraction

import numpy as np

from oracle import codec, gemm, mx, per_tensor
from block_quant_gemm_amd import workloads


def frac_e4m3(c):
    """Exact value of an E4M3 code from its bit fields, in Fractions."""
    s = -1 if c & 0x80 else 1
    e = (c >> 3) & 0xF
    m = c & 7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 64)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def brute_mx_gemm(aq, asc, bq, bsc):
    M, K = aq.shape
    N = bq.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            for k in range(K):
                sa = Fraction(2) ** (int(asc[i, k // 32]) - 127)
                sb = Fraction(2) ** (int(bsc[j, k // 32]) - 127)
                acc += frac_e4m3(int(aq[i, k])) * sa * frac_e4m3(int(bq[j, k])) * sb
            out[i][j] = acc
    return out


def _q(shape, sigma, seed, name, **kw):
    return mx.mx_quantize_rowwise(workloads.bf16_normal(shape, sigma, seed=seed,
                                                        name=name, **kw))


def test_brute_force_tiny_mx_gemm():
    aq, asc = _q((3, 96), 1.0, 1, "ga", outlier_frac=0.05, outlier_scale=100.0)
    bq, bsc = _q((4, 96), 0.02, 1, "gb")
    Y, S = gemm.gemm_ref(mx.mx_dequantize(aq, asc), mx.mx_dequantize(bq, bsc))
    ref = brute_mx_gemm(aq, asc, bq, bsc)
    for i in range(3):
        for j in range(4):
            assert abs(Fraction(Y[i, j]) - ref[i][j]) <= Fraction(96) * Fraction(2) ** -53 * Fraction(S[i, j])


def test_integer_special_case():
    """All scales 2^0 and codes of small integers: an int64 matmul."""
    rng = np.random.default_rng(0)
    ints = np.arange(-16, 17)
    codes_of = {int(v): int(codec.e4m3_encode(np.array([float(v)]))[0]) for v in ints}
    A = rng.choice(ints, size=(16, 128))
    B = rng.choice(ints, size=(8, 128))
    aq = np.vectorize(codes_of.get)(A).astype(np.uint8)
    bq = np.vectorize(codes_of.get)(B).astype(np.uint8)
    ones_a = np.full((16, 4), 127, np.uint8)
    ones_b = np.full((8, 4), 127, np.uint8)
    Y, S = gemm.gemm_ref(mx.mx_dequantize(aq, ones_a), mx.mx_dequantize(bq, ones_b))
    assert np.array_equal(Y, (A @ B.T).astype(np.float64))
    assert np.array_equal(S, (np.abs(A) @ np.abs(B).T).astype(np.float64))


def test_mx_unit_scale_equals_per_tensor_unit_scale():
    rng = np.random.default_rng(1)
    aq = rng.integers(0, 0x7E, (8, 64)).astype(np.uint8)
    bq = rng.integers(0, 0x7E, (8, 64)).astype(np.uint8)
    u = np.full((8, 2), 127, np.uint8)
    Ya, _ = gemm.gemm_ref(mx.mx_dequantize(aq, u), mx.mx_dequantize(bq, u))
    Yb, _ = gemm.gemm_ref(per_tensor.pt_dequantize(aq, 1.0), per_tensor.pt_dequantize(bq, 1.0))
    assert np.array_equal(Ya, Yb)


def test_grouped_one_expert_equals_dense():
    aq, asc = _q((70, 64), 1.0, 2, "g1a")
    bq, bsc = _q((48, 64), 0.02, 2, "g1b")
    A, B = mx.mx_dequantize(aq, asc), mx.mx_dequantize(bq, bsc)
    Yg, Sg = gemm.grouped_gemm_ref(A, B[None], np.array([0, 70]))
    Yd, Sd = gemm.gemm_ref(A, B)
    assert np.array_equal(Yg, Yd) and np.array_equal(Sg, Sd)


def test_grouped_rows_use_their_expert():
    counts = np.array([5, 0, 7, 0, 3])
    offs = workloads.offsets_from_counts(counts)
    A = np.random.default_rng(3).standard_normal((15, 64))
    B = np.random.default_rng(4).standard_normal((5, 6, 64))
    Y, S = gemm.grouped_gemm_ref(A, B, offs)
    for r in range(15):
        e = int(np.searchsorted(offs, r, side="right") - 1)
        assert np.allclose(Y[r], B[e] @ A[r], rtol=0, atol=1e-12)


def test_wgrad_one_expert_is_dense_on_transposes_and_empty_is_zero():
    rng = np.random.default_rng(5)
    at = rng.standard_normal((6, 64))
    bt = rng.standard_normal((5, 64))
    Y, S = gemm.grouped_wgrad_ref(at, bt, np.array([0, 0, 64, 64]))
    assert np.all(Y[0] == 0) and np.all(Y[2] == 0) and np.all(S[0] == 0)
    Yd, _ = gemm.gemm_ref(at, bt)
    assert np.array_equal(Y[1], Yd)


def test_wgrad_sum_over_tokens():
    rng = np.random.default_rng(6)
    at = rng.standard_normal((3, 96))
    bt = rng.standard_normal((2, 96))
    offs = np.array([0, 32, 96])
    Y, _ = gemm.grouped_wgrad_ref(at, bt, offs)
    for e in range(2):
        for n in range(3):
            for k in range(2):
                ref = sum(at[n, t] * bt[k, t] for t in range(offs[e], offs[e + 1]))
                assert abs(Y[e, n, k] - ref) < 1e-12


def test_acceptance_check_fp32_and_planted_mistakes():
    aq, asc = _q((32, 256), 1.0, 7, "ca")
    bq, bsc = _q((24, 256), 1.0, 7, "cb")
    A, B = mx.mx_dequantize(aq, asc), mx.mx_dequantize(bq, bsc)
    Y, S = gemm.gemm_ref(A, B)
    c32 = (A.astype(np.float32) @ B.astype(np.float32).T)      # FP32 accumulate
    assert gemm.check_fp32(c32, Y, S).all()
    # planted mistakes: a dropped k-block, a transposed operand, a wrong sign
    dropped, _ = gemm.gemm_ref(A[:, :224], B[:, :224])
    assert not gemm.check_fp32(dropped, Y, S).all()
    assert not gemm.check_fp32(-Y, Y, S).all()
    wrong_b, _ = gemm.gemm_ref(A, B[::-1])
    assert not gemm.check_fp32(wrong_b, Y, S).all()


def test_acceptance_check_bf16_bracket():
    Y = np.array([1.0, 1.0, 1.00390625, 3.0, -5.0])
    S = np.zeros(5)
    ok = codec.bf16_round_to_bits(Y)
    assert gemm.check_bf16(ok, Y, S).all()
    # one BF16 ulp off with a tiny tolerance fails
    bad = ok.copy()
    bad[0] += 1
    assert not gemm.check_bf16(bad, Y, S)[0]
    # midpoint 1 + 2^-8: both neighbours lie within tol when S is large enough
    Y2 = np.array([1.00390625])
    lo = codec.bf16_round_to_bits(np.array([1.0]))
    hi = codec.bf16_round_to_bits(np.array([1.0078125]))
    assert gemm.check_bf16(lo, Y2, np.array([1e3])).all()
    assert gemm.check_bf16(hi, Y2, np.array([1e3])).all()
    # just below the tie, farther than the 1e-6 absolute floor: only 1.0
    Y3 = np.array([1.00390625 - 1e-5])
    assert gemm.check_bf16(lo, Y3, np.array([0.0])).all()
    assert not gemm.check_bf16(hi, Y3, np.array([0.0])).all()
