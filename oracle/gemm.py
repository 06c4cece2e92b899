"""GEMM oracle: dequantize, then multiply in float64.  Test infrastructure.

[HP329] §8: forward, dgrad and wgrad are each one quantized matmul on the
oriented operands; §13.4: ``low_precision_matmul`` / ``low_precision_grouped_
matmul(left, right, group_list, ...)`` return a high-precision output.
[FPBLOG] §五.1: low-precision inputs are multiplied and the products summed in
an FP32 accumulator, then rounded once to BF16.  [FPBLOG] §八.3: a kernel's
difference from a reference is judged against sum_k |a_k b_k| when terms
cancel.

The oracle's plain definition: with Â and B̂ the exact dequantized operands,
``Y = Â · B̂ᵀ`` in float64 and the cancellation-free magnitude
``S = |Â| · |B̂|ᵀ``.  A result C is accepted per element when
``|C - Y| <= 1e-5 * S + 1e-6`` (FP32 output), or, for BF16 output, when C is
the BF16 rounding of some value within that distance of Y.
"""

import numpy as np

from .codec import bf16_bits_to_f64, bf16_round

REL_TOL = 1e-5
ABS_TOL = 1e-6


def gemm_ref(a_vals, b_vals):
    """Y = A · Bᵀ and S = |A| · |B|ᵀ in float64; A [M, K], B [N, K]."""
    a = np.asarray(a_vals, dtype=np.float64)
    b = np.asarray(b_vals, dtype=np.float64)
    return a @ b.T, np.abs(a) @ np.abs(b).T


def gemm_ref_entries(a_vals, b_vals, rows, cols):
    """Selected entries Y[rows[i], cols[i]] and S of A · Bᵀ, one dot each."""
    a = np.asarray(a_vals, dtype=np.float64)[rows]
    b = np.asarray(b_vals, dtype=np.float64)[cols]
    return np.einsum("ik,ik->i", a, b), np.einsum("ik,ik->i", np.abs(a), np.abs(b))


def grouped_gemm_ref(a_vals, b_vals, offsets):
    """Variable-M grouped GEMM: rows [o_e, o_{e+1}) of A times B_eᵀ.

    A [M, K], B [E, N, K], offsets [E+1] -> Y, S [M, N].  An empty group
    contributes no rows.
    """
    a = np.asarray(a_vals, dtype=np.float64)
    b = np.asarray(b_vals, dtype=np.float64)
    E, N, _ = b.shape
    M = a.shape[0]
    Y = np.zeros((M, N))
    S = np.zeros((M, N))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            Y[lo:hi], S[lo:hi] = gemm_ref(a[lo:hi], b[e])
    return Y, S


def grouped_wgrad_ref(at_vals, bt_vals, offsets):
    """Variable-K grouped GEMM (weight gradient), contraction over tokens.

    Aᵀ [N, T] and Bᵀ [K, T] hold the token dimension T contiguously; group e
    owns tokens [o_e, o_{e+1}).  dW_e = Aᵀ[:, group] · (Bᵀ[:, group])ᵀ, shape
    [N, K]; an empty group gives dW_e = 0.  Returns Y, S [E, N, K].
    """
    at = np.asarray(at_vals, dtype=np.float64)
    bt = np.asarray(bt_vals, dtype=np.float64)
    E = len(offsets) - 1
    N, K = at.shape[0], bt.shape[0]
    Y = np.zeros((E, N, K))
    S = np.zeros((E, N, K))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            Y[e], S[e] = gemm_ref(at[:, lo:hi], bt[:, lo:hi])
    return Y, S


def tolerance(S):
    return REL_TOL * np.asarray(S, dtype=np.float64) + ABS_TOL


def check_fp32(c, Y, S):
    """Boolean mask of elements of an FP32 result C that pass."""
    c = np.asarray(c, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        ok = np.abs(c - Y) <= tolerance(S)
    both_nan = np.isnan(c) & np.isnan(Y)
    return ok | both_nan


def check_bf16(c_bits, Y, S):
    """Boolean mask of elements of a BF16 result (bit patterns) that pass.

    Rounding to BF16 is monotone, so C is the rounding of some value in
    [Y - tol, Y + tol] exactly when bf16(Y - tol) <= C <= bf16(Y + tol).
    """
    c = bf16_bits_to_f64(c_bits)
    tol = tolerance(S)
    lo = bf16_round(Y - tol)
    hi = bf16_round(Y + tol)
    with np.errstate(invalid="ignore"):
        ok = (c >= lo) & (c <= hi)
    both_nan = np.isnan(c) & np.isnan(Y)
    return ok | both_nan
