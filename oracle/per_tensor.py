"""Per-tensor current-scaling FP8 (E4M3) oracle.  Test infrastructure.

[HP329] §3.2: the current-scaling recipe divides the tensor's amax by the
format's largest value when that amax is usable, and uses 1 otherwise; the
scale is held in FP32 and recomputed from the current tensor each call.  [FPBLOG] §七.2: per-tensor scaling shares one scale over the whole
tensor, found by a first pass over it (amax), then a second pass quantizes.

Readings: format_max is E4M3's 448; "valid" means finite and > 0; amax is
NaN-propagating; the data are ``E4M3_RNE_sat(fp32(x) / scale)`` with an IEEE
FP32 division (round to nearest even), and dequantization is ``q * scale``.
"""

import numpy as np

from .codec import E4M3_MAX, bf16_bits_to_f64, e4m3_decode, e4m3_encode


def pt_scale(x_bf16_bits):
    """FP32 scale of a BF16 tensor: fp32(amax) / fp32(448), or 1.0."""
    x = bf16_bits_to_f64(np.asarray(x_bf16_bits).ravel())
    if x.size == 0:
        return np.float32(1.0)
    a = np.abs(x)
    amax = np.nan if np.isnan(a).any() else a.max()
    if not np.isfinite(amax) or amax <= 0:
        return np.float32(1.0)
    # amax is a BF16 value, so float32(amax) is exact; the division is FP32.
    return np.float32(amax) / np.float32(E4M3_MAX)


def pt_quantize(x_bf16_bits):
    """Returns (codes uint8 of x's shape, scale np.float32)."""
    bits = np.asarray(x_bf16_bits, dtype=np.uint16)
    s = pt_scale(bits)
    x32 = bf16_bits_to_f64(bits).astype(np.float32)      # exact
    with np.errstate(over="ignore", invalid="ignore"):
        q = x32 / np.float32(s)                          # IEEE FP32, RNE
    return e4m3_encode(q.astype(np.float64)), np.float32(s)


def pt_scale_of_amax(amax):
    """The scale rule applied to an amax that is given rather than found by a
    pass over the tensor ([FPBLOG] §七.2: the producing matmul can supply the
    amax): fp32(amax) / fp32(448) when amax is finite and > 0, else 1.0."""
    a = np.float32(amax)
    if not np.isfinite(a) or a <= 0:
        return np.float32(1.0)
    return a / np.float32(E4M3_MAX)


def pt_quantize_given_amax(x_bf16_bits, amax):
    """pt_quantize with the scale taken from a given amax.  Returns (codes
    uint8 of x's shape, scale np.float32)."""
    bits = np.asarray(x_bf16_bits, dtype=np.uint16)
    s = pt_scale_of_amax(amax)
    x32 = bf16_bits_to_f64(bits).astype(np.float32)      # exact
    with np.errstate(over="ignore", invalid="ignore"):
        q = x32 / np.float32(s)                          # IEEE FP32, RNE
    return e4m3_encode(q.astype(np.float64)), np.float32(s)


def pt_dequantize(codes, scale):
    """Exact float64 values q * scale."""
    return e4m3_decode(codes) * np.float64(np.float32(scale))


def pg_quantize(x_bf16_bits, offsets):
    """Per-group current scaling of a 2-D BF16 tensor whose rows are grouped
    by expert: rows [offsets[e], offsets[e+1]) share one FP32 scale, found by
    the per-tensor rule above from that group's own amax.

    [HP329] §3 (format table: HiF8 current scaling keeps one FP32 scale per
    dense tensor and, for grouped tensors, one per leading group) and §3.2
    (the scale rule above; 3-D grouped weights use a per-leading-group
    scale); [TTNPU] MoE expert layers (each expert
    group shares one scale).  Reading: the groups of a [M, K] activation are
    its expert row ranges; a 3-D weight [E, N, K] is the same with offsets
    e * N; an empty group gets 1.0.

    Returns (codes uint8 [M, K], scales float32 [E])."""
    bits = np.asarray(x_bf16_bits, dtype=np.uint16)
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.size - 1
    codes = np.zeros(bits.shape, dtype=np.uint8)
    scales = np.ones(E, dtype=np.float32)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            codes[lo:hi], scales[e] = pt_quantize(bits[lo:hi])
    return codes, scales


def pg_dequantize(codes, scales, offsets):
    """Exact float64 values: row r of group e is codes[r] * scales[e]."""
    offsets = np.asarray(offsets, dtype=np.int64)
    out = np.zeros(np.shape(codes), dtype=np.float64)
    for e in range(offsets.size - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            out[lo:hi] = pt_dequantize(codes[lo:hi], scales[e])
    return out


def pg_quantize_colwise(x_bf16_bits, offsets):
    """The transposed copy of the per-group quantization, for products that
    contract over the rows (the weight gradient over each expert's tokens, the
    data gradient over a weight's output rows).  [HP329] §3: with per-tensor
    or per-group FP32 scales the quantized data do not depend on the
    direction, only the operand layout does; the transposed copy therefore
    holds the same codes as ``pg_quantize``.  The layout follows the grouped
    column-wise MX copy: each group padded with zero rows to a multiple of 32.

    Returns (codesT uint8 [K, M_pad], scales float32 [E], padded offsets
    int64 [E+1])."""
    bits = np.asarray(x_bf16_bits, dtype=np.uint16)
    offsets = np.asarray(offsets, dtype=np.int64)
    codes, scales = pg_quantize(bits, offsets)
    counts = np.diff(offsets)
    poff = np.concatenate([[0], np.cumsum((counts + 31) // 32 * 32)]).astype(np.int64)
    out = np.zeros((bits.shape[1], int(poff[-1])), dtype=np.uint8)
    for e in range(offsets.size - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        out[:, int(poff[e]):int(poff[e]) + (hi - lo)] = codes[lo:hi].T
    return out, scales, poff
