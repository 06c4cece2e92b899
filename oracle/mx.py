"""MX block quantization oracle (E4M3 data, E8M0 shared scale per 32 values).
Test infrastructure.

[HP329] §3 table: MXFP8 stores E4M3 data with an E8M0 scale per 1x32 or 32x1
block, the scale taken from the current input's MX block; §3.1: row and col
quantization are distinct physical copies.  [TTNPU] "线性层低精度": block size
32, every 32 elements share one scale; "MoE 专家层低精度": the wgrad operands
go through a grouped MX quant.

Readings (the pages do not state them): the shared exponent of a block is
``floor(log2(amax)) - 8`` (8 = E4M3's largest exponent), clamped below at -127
and -127 for an all-zero block; the scale code is that exponent + 127; a block
with NaN or Inf gets scale 0xFF and all codes 0x7F; element codes are
``RNE_E4M3_sat(x * 2^-e)``.
"""

import numpy as np

from .codec import (E4M3_EMAX, E4M3_NAN_CODE, E8M0_BIAS, E8M0_NAN_CODE,
                    bf16_bits_to_f64, e4m3_decode, e4m3_encode, e8m0_decode)

BLOCK = 32


def block_shared_exponent(amax):
    """Shared exponent of MX blocks from their float64 amax (NaN/Inf allowed).

    Returns (exponent int64, nonfinite bool).  ``floor(log2(amax))`` is read
    exactly from ``frexp``: amax = f * 2^x with f in [0.5, 1) -> x - 1.
    """
    amax = np.asarray(amax, dtype=np.float64)
    nonfinite = ~np.isfinite(amax)
    pos = (amax > 0) & ~nonfinite
    _, fx = np.frexp(np.where(pos, amax, 1.0))
    e = fx.astype(np.int64) - 1 - E4M3_EMAX
    e = np.where(pos, np.maximum(e, -E8M0_BIAS), -E8M0_BIAS)
    return e, nonfinite


def quantize_blocks(vals):
    """Quantize float64 values shaped [..., nblocks, 32] block by block.

    Returns (codes uint8 [..., nblocks, 32], scales uint8 [..., nblocks]).
    """
    vals = np.asarray(vals, dtype=np.float64)
    assert vals.shape[-1] == BLOCK
    amax = np.max(np.abs(vals), axis=-1)          # NaN propagates
    e, nonfinite = block_shared_exponent(amax)
    scaled = np.ldexp(vals, -e[..., None])        # exact: power-of-two scaling
    codes = e4m3_encode(scaled)
    codes = np.where(nonfinite[..., None], np.uint8(E4M3_NAN_CODE), codes)
    scales = np.where(nonfinite, E8M0_NAN_CODE, e + E8M0_BIAS).astype(np.uint8)
    return codes.astype(np.uint8), scales


def mx_quantize_rowwise(x_bf16_bits):
    """Row-wise (1x32) MX quantization of a BF16 matrix [M, K], K % 32 == 0.

    Blocks run along the contiguous dimension K.  Returns
    (codes uint8 [M, K], scales uint8 [M, K/32]).
    """
    x = bf16_bits_to_f64(x_bf16_bits)
    M, K = x.shape
    assert K % BLOCK == 0, "K must be a multiple of 32"
    codes, scales = quantize_blocks(x.reshape(M, K // BLOCK, BLOCK))
    return codes.reshape(M, K), scales


def mx_quantize_colwise(x_bf16_bits):
    """Column-wise (32x1) MX quantization of a BF16 matrix [M, K], M % 32 == 0.

    Blocks run down dimension M.  The result is stored transposed so that the
    blocks are contiguous: codes [K, M], scales [K, M/32].  By definition this
    is the row-wise quantization of the transpose.
    """
    xt = np.ascontiguousarray(np.asarray(x_bf16_bits, dtype=np.uint16).T)
    assert xt.shape[1] % BLOCK == 0, "M must be a multiple of 32"
    return mx_quantize_rowwise(xt)


def padded_offsets(offsets):
    """Per-group offsets after padding every group to a multiple of 32 rows."""
    offsets = np.asarray(offsets, dtype=np.int64)
    counts = np.diff(offsets)
    padded = (counts + BLOCK - 1) // BLOCK * BLOCK
    return np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)


def mx_quantize_grouped_colwise(x_bf16_bits, offsets):
    """Grouped column-wise MX quantization for the wgrad operands.

    Rows [offsets[g], offsets[g+1]) form group g.  Each group is padded with
    zero rows to a multiple of 32 and column-quantized on its own, so no
    32-row block spans two groups.  Returns (codesT uint8 [K, M_pad],
    scalesT uint8 [K, M_pad/32], padded offsets int64 [G+1]).
    """
    x = bf16_bits_to_f64(np.asarray(x_bf16_bits, dtype=np.uint16))
    return mx_quantize_grouped_colwise_values(x, offsets)


def mx_quantize_grouped_colwise_values(x, offsets):
    """mx_quantize_grouped_colwise of a float64 matrix [M, K] (any real
    values, not only BF16 ones): the same padding and blocking."""
    x = np.asarray(x, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    K = x.shape[1]
    poff = padded_offsets(offsets)
    M_pad = int(poff[-1])
    codes = np.zeros((K, M_pad), np.uint8)
    scales = np.zeros((K, M_pad // BLOCK), np.uint8)
    for g in range(len(offsets) - 1):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        plo, phi = int(poff[g]), int(poff[g + 1])
        if phi == plo:
            continue
        block = np.zeros((phi - plo, K))              # +0.0 padding rows
        block[: hi - lo] = x[lo:hi]
        c, s = quantize_blocks(block.T.reshape(K, (phi - plo) // BLOCK, BLOCK))
        codes[:, plo:phi] = c.reshape(K, phi - plo)
        scales[:, plo // BLOCK: phi // BLOCK] = s
    return codes, scales, poff


def mx_dequantize(codes, scales):
    """Exact float64 values of an MX operand: codes [R, C], scales [R, C/32]."""
    codes = np.asarray(codes)
    R, C = codes.shape
    v = e4m3_decode(codes).reshape(R, C // BLOCK, BLOCK)
    s = e8m0_decode(scales)[..., None]
    return (v * s).reshape(R, C)
