"""DeepSeek-V3-style blockwise FP8 (E4M3) oracle: the comparison recipe.
Test infrastructure.

[FPBLOG] §七.3: activations carry one scale per 1x128 block (per token, per
128 channels) and weights one per 128x128 block; a block's outlier then only
affects its own block.  The GEMM multiplies each 128-wide slice of the
contraction by that slice's s_a * s_w before adding it to the FP32 sum
(promotion at the block boundary, which is also the scale boundary).

Readings (the passage names the block shapes and FP32 scales, not the scale
rule): each block is quantized by the current-scaling rule of
``per_tensor`` (scale = amax / 448 in FP32 if amax is finite and > 0, else
1.0; codes RNE_E4M3(fp32(x) / scale)), i.e. the block is a tensor of its own.
A weight's last block row may hold fewer than 128 rows (N % 128 != 0); K is a
multiple of 128.  The exact product is the float64 matmul of the dequantized
operands (codes times their block's scale): the promotion order changes only
rounding.
"""

import numpy as np

from .per_tensor import pt_quantize

BLOCK = 128


def bw_quantize_act(x_bf16_bits):
    """1x128 blocks of a BF16 [M, K] matrix (K % 128 == 0).
    Returns (codes uint8 [M, K], scales float32 [M, K/128])."""
    bits = np.asarray(x_bf16_bits, dtype=np.uint16)
    M, K = bits.shape
    assert K % BLOCK == 0, "K must be a multiple of 128"
    codes = np.zeros((M, K), np.uint8)
    scales = np.ones((M, K // BLOCK), np.float32)
    for m in range(M):
        for b in range(K // BLOCK):
            codes[m, BLOCK * b:BLOCK * b + BLOCK], scales[m, b] = \
                pt_quantize(bits[m, BLOCK * b:BLOCK * b + BLOCK])
    return codes, scales


def bw_quantize_weight(w_bf16_bits):
    """128x128 blocks of a BF16 [N, K] weight (K % 128 == 0; the last block
    row may be partial).  Returns (codes uint8 [N, K], scales float32
    [ceil(N/128), K/128])."""
    bits = np.asarray(w_bf16_bits, dtype=np.uint16)
    N, K = bits.shape
    assert K % BLOCK == 0, "K must be a multiple of 128"
    nb = (N + BLOCK - 1) // BLOCK
    codes = np.zeros((N, K), np.uint8)
    scales = np.ones((nb, K // BLOCK), np.float32)
    for r in range(nb):
        rows = slice(BLOCK * r, min(N, BLOCK * r + BLOCK))
        for b in range(K // BLOCK):
            cols = slice(BLOCK * b, BLOCK * b + BLOCK)
            codes[rows, cols], scales[r, b] = pt_quantize(bits[rows, cols])
    return codes, scales


def bw_dequantize_act(codes, scales):
    """Exact float64 values of 1x128-blocked codes."""
    from .codec import e4m3_decode
    v = e4m3_decode(codes)
    return v * np.repeat(np.asarray(scales, np.float64), BLOCK, axis=1)


def bw_dequantize_weight(codes, scales):
    """Exact float64 values of 128x128-blocked codes."""
    from .codec import e4m3_decode
    v = e4m3_decode(codes)
    N = v.shape[0]
    s = np.repeat(np.repeat(np.asarray(scales, np.float64), BLOCK, axis=0), BLOCK, axis=1)
    return v * s[:N]
