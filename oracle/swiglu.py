"""SwiGLU of the routed experts' gate/up product and the MX quantization of
its output: what the fused gate/up producer computes.  Test infrastructure.

[HP329] §5.2: the routed experts hold a stacked gate_up weight [E, 2F, H]
and a down weight [E, H, F]; the grouped SwiGLU between them is part of the
expert computation (forward, dgrad and wgrad), and the down matmul consumes
its output in MX-FP8: row copy (1x32 blocks along F) for the forward,
grouped column copy (32x1 blocks along the expert's tokens, each expert
zero-padded to a multiple of 32) for the weight gradient (§3 table, [TTNPU]
"MoE 专家层低精度").  [HP329] §1 defers fused low-precision SwiGLU kernels
and [FPBLOG] §七.2 puts amax bookkeeping into the producing matmul's
epilogue; quantizing h there is that fusion.

Readings (the pages do not spell them out):
- Of each expert's 2F gate_up outputs the first F are the gate g and the
  last F the up projection u (the order of the stacked weight's rows).
- SwiGLU: h = silu(g) * u with silu(x) = x / (1 + exp(-x)).
- h is quantized from the matmul's accumulators directly: no BF16 rounding of
  g, u or h in between.  (The kernel's accumulators and its FP32 SwiGLU are
  not exact, so its codes are checked against intervals of h; the oracle
  here is exact in float64.)
"""

import numpy as np

from .mx import BLOCK, mx_quantize_grouped_colwise_values, quantize_blocks


def silu(x):
    """x * sigmoid(x) = x / (1 + exp(-x)) in float64.  exp(-x) overflows to
    +inf for x < -709, giving the correct limit -0.0."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu(g, u):
    """h = silu(g) * u, elementwise, float64."""
    return silu(g) * np.asarray(u, dtype=np.float64)


def split_gate_up(gu):
    """(g, u) from a gate_up output [M, 2F]: columns [0, F) and [F, 2F)."""
    gu = np.asarray(gu, dtype=np.float64)
    F = gu.shape[1] // 2
    return gu[:, :F], gu[:, F:]


def swiglu_mx(g, u, offsets):
    """MX copies of h = swiglu(g, u) for the down matmul.

    g, u: float64 [M, F] (F % 32 == 0); offsets: int64 [E+1] expert row
    ranges.  Returns (hq uint8 [M, F], hs uint8 [M, F/32], hqT uint8
    [F, M_pad], hsT uint8 [F, M_pad/32], padded offsets int64 [E+1]).
    """
    h = swiglu(g, u)
    M, F = h.shape
    assert F % BLOCK == 0, "F must be a multiple of 32"
    hq, hs = quantize_blocks(h.reshape(M, F // BLOCK, BLOCK))
    hqT, hsT, poff = mx_quantize_grouped_colwise_values(h, offsets)
    return hq.reshape(M, F), hs, hqT, hsT, poff
