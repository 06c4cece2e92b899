"""Parity of the fused gate/up product (grouped MX GEMM + SwiGLU + MX row and
grouped column copies of h from the epilogue) with the oracle, through the
C ABI.

The gate/up output (BF16) is checked as every grouped GEMM output is
(oracle.gemm tolerance plus the FP8 matrix unit's truncation allowance).
The codes of h come from FP32 accumulators and an FP32 SwiGLU, so they are
checked against intervals of h (tests/mx_interval.py): with g, u the exact
products and dg, du their allowances, the kernel's h lies within

    1.1 (|u| + du) dg + (|silu(g)| + 1.1 dg) du            (|silu'| <= 1.1)
  + (|g| + dg + 16) 2^-22 (|h| + ...)                       (FP32 exp, rcp, products)
  + 2^-126 (1 + |u| + du)                                   (FP32 underflow)
  + (|u| + du)(|g| + dg) e^(g + dg)  where g + dg < -80     (e^-g overflows to inf)

of the exact h.  Where the interval fixes the code it must equal the
oracle's (most elements); elsewhere it must be one of the codes the interval
allows."""

import numpy as np
import pytest
import torch

from block_quant_gemm_amd import mxq, workloads
from oracle import gemm, mx
from oracle import swiglu as sw
from tests import fp8_mode as f8
from tests.gpu_helpers import host, say, to_dev, to_dev_bf16
from tests.mx_interval import mx_valid
from tests.test_gpu_gemm import _relayout_scales

pytestmark = pytest.mark.gpu

SENTINEL = 0xAB


def h_bounds(g, u, dg, du):
    """[lo, hi] around the exact h = silu(g) u for the kernel's h."""
    h = sw.swiglu(g, u)
    au, ag = np.abs(u) + du, np.abs(g) + dg
    d = 1.1 * au * dg + (np.abs(sw.silu(g)) + 1.1 * dg) * du
    d += (ag + 16.0) * 2.0 ** -22 * (np.abs(h) + d)
    d += 2.0 ** -126 * (1.0 + au)
    with np.errstate(over="ignore", under="ignore"):
        d += np.where(g + dg < -80.0, au * ag * np.exp(np.minimum(g + dg, 0.0)), 0.0)
    return h - d, h + d


def _operands(counts, F, K, seed, w_sigma=0.02):
    counts = np.array(counts, np.int64)
    offs = workloads.offsets_from_counts(counts)
    E, M = len(counts), int(counts.sum())
    x = workloads.bf16_normal((M, K), 1.0, seed=seed, name="sx")
    w = workloads.bf16_normal((E * 2 * F, K), w_sigma, seed=seed, name="sw")
    xq, xs = mx.mx_quantize_rowwise(x)
    wq, ws = mx.mx_quantize_rowwise(w)
    return offs, xq, xs, wq, ws


def _reference(offs, xq, xs, wq, ws, F):
    """Exact gate/up product Y [M, 2F], magnitude S and truncation allowance T."""
    E, M, K = len(offs) - 1, xq.shape[0], xq.shape[1]
    A, B = mx.mx_dequantize(xq, xs), mx.mx_dequantize(wq, ws)
    Y, S = gemm.grouped_gemm_ref(A, B.reshape(E, 2 * F, K), offs)
    rows = np.repeat(np.arange(M), 2 * F)
    expert = np.searchsorted(offs, np.arange(M), side="right") - 1
    cols = np.repeat(expert, 2 * F) * 2 * F + np.tile(np.arange(2 * F), M)
    T = f8.fp8_mfma_truncation_bound(xq, xs, wq, ws, rows, cols).reshape(M, 2 * F)
    return Y, S, T


def _scales(s, layout):
    """Device copy of scales [rows, nb]: 'pad16' row stride a multiple of 16
    (16-byte windows), 'odd' an odd stride (byte path), 'shift5' windows
    whose first block sits 5 bytes into a window."""
    if layout == "pad16":
        buf = mxq._scale_buffer(s.shape[0], s.shape[1], "cuda")
        buf.copy_(to_dev(s))
        return buf
    return _relayout_scales(to_dev(s), layout)


def _run(offs, xq, xs, wq, ws, F, layout="pad16", gu=True):
    E, M, K = len(offs) - 1, xq.shape[0], xq.shape[1]
    aq, bq = to_dev(xq), to_dev(wq)
    asc, bsc = _scales(xs, layout), _scales(ws, layout)
    cap = mxq.colwise_capacity(M, E)
    hq = torch.full((M, F), SENTINEL, dtype=torch.uint8, device="cuda")
    hqT = torch.full((F, cap), SENTINEL, dtype=torch.uint8, device="cuda")
    hsT = mxq._scale_buffer(F, cap // 32, "cuda")
    hsT.fill_(SENTINEL)
    out = mxq.mx_grouped_gemm_swiglu(aq, asc, bq.view(E, 2 * F, K),
                                     bsc.view(E, 2 * F, K // 32), to_dev(offs), gu=gu,
                                     M_cap=cap, hq=hq, hqT=hqT, hsT=hsT)
    return [None if t is None else host(t) for t in out]


def _check_h(offs, Y, S, T, F, hq, hs, hqT, hsT, poff):
    M = Y.shape[0]
    g, u = sw.split_gate_up(Y)
    dY = gemm.tolerance(S) + T
    lo, hi = h_bounds(g, u, dY[:, :F], dY[:, F:])
    # row copy
    ok_c, ok_s, uniq = mx_valid(hq, hs, lo, hi)
    say(f"  row copy: codes fixed by the bounds {uniq.mean():.5f}; "
        f"bad codes {(~ok_c).sum()}, bad scales {(~ok_s).sum()}")
    assert ok_s.all() and ok_c.all()
    # column copy on the padded layout (padding rows are exact zeros)
    np.testing.assert_array_equal(poff, mx.padded_offsets(offs))
    Mp = int(poff[-1])
    loT, hiT = np.zeros((F, Mp)), np.zeros((F, Mp))
    for e in range(len(offs) - 1):
        a, b, p = int(offs[e]), int(offs[e + 1]), int(poff[e])
        loT[:, p:p + b - a] = lo[a:b].T
        hiT[:, p:p + b - a] = hi[a:b].T
    ok_c, ok_s, uniq = mx_valid(hqT[:, :Mp], hsT[:, :Mp // 32], loT, hiT)
    say(f"  column copy: codes fixed by the bounds {uniq.mean():.5f}; "
        f"bad codes {(~ok_c).sum()}, bad scales {(~ok_s).sum()}")
    assert ok_s.all() and ok_c.all()
    # nothing past the padded columns
    assert (hqT[:, Mp:] == SENTINEL).all() and (hsT[:, Mp // 32:] == SENTINEL).all()
    return uniq


CASES = [
    ([300, 0, 1, 257, 31, 600], 320, 256),      # partial h tile, 1-row and 257-row groups
    ([5], 32, 64),
    ([128, 128, 0, 1, 127, 129], 128, 1408),
    ([40, 0, 2, 700], 96, 96),                  # odd k-step count
    ([0, 0, 513], 1408, 128),                   # the expert FFN width, 11 h tiles
]


@pytest.mark.parametrize("counts,F,K", CASES)
@pytest.mark.parametrize("layout", ["pad16", "odd", "shift5"])
def test_swiglu_product(counts, F, K, layout):
    say(f"SwiGLU product counts={counts} F={F} K={K} scales={layout}")
    offs, xq, xs, wq, ws = _operands(counts, F, K, seed=len(counts) * 31 + F + K)
    gu, hq, hs, hqT, hsT, poff = _run(offs, xq, xs, wq, ws, F, layout)
    Y, S, T = _reference(offs, xq, xs, wq, ws, F)
    ok = f8.check_bf16_extra(gu, Y, S, T)
    say(f"  gate/up BF16 within tolerance: {ok.mean():.6f}")
    assert ok.all()
    _check_h(offs, Y, S, T, F, hq, hs, hqT, hsT, poff)


def test_swiglu_product_without_gate_up_output():
    offs, xq, xs, wq, ws = _operands([77, 0, 300], 160, 192, seed=3)
    with_gu = _run(offs, xq, xs, wq, ws, 160, gu=True)
    without = _run(offs, xq, xs, wq, ws, 160, gu=False)
    assert without[0] is None
    for a, b in zip(with_gu[1:], without[1:]):
        np.testing.assert_array_equal(a, b)


def test_swiglu_product_large_gate_values():
    """Weights 100x larger: gate values reach |g| ~ 100, past where e^-g
    overflows in FP32 (g < -88) and where silu(g) = g in FP32 (g > 17)."""
    offs, xq, xs, wq, ws = _operands([200, 61], 96, 256, seed=4, w_sigma=2.0)
    gu, hq, hs, hqT, hsT, poff = _run(offs, xq, xs, wq, ws, 96)
    Y, S, T = _reference(offs, xq, xs, wq, ws, 96)
    g = Y[:, :96]
    say(f"  gate range [{g.min():.1f}, {g.max():.1f}]")
    assert g.min() < -88 and g.max() > 88
    assert f8.check_bf16_extra(gu, Y, S, T).all()
    _check_h(offs, Y, S, T, 96, hq, hs, hqT, hsT, poff)


def test_swiglu_product_no_rows():
    """M == 0: only the padded offsets (all zero) are written."""
    offs = np.zeros(4, np.int64)
    aq = torch.empty((0, 64), dtype=torch.uint8, device="cuda")
    asc = torch.empty((0, 2), dtype=torch.uint8, device="cuda")
    bq = torch.zeros((3, 64, 64), dtype=torch.uint8, device="cuda")
    bsc = torch.full((3, 64, 2), 127, dtype=torch.uint8, device="cuda")
    poff = torch.full((4,), -1, dtype=torch.int64, device="cuda")
    out = mxq.mx_grouped_gemm_swiglu(aq, asc, bq, bsc, to_dev(offs), offsets_padded=poff)
    torch.cuda.synchronize()
    assert host(out[5]).tolist() == [0, 0, 0, 0]


def _sampled_blocks_check(offs, xq, xs, wq, ws, F, hq, hs, hqT, hsT, poff, rng, n=48):
    """Row blocks (row, 32 h columns) and column blocks (h column, 32 padded
    rows) at random, each from its own dot products."""
    E, M = len(offs) - 1, xq.shape[0]
    A_rows = {}

    def arow(r):
        if r not in A_rows:
            A_rows[r] = mx.mx_dequantize(xq[r:r + 1], xs[r:r + 1])[0]
        return A_rows[r]

    def gu_vals(rows, hcols):
        e = np.searchsorted(offs, rows, side="right") - 1
        gr, ur = e * 2 * F + hcols, e * 2 * F + F + hcols
        A = np.stack([arow(int(r)) for r in rows])
        out = []
        for wr in (gr, ur):
            Bv = mx.mx_dequantize(wq[wr], ws[wr])
            idx = np.arange(len(rows))
            Y, S = gemm.gemm_ref_entries(A, Bv, idx, idx)
            T = f8.fp8_mfma_truncation_bound(xq[rows], xs[rows], wq[wr], ws[wr], idx, idx)
            out.append((Y, gemm.tolerance(S) + T))
        return out

    for _ in range(n):
        r = int(rng.integers(0, M))
        b = int(rng.integers(0, F // 32))
        hc = np.arange(32 * b, 32 * b + 32)
        (g, dg), (u, du) = gu_vals(np.full(32, r), hc)
        lo, hi = h_bounds(g, u, dg, du)
        ok_c, ok_s, _ = mx_valid(hq[r:r + 1, 32 * b:32 * b + 32], hs[r:r + 1, b:b + 1],
                                 lo[None], hi[None])
        assert ok_c.all() and ok_s.all(), (r, b)
    for _ in range(n):
        e = int(rng.integers(0, E))
        cnt = int(offs[e + 1] - offs[e])
        if cnt == 0:
            continue
        blk = int(rng.integers(0, (cnt + 31) // 32))
        k = int(rng.integers(0, F))
        rows = int(offs[e]) + 32 * blk + np.arange(32)
        valid = rows < offs[e + 1]
        lo, hi = np.zeros(32), np.zeros(32)
        if valid.any():
            (g, dg), (u, du) = gu_vals(rows[valid], np.full(valid.sum(), k))
            lo[valid], hi[valid] = h_bounds(g, u, dg, du)
        p = int(poff[e]) + 32 * blk
        ok_c, ok_s, _ = mx_valid(hqT[k:k + 1, p:p + 32], hsT[k:k + 1, p // 32:p // 32 + 1],
                                 lo[None], hi[None])
        assert ok_c.all() and ok_s.all(), (e, blk, k)


def test_swiglu_moe_gate_up_full_size_sampled():
    """The expert layer's gate/up forward at full size (49152 rows, 64 Zipf
    experts, F 1408, K 2048): sampled gate/up outputs, row blocks and column
    blocks against their dot products; padded offsets exact."""
    say("SwiGLU product 49152 x (2 x 1408) x 2048, 64 experts")
    d = workloads.moe_forward(0)
    offs, E, F, K = d["offsets"], 64, workloads.MOE_FFN, workloads.HIDDEN
    xq_d, xs_d = mxq.mx_quantize_rowwise(to_dev_bf16(d["X"]))
    wq_d, ws_d = mxq.mx_quantize_rowwise(to_dev_bf16(d["W_gu"].reshape(E * 2 * F, K)))
    gu, hq, hs, hqT, hsT, poff = mxq.mx_grouped_gemm_swiglu(
        xq_d, xs_d, wq_d.view(E, 2 * F, K), ws_d.view(E, 2 * F, K // 32), to_dev(offs))
    torch.cuda.synchronize()
    xq, xs, wq, ws = host(xq_d), host(xs_d), host(wq_d), host(ws_d)
    rng = np.random.default_rng(11)
    # the operand codes used below equal the oracle's on sampled rows
    for src, q, s, n in ((d["X"], xq, xs, 16), (d["W_gu"].reshape(E * 2 * F, K), wq, ws, 16)):
        rows = np.sort(rng.choice(src.shape[0], n, replace=False))
        rc, rs = mx.mx_quantize_rowwise(np.ascontiguousarray(src[rows]))
        assert np.array_equal(q[rows], rc) and np.array_equal(s[rows], rs)
    poff = host(poff)
    np.testing.assert_array_equal(poff, mx.padded_offsets(offs))
    hq, hs, hqT, hsT, guh = host(hq), host(hs), host(hqT), host(hsT), host(gu)
    # gate/up outputs
    M = xq.shape[0]
    r, n = rng.integers(0, M, 600), rng.integers(0, 2 * F, 600)
    e = np.searchsorted(offs, r, side="right") - 1
    idx = np.arange(600)
    A = mx.mx_dequantize(xq[r], xs[r])
    Bv = mx.mx_dequantize(wq[e * 2 * F + n], ws[e * 2 * F + n])
    Y, S = gemm.gemm_ref_entries(A, Bv, idx, idx)
    T = f8.fp8_mfma_truncation_bound(xq[r], xs[r], wq[e * 2 * F + n], ws[e * 2 * F + n],
                                       idx, idx)
    assert f8.check_bf16_extra(guh[r, n], Y, S, T).all()
    _sampled_blocks_check(offs, xq, xs, wq, ws, F, hq, hs, hqT, hsT, poff, rng)
