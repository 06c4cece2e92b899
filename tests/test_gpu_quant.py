"""Bit-exact parity of the HIP quantization kernels with the CPU oracle.

Runs through the C ABI (ctypes binding).  Codes and scales must be equal byte
for byte, padding included."""

import numpy as np
import pytest
import torch

from block_quant_gemm_amd import mxq, workloads
from oracle import codec, mx, per_tensor
from tests.gpu_helpers import host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def bf16(vals):
    t = torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


ANCHORS = [2.0 ** -133, 2.0 ** -126, 2.0 ** -119, 2.0 ** -60, 1.0 / 3, 1.0, 255.0,
           448.0, 3.0e4, 2.0 ** 100, 3.0e38]


@pytest.mark.parametrize("anchor", ANCHORS)
def test_rowwise_every_bf16_pattern(anchor):
    say(f"rowwise all patterns, anchor {anchor}")
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = np.zeros((65536, 32), np.uint16)
    x[:, 0] = bf16([anchor])[0]
    x[:, 1] = pats
    x[:, 2] = pats[::-1]
    q, s = mxq.mx_quantize_rowwise(to_dev_bf16(x))
    torch.cuda.synchronize()
    rc, rs = mx.mx_quantize_rowwise(x)
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(q), rc)


def test_rowwise_tiny_linear():
    d = workloads.tiny_linear(0)
    for name in ("A", "W"):
        q, s = mxq.mx_quantize_rowwise(to_dev_bf16(d[name]))
        rc, rs = mx.mx_quantize_rowwise(d[name])
        assert np.array_equal(host(q), rc) and np.array_equal(host(s), rs), name


def test_rowwise_dense_ffn_full_size():
    say("rowwise dense FFN X 8192x2048, W 10944x2048")
    d = workloads.dense_ffn(0)
    for name in ("X", "W"):
        q, s = mxq.mx_quantize_rowwise(to_dev_bf16(d[name]))
        rc, rs = mx.mx_quantize_rowwise(d[name])
        assert np.array_equal(host(s), rs), name
        assert np.array_equal(host(q), rc), name


@pytest.mark.parametrize("M,K", [(1, 32), (37, 96), (5, 544), (130, 1408)])
def test_rowwise_strided_ragged(M, K):
    say(f"rowwise strided M={M} K={K}")
    ldx = K + 24
    big = workloads.bf16_normal((M, ldx), 1.0, seed=M, name="rs", outlier_frac=0.02,
                                outlier_scale=80.0)
    xd = to_dev_bf16(big)[:, :K]
    ldq = (K + 16 + 15) // 16 * 16
    qbuf = torch.full((M, ldq), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((M, K // 32 + 3), 0xCD, dtype=torch.uint8, device="cuda")
    mxq.mx_quantize_rowwise(xd, qbuf[:, :K], sbuf[:, :K // 32])
    rc, rs = mx.mx_quantize_rowwise(np.ascontiguousarray(big[:, :K]))
    qh, sh = host(qbuf), host(sbuf)
    assert np.array_equal(qh[:, :K], rc) and np.array_equal(sh[:, :K // 32], rs)
    assert np.all(qh[:, K:] == 0xAB) and np.all(sh[:, K // 32:] == 0xCD)   # untouched


def test_rowwise_special_blocks():
    x = np.zeros((3, 96), np.uint16)
    x[0, 32:64] = bf16(np.linspace(-1, 1, 32))
    x[0, 40] = 0x7F80
    x[0, 64:96] = bf16(np.linspace(-3, 3, 32))
    x[0, 70] = 0xFFC1
    x[0, 5] = 0x8000
    x[1, :] = np.arange(96) + 1                      # BF16 subnormals only
    x[2, :32] = 0x0001
    x[2, 32:64] = bf16(np.full(32, 500.0))
    x[2, 64:96] = bf16(np.full(32, -448.0))
    q, s = mxq.mx_quantize_rowwise(to_dev_bf16(x))
    rc, rs = mx.mx_quantize_rowwise(x)
    assert np.array_equal(host(s), rs) and np.array_equal(host(q), rc)


def test_rowwise_empty_is_noop():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, s = mxq.mx_quantize_rowwise(x)
    assert q.shape == (0, 64) and s.shape == (0, 2)


def test_rowwise_batch_equals_single_calls():
    """One launch for several matrices: a Linear's input and weight (contiguous,
    one long row each), a strided view (row by row, segment groups that end
    mid-row), an empty item in between, and a matrix of one segment: every
    item bit-equal to its own mx_quantize_rowwise call and to the oracle."""
    say("rowwise batch: 4096x2048 input, 2048x2048 weight, strided 37x544, empty, 1x32")
    a = workloads.bf16_normal((4096, 2048), 1.0, seed=1, name="rb_a", outlier_frac=0.01,
                              outlier_scale=100.0)
    w = workloads.bf16_normal((2048, 2048), 0.02, seed=2, name="rb_w")
    big = workloads.bf16_normal((37, 544 + 40), 1.0, seed=3, name="rb_s")
    one = workloads.bf16_normal((1, 32), 1.0, seed=4, name="rb_o")
    xs = [to_dev_bf16(a), to_dev_bf16(w), to_dev_bf16(big)[:, :544],
          torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), to_dev_bf16(one)]
    hosts = [a, w, np.ascontiguousarray(big[:, :544]), None, one]
    outs = mxq.mx_quantize_rowwise_batch(xs[:4])
    outs += mxq.mx_quantize_rowwise_batch(xs[4:])
    assert outs[3][0].shape == (0, 64)
    for i, (x, xh, (q, s)) in enumerate(zip(xs, hosts, outs)):
        if xh is None:
            continue
        q1, s1 = mxq.mx_quantize_rowwise(x)
        assert torch.equal(q, q1) and torch.equal(s, s1), f"item {i} differs from its own call"
        rc, rs = mx.mx_quantize_rowwise(xh)
        assert np.array_equal(host(q), rc) and np.array_equal(host(s), rs), f"item {i} vs oracle"


# ---------------------------------------------------------------------------
# column-wise
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K", [(32, 16), (256, 96), (160, 1408), (96, 2064)])
def test_colwise_plain(M, K):
    say(f"colwise M={M} K={K}")
    x = workloads.bf16_normal((M, K), 1.0, seed=K, name="cw", outlier_frac=0.01,
                              outlier_scale=100.0)
    qT, sT, _ = mxq.mx_quantize_colwise(to_dev_bf16(x))
    rc, rs = mx.mx_quantize_colwise(x)
    qh, sh = host(qT), host(sT)
    assert np.array_equal(qh[:, :M], rc) and np.array_equal(sh[:, :M // 32], rs)
    assert np.all(qh[:, M:] == 0) and np.all(sh[:, M // 32:] == 0)


@pytest.mark.parametrize("counts", [
    [40, 0, 1, 32, 0, 70, 0],
    [0, 0, 0, 5],
    [300],
    [1] * 9 + [0] * 3 + [77],
])
def test_colwise_grouped(counts):
    say(f"colwise grouped counts={counts}")
    counts = np.array(counts, np.int64)
    offs = workloads.offsets_from_counts(counts)
    M, K = int(counts.sum()), 208
    x = workloads.bf16_normal((M, K), 1e-3, seed=int(M), name="cg", outlier_frac=0.01,
                              outlier_scale=30.0)
    qT, sT, poff = mxq.mx_quantize_colwise(to_dev_bf16(x), to_dev(offs))
    rc, rs, rpoff = mx.mx_quantize_grouped_colwise(x, offs)
    Mp = int(rpoff[-1])
    assert np.array_equal(host(poff), rpoff)
    qh, sh = host(qT), host(sT)
    assert np.array_equal(qh[:, :Mp], rc) and np.array_equal(sh[:, :Mp // 32], rs)
    assert np.all(qh[:, Mp:] == 0) and np.all(sh[:, Mp // 32:] == 0)


def test_colwise_grouped_moe_backward_sampled_columns():
    """Full-size grouped column quant of dY [49152, 2048] with Zipf expert
    counts; the oracle checks 48 sampled columns (columns are independent)."""
    say("colwise grouped dY 49152x2048")
    counts = workloads.moe_counts(0)
    offs = workloads.offsets_from_counts(counts)
    dY = workloads.moe_backward(0)["dY"]
    qT, sT, poff = mxq.mx_quantize_colwise(to_dev_bf16(dY), to_dev(offs))
    cols = np.random.default_rng(0).choice(dY.shape[1], 48, replace=False)
    rc, rs, rpoff = mx.mx_quantize_grouped_colwise(np.ascontiguousarray(dY[:, cols]), offs)
    Mp = int(rpoff[-1])
    assert np.array_equal(host(poff), rpoff)
    qh = host(qT[torch.from_numpy(cols).cuda()])
    sh = host(sT[torch.from_numpy(cols).cuda()])
    assert np.array_equal(qh[:, :Mp], rc) and np.array_equal(sh[:, :Mp // 32], rs)


def test_colwise_matches_rowwise_of_transpose_on_gpu():
    x = workloads.bf16_normal((128, 192), 1.0, seed=3, name="ct")
    qT, sT, _ = mxq.mx_quantize_colwise(to_dev_bf16(x))
    q2, s2 = mxq.mx_quantize_rowwise(to_dev_bf16(np.ascontiguousarray(x.T)))
    assert torch.equal(qT[:, :128], q2) and torch.equal(sT[:, :4], s2)


# ---------------------------------------------------------------------------
# dual-axis (row and column copies from one read)
# ---------------------------------------------------------------------------

def _check_dual(x, out, offs=None):
    """Compare mx_quantize_dual's five outputs with the oracle's row-wise and
    (grouped) column-wise quantization of the same BF16 matrix."""
    q, s, qT, sT, poff = out
    M, K = x.shape
    rc, rs = mx.mx_quantize_rowwise(x)
    assert np.array_equal(host(s), rs), "row scales"
    assert np.array_equal(host(q), rc), "row codes"
    if offs is None:
        # one group of all rows: padded with zero rows to a multiple of 32
        cc, cs, rpoff = mx.mx_quantize_grouped_colwise(x, np.array([0, M], np.int64))
    else:
        cc, cs, rpoff = mx.mx_quantize_grouped_colwise(x, offs)
        assert np.array_equal(host(poff), rpoff)
    Mp = int(rpoff[-1])
    qh, sh = host(qT), host(sT)
    assert np.array_equal(qh[:, :cc.shape[1]], cc) and np.array_equal(sh[:, :cs.shape[1]], cs)
    assert np.all(qh[:, Mp:] == 0) and np.all(sh[:, Mp // 32:] == 0), "padding"


@pytest.mark.parametrize("M,K", [(32, 32), (256, 96), (160, 1408), (97, 2080), (1, 64)])
def test_dual_plain(M, K):
    say(f"dual M={M} K={K}")
    x = workloads.bf16_normal((M, K), 1.0, seed=K + M, name="dp", outlier_frac=0.01,
                              outlier_scale=100.0)
    _check_dual(x, mxq.mx_quantize_dual(to_dev_bf16(x)))


@pytest.mark.parametrize("counts", [
    [40, 0, 1, 32, 0, 70, 0],
    [0, 0, 0, 5],
    [300],
    [1] * 9 + [0] * 3 + [77],
])
def test_dual_grouped(counts):
    say(f"dual grouped counts={counts}")
    counts = np.array(counts, np.int64)
    offs = workloads.offsets_from_counts(counts)
    M, K = int(counts.sum()), 224
    x = workloads.bf16_normal((M, K), 1e-3, seed=int(M) + 1, name="dg", outlier_frac=0.01,
                              outlier_scale=30.0)
    _check_dual(x, mxq.mx_quantize_dual(to_dev_bf16(x), to_dev(offs)), offs)


def test_dual_special_blocks():
    """NaN, Inf, zero and subnormal blocks along both axes."""
    x = workloads.bf16_normal((64, 96), 1.0, seed=5, name="ds")
    x[3, 40] = 0x7F80           # +Inf: row block 1 of row 3, column block 0 of column 40
    x[40, 7] = 0x7FC1           # NaN
    x[32:64, 64:96] = 0         # an all-zero 32 x 32 corner
    x[0:32, 64] = 0x0001        # BF16 subnormals down one column
    _check_dual(x, mxq.mx_quantize_dual(to_dev_bf16(x)))


def test_dual_strided_untouched():
    M, K = 70, 160
    ldx = K + 40
    big = workloads.bf16_normal((M, ldx), 1.0, seed=11, name="dsu", outlier_frac=0.02,
                                outlier_scale=50.0)
    xd = to_dev_bf16(big)[:, :K]
    qbuf = torch.full((M, K + 32), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((M, K // 32 + 3), 0xCD, dtype=torch.uint8, device="cuda")
    out = mxq.mx_quantize_dual(xd, q=qbuf[:, :K], scale=sbuf[:, :K // 32])
    x = np.ascontiguousarray(big[:, :K])
    _check_dual(x, out)
    assert np.all(host(qbuf)[:, K:] == 0xAB) and np.all(host(sbuf)[:, K // 32:] == 0xCD)


def test_dual_empty_rows_pads_only():
    offs = np.array([0, 0, 0], np.int64)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, s, qT, sT, poff = mxq.mx_quantize_dual(x, to_dev(offs))
    assert q.shape == (0, 64) and np.array_equal(host(poff), offs)
    assert int(host(qT).max(initial=0)) == 0 and int(host(sT).max(initial=0)) == 0


def test_dual_matches_single_axis_calls_full_size():
    """dGU [49152, 2816] with the Zipf expert counts: every byte of the dual
    outputs equals the row-wise and grouped column-wise kernels' outputs, and
    the oracle checks 64 sampled rows and 32 sampled columns."""
    say("dual dGU 49152x2816 vs single-axis kernels and sampled oracle")
    counts = workloads.moe_counts(0)
    offs = workloads.offsets_from_counts(counts)
    dGU = workloads.moe_backward(0)["dGU"]
    xd, od = to_dev_bf16(dGU), to_dev(offs)
    q, s, qT, sT, poff = mxq.mx_quantize_dual(xd, od)
    q1, s1 = mxq.mx_quantize_rowwise(xd)
    qT1, sT1, poff1 = mxq.mx_quantize_colwise(xd, od)
    assert torch.equal(q, q1) and torch.equal(s, s1)
    assert torch.equal(qT, qT1) and torch.equal(sT, sT1) and torch.equal(poff, poff1)
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(dGU.shape[0], 64, replace=False))
    rc, rs = mx.mx_quantize_rowwise(np.ascontiguousarray(dGU[rows]))
    ri = torch.from_numpy(rows).cuda()
    assert np.array_equal(host(q[ri]), rc) and np.array_equal(host(s[ri]), rs)
    cols = rng.choice(dGU.shape[1], 32, replace=False)
    cc, cs, rpoff = mx.mx_quantize_grouped_colwise(np.ascontiguousarray(dGU[:, cols]), offs)
    ci = torch.from_numpy(cols).cuda()
    Mp = int(rpoff[-1])
    assert np.array_equal(host(qT[ci])[:, :Mp], cc) and np.array_equal(host(sT[ci])[:, :Mp // 32], cs)


def test_dual_batch_equals_single_calls():
    """One launch for several matrices with their own groups: an activation
    with empty and one-row experts, a weight stack with offsets e*N (N/32 odd,
    so each expert's column scales start mid-word), one group of all rows, an
    empty grouped item (only the column copy's zero padding) and K = 1408
    (a half-full last K chunk): every output of each item is bit-equal to its
    own mx_quantize_dual call, and the oracle checks the row and grouped column
    copies of every item."""
    say("dual batch: 300-row activation in 7 groups, 3x96-row weight stack, "
        "200x1408 one group, empty grouped; then 2 items")
    counts = np.array([40, 0, 1, 32, 0, 226, 1], np.int64)
    offs = workloads.offsets_from_counts(counts)
    a = workloads.bf16_normal((300, 224), 1.0, seed=21, name="db_a", outlier_frac=0.01,
                              outlier_scale=100.0)
    w = workloads.bf16_normal((3 * 96, 224), 0.02, seed=22, name="db_w")
    w_offs = np.arange(4, dtype=np.int64) * 96
    h = workloads.bf16_normal((200, 1408), 1.0, seed=23, name="db_h")
    e_offs = np.zeros(3, np.int64)
    items = [(to_dev_bf16(a), to_dev(offs)), (to_dev_bf16(w), to_dev(w_offs)),
             (to_dev_bf16(h), None),
             (torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), to_dev(e_offs))]
    outs = mxq.mx_quantize_dual_batch(items)
    outs += mxq.mx_quantize_dual_batch(items[1:3])
    hosts = [(a, offs), (w, w_offs), (h, None), (None, e_offs), (w, w_offs), (h, None)]
    for i, ((x, o), (xh, oh), out) in enumerate(zip(items + items[1:3], hosts, outs)):
        single = mxq.mx_quantize_dual(x, o)
        for j, (u, v) in enumerate(zip(out, single)):
            if u is None:
                assert v is None
            else:
                assert torch.equal(u, v), f"item {i} output {j} differs from its own call"
        q, sc, qT, sT, poff = out
        if xh is None:
            assert np.array_equal(host(poff), oh)
            assert int(host(qT).max(initial=0)) == 0 and int(host(sT).max(initial=0)) == 0
            continue
        rc, rs = mx.mx_quantize_rowwise(xh)
        assert np.array_equal(host(q), rc) and np.array_equal(host(sc), rs), f"item {i} row copy"
        go = oh if oh is not None else np.array([0, xh.shape[0]], np.int64)
        cc, cs, rpoff = mx.mx_quantize_grouped_colwise(xh, go)
        Mp = int(rpoff[-1])
        assert np.array_equal(host(qT)[:, :Mp], cc) and np.array_equal(host(sT)[:, :Mp // 32], cs), \
            f"item {i} column copy"
        if oh is not None:
            assert np.array_equal(host(poff), rpoff)


# ---------------------------------------------------------------------------
# per-tensor
# ---------------------------------------------------------------------------

def _pt_check(bits):
    q, s = mxq.fp8_quantize_per_tensor(to_dev_bf16(bits))
    rc, rsc = per_tensor.pt_quantize(bits)
    assert host(s)[0] == rsc
    assert np.array_equal(host(q), rc)


@pytest.mark.parametrize("amax", [448.0, 1.0, 3.0e-3, 7.7e5, 2.0 ** -100, 2.0 ** -125,
                                  1.0e-37, 3.0e38])
def test_per_tensor_all_patterns_below_amax(amax):
    """Every finite BF16 pattern with |x| <= amax, plus amax itself."""
    say(f"per-tensor all patterns amax={amax}")
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = codec.bf16_bits_to_f64(pats)
    a = codec.bf16_bits_to_f64(bf16([amax]))[0]
    keep = pats[np.isfinite(v) & (np.abs(v) <= a)]
    bits = np.concatenate([bf16([amax, -amax]), keep])
    _pt_check(bits)


def test_per_tensor_workloads_full_size():
    d = workloads.dense_ffn(0)
    for name in ("X", "W"):
        say(f"per-tensor dense FFN {name}")
        _pt_check(d[name])


@pytest.mark.parametrize("n", [1, 7, 9, 1023, 4099])
def test_per_tensor_tails(n):
    _pt_check(workloads.bf16_normal((n,), 0.5, seed=n, name="pt"))


def test_per_tensor_nonfinite_and_zero():
    _pt_check(np.array([0x3F80, 0x7FC0, 0xFF80, 0x7F80, 0xC000, 0xFFC0, 0x0001, 0x8000] * 3,
                       np.uint16))
    _pt_check(np.zeros(40, np.uint16))
    _pt_check(np.full(24, 0x8000, np.uint16))


def test_per_tensor_empty():
    x = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    q, s = mxq.fp8_quantize_per_tensor(x)
    assert host(s)[0] == 1.0
