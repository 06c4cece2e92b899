"""The six products of the MoE routed-expert layer step at full size (49152
rows, 64 experts with Zipf(1.1) counts, hidden 2048, expert FFN 1408),
composed exactly as the benchmark composes them: every tensor's row and
(grouped) column copies from one dual-axis quantization, the dgrad products
reading the weights' column copies in place through per-expert strides
(gate/up: expert e's scales start at byte 88 e of each scale row, so odd
experts start 8 bytes into a 16-byte window; down: 44 e).

"DeepSeek-V3 16B FSDP2 MXFP8/HiF8 训练设计" §8 (forward row·row, dgrad row·col
of the weight, wgrad col·col along tokens) and §5.2 (routed experts).  Each
product is checked on sampled outputs (plus every expert's first and last
row) against the FP64 oracle, after the sampled operand rows / columns'
codes and scales are checked bit for bit against the oracle's quantization;
in the exact-product mode every sampled output must meet the contract's rule
|C - Y| <= 1e-5 * S + 1e-6."""

import numpy as np
import pytest
import torch

from block_quant_gemm_amd import mxq, workloads
from oracle import gemm, mx
from tests.fp8_mode import accept, fp8_mfma_truncation_bound
from tests.gpu_helpers import host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

E, H, F = 64, 2048, 1408
ACCS = [mxq.ACC_FP32, mxq.ACC_MFMA_FP8]


@pytest.fixture(scope="module")
def layer():
    say("expert layer: drawing inputs (49152 rows, 64 experts)")
    fw = workloads.moe_forward(0)
    bw = workloads.moe_backward(0)
    offs = fw["offsets"]
    offs_d = to_dev(offs)
    host_in = {"X": fw["X"], "h": fw["h"], "dY": bw["dY"], "dGU": bw["dGU"],
               "W_gu": fw["W_gu"].reshape(E * 2 * F, H), "W_dn": fw["W_dn"].reshape(E * H, F)}
    w_off = {"W_gu": np.arange(E + 1, dtype=np.int64) * 2 * F,
             "W_dn": np.arange(E + 1, dtype=np.int64) * H}
    q = {}
    for name, bits in host_in.items():
        o = offs if name not in w_off else w_off[name]
        q[name] = mxq.mx_quantize_dual(to_dev_bf16(bits), to_dev(o))
    torch.cuda.synchronize()
    say("expert layer: quantized")
    return {"offs": offs, "offs_d": offs_d, "in": host_in, "q": q, "w_off": w_off}


def _sample_rows(offs, n, seed):
    """n uniform rows plus every non-empty expert's first and last row."""
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, int(offs[-1]), n))
    for e in range(E):
        if offs[e + 1] > offs[e]:
            rows += [int(offs[e]), int(offs[e + 1]) - 1]
    return np.array(rows, np.int64)


def _check_row_codes(qd, bits, rows):
    """Row copy of the dual quantization, sampled rows vs the oracle."""
    q, s = qd[0], qd[1]
    gq, gs = host(q[to_dev(rows)]), host(s[to_dev(rows)])
    rq, rs = mx.mx_quantize_rowwise(bits[rows])
    assert np.array_equal(gq, rq) and np.array_equal(gs, rs), "row copy codes differ"
    return gq, gs


def _col_codes(qd, bits, offs, cols, groups):
    """Grouped column copy: for each (column c, group g) pair the codes of
    x[o_g:o_{g+1}, c] padded to 32, from the library and from the oracle."""
    qT, sT, poff = qd[2], qd[3], host(qd[4])
    assert np.array_equal(poff, mx.padded_offsets(offs)), "padded offsets differ"
    L = int(max(poff[g + 1] - poff[g] for g in set(groups.tolist())))
    out_q, out_s, ref_q, ref_s, lens = [], [], [], [], []
    qTh_rows = host(qT[to_dev(cols)])
    sTh_rows = host(sT[to_dev(cols)])
    for i, (c, g) in enumerate(zip(cols, groups)):
        lo, hi, plo, phi = int(offs[g]), int(offs[g + 1]), int(poff[g]), int(poff[g + 1])
        col = np.zeros((1, phi - plo), np.uint16)
        col[0, :hi - lo] = bits[lo:hi, c]
        rq, rs = mx.mx_quantize_rowwise(col) if phi > plo else (np.zeros((1, 0), np.uint8),
                                                                 np.zeros((1, 0), np.uint8))
        gq = qTh_rows[i, plo:phi][None]
        gs = sTh_rows[i, plo // 32:phi // 32][None]
        assert np.array_equal(gq, rq) and np.array_equal(gs, rs), "column copy codes differ"
        pad = L - (phi - plo)
        out_q.append(np.pad(gq[0], (0, pad)))
        out_s.append(np.pad(gs[0], (0, pad // 32)))
        lens.append(phi - plo)
    return np.array(out_q), np.array(out_s)


def _var_m(layer, a_name, w_name, N, K, dgrad, accum, seed):
    L, offs = layer, layer["offs"]
    qa, qw = L["q"][a_name], L["q"][w_name]
    if dgrad:
        # B operand: expert e's weight transposed, read in place from the
        # weight's grouped column copy ([in, E*out]), out = K here.
        bq, bs = mxq.expert_view(qw[2], qw[3], E, K)            # [E, N, K]
    else:
        bq, bs = qw[0].view(E, N, K), qw[1].view(E, N, K // 32)
    c = mxq.mx_grouped_gemm(qa[0], qa[1], bq, bs, L["offs_d"], out_dtype=mxq.OUT_BF16,
                            accum=accum)
    rows = _sample_rows(offs, 1500, seed)
    rng = np.random.default_rng(seed + 1)
    n = rng.integers(0, N, len(rows))
    n[:2] = [0, N - 1]
    e = np.searchsorted(offs, rows, side="right") - 1
    ah, ash = _check_row_codes(qa, L["in"][a_name], rows)
    wbits = L["in"][w_name]
    if dgrad:
        # B row (e, n) is column n of W_e ([K, N] as stored [E*K, N]),
        # quantized along K within expert e's group of K rows
        bh, bsh = _col_codes(qw, wbits, L["w_off"][w_name], n, e)
    else:
        bh, bsh = _check_row_codes(qw, wbits, e * N + n)
    idx = np.arange(len(rows))
    Y, S = gemm.gemm_ref_entries(mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh), idx, idx)
    ch = host(c[to_dev(rows), to_dev(n)])
    accept(ch, Y, S, False, accum == mxq.ACC_FP32,
           lambda: fp8_mfma_truncation_bound(ah, ash, bh, bsh, idx, idx),
           f"{a_name}x{w_name}{'(col)' if dgrad else ''}")


@pytest.mark.parametrize("accum", ACCS)
def test_gate_up_forward(layer, accum):
    say(f"gate/up forward 49152x2816x2048 accum={accum}")
    _var_m(layer, "X", "W_gu", 2 * F, H, False, accum, 11)


@pytest.mark.parametrize("accum", ACCS)
def test_down_forward(layer, accum):
    say(f"down forward 49152x2048x1408 accum={accum}")
    _var_m(layer, "h", "W_dn", H, F, False, accum, 12)


@pytest.mark.parametrize("accum", ACCS)
def test_down_dgrad_on_column_copy(layer, accum):
    say(f"down dgrad 49152x1408x2048 on W_dn's column copy accum={accum}")
    _var_m(layer, "dY", "W_dn", F, H, True, accum, 13)


@pytest.mark.parametrize("accum", ACCS)
def test_gate_up_dgrad_on_column_copy(layer, accum):
    say(f"gate/up dgrad 49152x2048x2816 on W_gu's column copy accum={accum}")
    _var_m(layer, "dGU", "W_gu", H, 2 * F, True, accum, 14)


def _wgrad(layer, a_name, b_name, N, K, accum, seed):
    L, offs = layer, layer["offs"]
    qa, qb = L["q"][a_name], L["q"][b_name]
    c = mxq.mx_grouped_gemm_wgrad(qa[2], qa[3], qb[2], qb[3], qa[4], out_dtype=mxq.OUT_BF16,
                                  accum=accum)
    rng = np.random.default_rng(seed)
    e = np.repeat(np.arange(E), 20)
    n = rng.integers(0, N, len(e))
    k = rng.integers(0, K, len(e))
    n[:2], k[:2] = [0, N - 1], [K - 1, 0]
    ah, ash = _col_codes(qa, L["in"][a_name], offs, n, e)
    bh, bsh = _col_codes(qb, L["in"][b_name], offs, k, e)
    idx = np.arange(len(e))
    Y, S = gemm.gemm_ref_entries(mx.mx_dequantize(ah, ash), mx.mx_dequantize(bh, bsh), idx, idx)
    ch = host(c[to_dev(e), to_dev(n), to_dev(k)])
    accept(ch, Y, S, False, accum == mxq.ACC_FP32,
           lambda: fp8_mfma_truncation_bound(ah, ash, bh, bsh, idx, idx),
           f"d{b_name}-wgrad")


@pytest.mark.parametrize("accum", ACCS)
def test_down_wgrad(layer, accum):
    say(f"down wgrad dW_dn [64, 2048, 1408] over 49152 tokens accum={accum}")
    _wgrad(layer, "dY", "h", H, F, accum, 21)


@pytest.mark.parametrize("accum", ACCS)
def test_gate_up_wgrad(layer, accum):
    say(f"gate/up wgrad dW_gu [64, 2816, 2048] over 49152 tokens accum={accum}")
    _wgrad(layer, "dGU", "X", 2 * F, H, accum, 22)
