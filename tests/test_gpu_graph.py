"""The expert-layer step through the C ABI captured in a HIP graph: every
library call enqueues kernels on the caller's stream and nothing else (no
allocation, synchronization or memset inside), so the step can be captured
once and replayed.  Each replay, with eager work and synchronizations in
between, must reproduce the eager step's outputs bit for bit (the kernels are
deterministic), as must a graph holding the fused producer and the
per-expert-scaling calls with their workspace-using quantizers."""

import numpy as np
import pytest
import torch

from block_quant_gemm_amd import mxq, workloads
from tests.gpu_helpers import say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

E, H, F = 8, 512, 256


def _inputs():
    counts = np.array([300, 0, 41, 513, 129, 1, 256, 90], np.int64)
    offs = workloads.offsets_from_counts(counts)
    M = int(offs[-1])
    Mp = int(((counts + 31) // 32 * 32).sum())          # columns the column copies fill
    bf = lambda shape, s, n: to_dev_bf16(workloads.bf16_normal(shape, s, seed=3, name=n))
    return dict(offs=to_dev(offs), M=M, Mp=Mp,
                X=bf((M, H), 1.0, "gX"), h=bf((M, F), 1.0, "gh"),
                Wgu=bf((E * 2 * F, H), 0.02, "gWgu"), Wdn=bf((E * H, F), 0.02, "gWdn"),
                dY=bf((M, H), 1e-3, "gdY"), dGU=bf((M, 2 * F), 1e-3, "gdGU"),
                w_off_gu=torch.arange(E + 1, dtype=torch.int64, device="cuda") * (2 * F),
                w_off_dn=torch.arange(E + 1, dtype=torch.int64, device="cuda") * H)


def _mx_step(d, batched=False):
    o = d["offs"]
    if batched:     # each forward product's activation and weights in one launch
        (xq, xs, xT, xTs, poff), (wq, ws, guT, guTs, _) = mxq.mx_quantize_dual_batch(
            [(d["X"], o), (d["Wgu"], d["w_off_gu"])])
    else:
        xq, xs, xT, xTs, poff = mxq.mx_quantize_dual(d["X"], o)
        wq, ws, guT, guTs, _ = mxq.mx_quantize_dual(d["Wgu"], d["w_off_gu"])
    gu = mxq.mx_grouped_gemm(xq, xs, wq.view(E, 2 * F, H), ws.view(E, 2 * F, H // 32), o)
    if batched:
        (hq, hs, hT, hTs, _), (dq, dsc, dnT, dnTs, _) = mxq.mx_quantize_dual_batch(
            [(d["h"], o), (d["Wdn"], d["w_off_dn"])])
    else:
        hq, hs, hT, hTs, _ = mxq.mx_quantize_dual(d["h"], o)
        dq, dsc, dnT, dnTs, _ = mxq.mx_quantize_dual(d["Wdn"], d["w_off_dn"])
    y = mxq.mx_grouped_gemm(hq, hs, dq.view(E, H, F), dsc.view(E, H, F // 32), o)
    gq, gs, dyT, dyTs, _ = mxq.mx_quantize_dual(d["dY"], o)
    bq, bs = mxq.expert_view(dnT, dnTs, E, H)
    dh = mxq.mx_grouped_gemm(gq, gs, bq, bs, o)
    uq, us, duT, duTs, _ = mxq.mx_quantize_dual(d["dGU"], o)
    bq2, bs2 = mxq.expert_view(guT, guTs, E, 2 * F)
    dx = mxq.mx_grouped_gemm(uq, us, bq2, bs2, o)
    dwdn = mxq.mx_grouped_gemm_wgrad(dyT, dyTs, hT, hTs, poff)
    dwgu = mxq.mx_grouped_gemm_wgrad(duT, duTs, xT, xTs, poff)
    return [gu, y, dh, dx, dwdn, dwgu, xq, xT[:, :d["Mp"]]]


def _mx_step_batched(d):
    return _mx_step(d, batched=True)


def _fused_and_per_group(d):
    o = d["offs"]
    xq, xs = mxq.mx_quantize_rowwise(d["X"])
    wq, ws = mxq.mx_quantize_rowwise(d["Wgu"])
    gu, hq, hs, hqT, hsT, poff = mxq.mx_grouped_gemm_swiglu(
        xq, xs, wq.view(E, 2 * F, H), ws.view(E, 2 * F, H // 32), o)
    pxq, pxs = mxq.fp8_quantize_per_group(d["X"], o)
    pwq, pws = mxq.fp8_quantize_per_group(d["Wgu"], d["w_off_gu"])
    _, ph, pam = mxq.fp8_grouped_gemm_per_group_swiglu(pxq, pxs, pwq.view(E, 2 * F, H), pws, o)
    q1, s1 = mxq.fp8_quantize_per_group_amax(ph, o, pam)
    t1, ts1, _ = mxq.fp8_quantize_per_group_colwise_amax(ph, o, pam)
    dq, dT, ds, _ = mxq.fp8_quantize_per_group_dual(ph, o, amax=pam)
    Mp = d["Mp"]
    return [gu, hq, hs, hqT[:, :Mp], hsT[:, :Mp // 32], poff, ph, pam, q1, s1, t1[:, :Mp], ts1,
            dq, dT[:, :Mp], ds]


def _bits(ts):
    return [t.detach().clone().view(torch.uint8) if t.dtype != torch.uint8 else t.clone()
            for t in ts]


@pytest.mark.parametrize("step", [_mx_step, _mx_step_batched, _fused_and_per_group])
def test_step_graph_replays_equal_eager(step):
    say(f"graph capture of {step.__name__}")
    d = _inputs()
    eager = _bits(step(d))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                  # warm-up on the capture stream
        step(d)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step(d)
    for r in range(3):
        for t in outs:                          # poison the outputs between replays
            t.view(torch.uint8).fill_(0xA5)
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_bits(outs), eager)):
            assert torch.equal(a, b), f"replay {r}: output {i} differs"
        del junk
