"""Every call enqueues its kernels on the caller's stream and shares no device
state with other calls (workspaces are the caller's): two independent chains
launched alternately on two streams, each with its own inputs, give exactly
what each chain gives alone on the default stream.  The chains cover the
batched dual-axis quantizer, the variable-M and variable-K grouped GEMMs
(device-side tile and expert ordering), a dense GEMM on the 128-row tiles,
and per-tensor current scaling with the amax from the GEMM's epilogue."""

import numpy as np
import pytest
import torch

from block_quant_gemm_amd import mxq, workloads
from tests.gpu_helpers import say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

E, H, F = 8, 512, 256


def _inputs(seed, counts):
    offs = workloads.offsets_from_counts(np.array(counts, np.int64))
    M = int(offs[-1])
    bf = lambda shape, s, n: to_dev_bf16(workloads.bf16_normal(shape, s, seed=seed, name=n))
    return dict(offs=to_dev(offs), X=bf((M, H), 1.0, "sX"), dY=bf((M, F), 1e-3, "sdY"),
                W=bf((E * F, H), 0.02, "sW"), D=bf((1024, H), 1.0, "sD"),
                w_off=torch.arange(E + 1, dtype=torch.int64, device="cuda") * F)


def _chain(d):
    o = d["offs"]
    (xq, xs, xT, xTs, poff), (wq, ws, wT, wTs, _) = mxq.mx_quantize_dual_batch(
        [(d["X"], o), (d["W"], d["w_off"])])
    y = mxq.mx_grouped_gemm(xq, xs, wq.view(E, F, H), ws.view(E, F, H // 32), o)
    gq, gs, gT, gTs, _ = mxq.mx_quantize_dual(d["dY"], o)
    dx = mxq.mx_grouped_gemm(gq, gs, *mxq.expert_view(wT, wTs, E, F), o)
    dw = mxq.mx_grouped_gemm_wgrad(gT, gTs, xT, xTs, poff)
    dq, ds = mxq.mx_quantize_rowwise(d["D"])
    dd = mxq.mx_gemm(dq, ds, wq[:F], ws[:F])
    pa, sa = mxq.fp8_quantize_per_tensor(d["D"])
    pb, sb = mxq.fp8_quantize_per_tensor(d["W"][:F])
    c, am = mxq.fp8_gemm_per_tensor_amax(pa, sa, pb, sb)
    cq, cs = mxq.fp8_quantize_per_tensor_amax(c, am)
    return [y, dx, dw, dd, c, am, cq, cs]


def _bits(ts):
    return [t.clone().view(torch.uint8) if t.dtype != torch.uint8 else t.clone() for t in ts]


def test_two_streams_equal_each_alone():
    say("two independent chains on two streams vs each alone")
    d1 = _inputs(31, [300, 0, 41, 513, 129, 1, 256, 90])
    d2 = _inputs(32, [17, 600, 0, 0, 222, 64, 300, 5])
    ref1, ref2 = _bits(_chain(d1)), _bits(_chain(d2))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    for rep in range(3):
        with torch.cuda.stream(s1):
            out1 = _chain(d1)
        with torch.cuda.stream(s2):
            out2 = _chain(d2)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_bits(out1), ref1)):
            assert torch.equal(a, b), f"rep {rep}: chain 1 output {i} differs"
        for i, (a, b) in enumerate(zip(_bits(out2), ref2)):
            assert torch.equal(a, b), f"rep {rep}: chain 2 output {i} differs"
