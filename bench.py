#!/usr/bin/env python3
"""Benchmark: one MoE routed-expert layer step (forward, dgrad and wgrad) of a
DeepSeek-V3 16B-shaped model with every operand MX-FP8 quantized on the fly,
on one MI355X.

Step (all on one HIP stream, inputs resident in HBM):
  forward   X·W_guᵀ (64 experts, grouped by rows) and h·W_dnᵀ
  dgrad     dY·W_dn and dGU·W_gu (weights column-quantized per expert)
  wgrad     dW_dn[e] = dY_eᵀ·h_e and dW_gu[e] = dGU_eᵀ·X_e over each expert's
            tokens (grouped column quantization, groups padded to 32)
  quantization of X, h, dY, dGU (row and grouped-column copies) and of W_gu,
  W_dn (row and column copies) every step, each tensor in one dual-axis pass
  (--separate-quant: one row-wise and one column-wise pass per tensor).
Synthetic inputs: 8192 tokens x top-6 = 49152 rows, expert counts drawn as a
multinomial over Zipf(1.1) expert probabilities (seed 0); BF16 N(0,1)
activations, N(0,0.02) weights, N(0,1e-3) gradients; h and dGU stand in for
the SwiGLU output and its backward.

Prints one JSON line: metric value = algorithmic GEMM FLOPs of the step
divided by the step time (quantization included).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MXFP8 grouped-GEMM TFLOP/s incl. quant (fwd+dgrad+wgrad); % MX-FP8 peak"
PEAK_MFMA_TFLOPS = 5000.0      # MI355X dense MX-FP8 (E4M3) matrix peak
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
MX_BYTES_PER_ELT = 2 + 1 + 1 / 32   # BF16 in, E4M3 code + E8M0 per 32 out
DUAL_BYTES_PER_ELT = 2 + 2 * (1 + 1 / 32)   # BF16 in once, row and column copies out
HIDDEN, FFN, E, TOKENS, TOP_K = 2048, 1408, 64, 8192, 6
COPY_CALIBRATION_BYTES = 1 << 30

# kernel-function names as rocprofv3 reports them
KFN = {
    "q_row": "k_mx_rowwise",
    "q_col": "k_mx_colwise<false>",
    "q_dual": "k_mx_colwise<true>",
    "gmm": "k_gemm<1,false,0,true,false>",
    "wgrad": "k_gemm<2,false,0,true,false>",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense FFN component")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the full block step (16384 tokens) component")
    ap.add_argument("--step-only", action="store_true",
                    help="only the expert-layer step (no dense, per-expert, fused or BF16 "
                         "components), e.g. for counter passes")
    ap.add_argument("--separate-quant", action="store_true",
                    help="quantize each tensor with separate row-wise and column-wise passes")
    ap.add_argument("--no-bf16-sweep", action="store_true",
                    help="skip the BF16 library GEMM comparison sweep")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a 1 GiB device-to-device copy (the known-size reference "
                         "that scales rocprofv3 FETCH_SIZE/WRITE_SIZE counts to bytes)")
    return ap.parse_args()


class HipEvent:
    """A HIP timing event created with hipEventDisableSystemFence: recording it
    skips the system-scope fence (a cache write-back and invalidation) that a
    default event performs, which the kernel after it would otherwise pay.
    Measured on the expert-layer step: events around the four variable-M
    launches add 19 us per step with torch's (default) events, 7 us with
    these.  Elapsed times are read after a device synchronization."""
    DISABLE_SYSTEM_FENCE = 0x20000000
    _hip = None

    def __init__(self, torch):
        import ctypes
        if HipEvent._hip is None:
            HipEvent._hip = ctypes.CDLL("libamdhip64.so")
        self.ctypes, self.torch = ctypes, torch
        self.e = ctypes.c_void_p()
        rc = HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.e),
                                                  ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)

    def record(self):
        stream = self.ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        if HipEvent._hip.hipEventRecord(self.e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        ms = self.ctypes.c_float()
        if HipEvent._hip.hipEventElapsedTime(self.ctypes.byref(ms), self.e, end.e) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if HipEvent._hip is not None and self.e:
            HipEvent._hip.hipEventDestroy(self.e)


class Timer:
    """Per-label HIP event pairs on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.ev = {}
        self.on = False
        self.only = None                         # record this label alone (None: all)

    def reset(self, only=None):
        self.ev = {}
        self.only = only

    def run(self, label, fn, *a, **k):
        if not self.on or (self.only is not None and label != self.only):
            return fn(*a, **k)
        s, e = HipEvent(self.torch), HipEvent(self.torch)
        s.record()
        r = fn(*a, **k)
        e.record()
        self.ev.setdefault(label, []).append((s, e))
        return r

    def ms(self):
        return {k: sum(s.elapsed_time(e) for s, e in v) / len(v) for k, v in self.ev.items()}

    def count(self):
        return {k: len(v) for k, v in self.ev.items()}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(collectives and sharding are out of scope); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from block_quant_gemm_amd import mxq, workloads

    mxq.load()                                   # fails loudly without the HIP library
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")

    def to_dev(bits):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return t.view(torch.bfloat16).to(dev)

    # ---------------- inputs ----------------
    fw = workloads.moe_forward(args.seed, TOKENS, TOP_K, E)
    bw = workloads.moe_backward(args.seed, TOKENS, TOP_K, E)
    counts, offs = fw["counts"], fw["offsets"]
    M = int(counts.sum())
    X, h = to_dev(fw["X"]), to_dev(fw["h"])
    Wgu = to_dev(fw["W_gu"].reshape(E * 2 * FFN, HIDDEN))
    Wdn = to_dev(fw["W_dn"].reshape(E * HIDDEN, FFN))
    dY, dGU = to_dev(bw["dY"]), to_dev(bw["dGU"])
    offs_d = torch.from_numpy(offs).to(dev)
    w_off_gu = torch.arange(E + 1, dtype=torch.int64, device=dev) * (2 * FFN)
    w_off_dn = torch.arange(E + 1, dtype=torch.int64, device=dev) * HIDDEN

    if args.copy_calibration:
        src = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    T = Timer(torch)

    def step_dual():
        # forward (each tensor's row and column copies come from one pass; a
        # product's activation and expert weights are quantized in one launch)
        (xq, xs, xT, xTs, poff), (wq, ws, guT, guTs, _) = T.run(
            "q_dual", mxq.mx_quantize_dual_batch, [(X, offs_d), (Wgu, w_off_gu)])
        gu = T.run("gmm", mxq.mx_grouped_gemm, xq, xs, wq.view(E, 2 * FFN, HIDDEN),
                   ws.view(E, 2 * FFN, HIDDEN // 32), offs_d)
        (hq, hs, hT, hTs, _), (dq, dsc, dnT, dnTs, _) = T.run(
            "q_dual", mxq.mx_quantize_dual_batch, [(h, offs_d), (Wdn, w_off_dn)])
        y = T.run("gmm", mxq.mx_grouped_gemm, hq, hs, dq.view(E, HIDDEN, FFN),
                  dsc.view(E, HIDDEN, FFN // 32), offs_d)
        # dgrad
        gq, gs, dyT, dyTs, _ = T.run("q_dual", mxq.mx_quantize_dual, dY, offs_d)
        bq, bs = mxq.expert_view(dnT, dnTs, E, HIDDEN)          # [E, 1408, 2048]
        dh = T.run("gmm", mxq.mx_grouped_gemm, gq, gs, bq, bs, offs_d)
        uq, us, duT, duTs, _ = T.run("q_dual", mxq.mx_quantize_dual, dGU, offs_d)
        bq2, bs2 = mxq.expert_view(guT, guTs, E, 2 * FFN)       # [E, 2048, 2816]
        dx = T.run("gmm", mxq.mx_grouped_gemm, uq, us, bq2, bs2, offs_d)
        # wgrad
        dwdn = T.run("wgrad", mxq.mx_grouped_gemm_wgrad, dyT, dyTs, hT, hTs, poff)
        dwgu = T.run("wgrad", mxq.mx_grouped_gemm_wgrad, duT, duTs, xT, xTs, poff)
        return gu, y, dh, dx, dwdn, dwgu

    def step_separate():
        # forward
        xq, xs = T.run("q_row", mxq.mx_quantize_rowwise, X)
        wq, ws = T.run("q_row", mxq.mx_quantize_rowwise, Wgu)
        gu = T.run("gmm", mxq.mx_grouped_gemm, xq, xs, wq.view(E, 2 * FFN, HIDDEN),
                   ws.view(E, 2 * FFN, HIDDEN // 32), offs_d)
        hq, hs = T.run("q_row", mxq.mx_quantize_rowwise, h)
        dq, dsc = T.run("q_row", mxq.mx_quantize_rowwise, Wdn)
        y = T.run("gmm", mxq.mx_grouped_gemm, hq, hs, dq.view(E, HIDDEN, FFN),
                  dsc.view(E, HIDDEN, FFN // 32), offs_d)
        # dgrad
        gq, gs = T.run("q_row", mxq.mx_quantize_rowwise, dY)
        dnT, dnTs, _ = T.run("q_col", mxq.mx_quantize_colwise, Wdn, w_off_dn)
        bq, bs = mxq.expert_view(dnT, dnTs, E, HIDDEN)          # [E, 1408, 2048]
        dh = T.run("gmm", mxq.mx_grouped_gemm, gq, gs, bq, bs, offs_d)
        uq, us = T.run("q_row", mxq.mx_quantize_rowwise, dGU)
        guT, guTs, _ = T.run("q_col", mxq.mx_quantize_colwise, Wgu, w_off_gu)
        bq2, bs2 = mxq.expert_view(guT, guTs, E, 2 * FFN)       # [E, 2048, 2816]
        dx = T.run("gmm", mxq.mx_grouped_gemm, uq, us, bq2, bs2, offs_d)
        # wgrad
        dyT, dyTs, poff = T.run("q_col", mxq.mx_quantize_colwise, dY, offs_d)
        hT, hTs, _ = T.run("q_col", mxq.mx_quantize_colwise, h, offs_d)
        dwdn = T.run("wgrad", mxq.mx_grouped_gemm_wgrad, dyT, dyTs, hT, hTs, poff)
        duT, duTs, _ = T.run("q_col", mxq.mx_quantize_colwise, dGU, offs_d)
        xT, xTs, _ = T.run("q_col", mxq.mx_quantize_colwise, X, offs_d)
        dwgu = T.run("wgrad", mxq.mx_grouped_gemm_wgrad, duT, duTs, xT, xTs, poff)
        return gu, y, dh, dx, dwdn, dwgu

    step = step_separate if args.separate_quant else step_dual
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Breakdown pass (K steps, not the timed region): HIP events around every
    # launch give each kernel class's share of the step.  Each recorded event
    # still costs the stream a little, so the timed region below records
    # events around the roofline kernel's launches only.
    T.on = True
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    T.on = False
    avg_ms = T.ms()
    n_launch = T.count()
    per_step_ms = {k: avg_ms[k] * n_launch[k] / args.steps for k in avg_ms}
    dom = max(per_step_ms, key=per_step_ms.get)

    T.reset(only=dom)
    T.on = True
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    T.on = False
    ms_step = (t1 - t0) * 1e3 / args.steps
    dom_ms = T.ms()[dom]                          # the roofline kernel, timed region

    # ---------------- algorithmic work ----------------
    per_dir = 2 * M * (2 * FFN * HIDDEN + HIDDEN * FFN)       # fwd (= dgrad = wgrad) FLOPs
    flops = 3 * per_dir
    value = flops / (ms_step * 1e-3) / 1e12
    quant_elts = {
        "q_row": [M * HIDDEN, E * 2 * FFN * HIDDEN, M * FFN, E * HIDDEN * FFN, M * HIDDEN,
                  M * 2 * FFN],
        "q_col": [E * HIDDEN * FFN, E * 2 * FFN * HIDDEN, M * HIDDEN, M * FFN, M * 2 * FFN,
                  M * HIDDEN],
        "q_dual": [M * HIDDEN, E * 2 * FFN * HIDDEN, M * FFN, E * HIDDEN * FFN, M * HIDDEN,
                   M * 2 * FFN],
    }
    quant_bpe = {"q_row": MX_BYTES_PER_ELT, "q_col": MX_BYTES_PER_ELT,
                 "q_dual": DUAL_BYTES_PER_ELT}
    qkeys = [k for k in ("q_row", "q_col", "q_dual") if k in avg_ms]
    gemm_flops = {
        "gmm": [2 * M * 2 * FFN * HIDDEN, 2 * M * HIDDEN * FFN, 2 * M * FFN * HIDDEN,
                2 * M * HIDDEN * 2 * FFN],
        "wgrad": [2 * M * HIDDEN * FFN, 2 * M * 2 * FFN * HIDDEN],
    }
    breakdown = {}
    for k in qkeys:
        work = sum(quant_elts[k]) * quant_bpe[k]
        breakdown[KFN[k]] = {
            "launches_per_step": n_launch[k] // args.steps, "ms_per_step": per_step_ms[k],
            "avg_launch_us": avg_ms[k] * 1e3,
            "GB_per_s": work / (per_step_ms[k] * 1e-3) / 1e9,
            "frac_hbm_peak": work / (per_step_ms[k] * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    for k in ("gmm", "wgrad"):
        work = sum(gemm_flops[k])
        breakdown[KFN[k]] = {
            "launches_per_step": n_launch[k] // args.steps, "ms_per_step": per_step_ms[k],
            "avg_launch_us": avg_ms[k] * 1e3,
            "TFLOP_per_s": work / (per_step_ms[k] * 1e-3) / 1e12,
            "frac_mfma_peak": work / (per_step_ms[k] * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS}
    gemm_ms = per_step_ms["gmm"] + per_step_ms["wgrad"]
    quant_ms = sum(per_step_ms[k] for k in qkeys)
    quant_bytes = sum(sum(quant_elts[k]) * quant_bpe[k] for k in qkeys)

    if dom in gemm_flops:
        per_launch = sum(gemm_flops[dom]) / len(gemm_flops[dom])
        achieved = per_launch / (dom_ms * 1e-3) / 1e12
        roof = {"kernel": KFN[dom], "avg_launch_us": dom_ms * 1e3, "bound": "mfma",
                "achieved": achieved,
                "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_MFMA_TFLOPS}
    else:
        per_launch = sum(quant_elts[dom]) * quant_bpe[dom] / len(quant_elts[dom])
        achieved = per_launch / (dom_ms * 1e-3) / 1e9
        roof = {"kernel": KFN[dom], "avg_launch_us": dom_ms * 1e3, "bound": "hbm",
                "achieved": achieved,
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS}
    roof["traffic"] = measured_traffic(roof["kernel"])

    components = {"moe_step": breakdown,
                  "gemm_only_TFLOP_per_s": flops / (gemm_ms * 1e-3) / 1e12,
                  "quant_only_GB_per_s": quant_bytes / (quant_ms * 1e-3) / 1e9,
                  "gemm_ms_per_step": gemm_ms, "quant_ms_per_step": quant_ms}
    if not args.step_only:
        components["step_distribution"] = step_distribution(torch, step, flops)
        components["step_as_hip_graph"] = graph_step(torch, step, flops, args.steps)
        components["weights_quantized_once"] = weights_once_step(
            torch, mxq, X, h, Wgu, Wdn, dY, dGU, offs_d, w_off_gu, w_off_dn, flops)
    if not args.no_dense and not args.step_only:
        components["dense_ffn"] = dense_component(torch, mxq, workloads, to_dev, args.seed)
    if not args.step_only:
        components["exact_accumulation"] = exact_mode(
            torch, mxq, workloads, to_dev, args.seed, X, h, Wgu, Wdn, dY, dGU, offs_d,
            w_off_gu, w_off_dn, flops, ms_step)
    if not args.step_only:
        components["per_expert_scaling_step"] = per_expert_step(
            torch, mxq, X, h, Wgu, Wdn, dY, dGU, offs_d, w_off_gu, w_off_dn, flops)
        components["fused_swiglu_producer"] = fused_producer(
            torch, mxq, X, Wgu, Wdn, dY, dGU, offs_d, w_off_gu, w_off_dn, flops)
    if not args.no_block and not args.step_only:
        components["full_block_step"] = full_block_step(torch, mxq, workloads, args.seed)
    if not args.no_bf16_sweep and not args.step_only:
        components["bf16_vs_mx_forward_sweep"] = bf16_sweep(torch, mxq)
        components["bf16_moe_step"] = bf16_moe_step(torch, X, h, Wgu, Wdn, dY, dGU, counts,
                                                    ms_step)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(fw, bw, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8_e4m3", "data": "synthetic",
        "config": {"workload": "moe_expert_layer_fwd_dgrad_wgrad", "tokens": TOKENS,
                   "top_k": TOP_K, "rows": M, "experts": E, "hidden": HIDDEN,
                   "moe_ffn": FFN, "expert_counts": "multinomial over Zipf(1.1), seed %d" % args.seed,
                   "max_expert_rows": int(counts.max()), "min_expert_rows": int(counts.min()),
                   "weights_quantized_each_step": True,
                   "quantization": "separate row and column passes" if args.separate_quant
                   else "dual-axis (one pass per tensor; each product's activation and "
                   "expert weights in one launch)",
                   "algorithmic_flops": flops},
        "pct_mx_fp8_peak": 100.0 * value / PEAK_MFMA_TFLOPS,
        "roofline": roof,
        "cpu_baseline": cpu,
        "components": components,
    }
    print(json.dumps(line), flush=True)


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        from block_quant_gemm_amd.build import source_digest
        if rec.get("source_digest") != source_digest():
            return None
        k = rec.get("kernels", {}).get(kernel)
        return None if k is None else k.get("hbm_bytes_per_launch")
    except Exception:
        return None


def dense_component(torch, mxq, workloads, to_dev, seed, reps=5):
    """Dense FFN gate/up projection: X 8192x2048 (0.5% outliers x50), W
    10944x2048: MX row quant of both and the forward GEMM; per-tensor E4M3
    quant of both and the per-tensor GEMM."""
    d = workloads.dense_ffn(seed)
    X, W = to_dev(d["X"]), to_dev(d["W"])
    nX, nW = X.numel(), W.numel()
    flops = 2 * X.shape[0] * W.shape[0] * X.shape[1]

    def timed(fn, *a):
        for _ in range(2):
            r = fn(*a)
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            r = fn(*a)
        e.record()
        torch.cuda.synchronize()
        return r, s.elapsed_time(e) / reps

    (xq, xs), t_qx = timed(mxq.mx_quantize_rowwise, X)
    (wq, ws), t_qw = timed(mxq.mx_quantize_rowwise, W)
    _, t_g = timed(mxq.mx_gemm, xq, xs, wq, ws)
    (px, sx), t_px = timed(mxq.fp8_quantize_per_tensor, X)
    (pw, sw), t_pw = timed(mxq.fp8_quantize_per_tensor, W)
    _, t_pg = timed(mxq.fp8_gemm_per_tensor, px, sx, pw, sw)
    # The product's output quantized per tensor for the next product: the
    # amax from a pass over C, or from the GEMM's epilogue (no amax pass).
    c_pt = mxq.fp8_gemm_per_tensor(px, sx, pw, sw)
    (cq, cs), t_cq2 = timed(mxq.fp8_quantize_per_tensor, c_pt)
    (_, c_amax), t_pga = timed(mxq.fp8_gemm_per_tensor_amax, px, sx, pw, sw)
    (cq1, cs1), t_cq1 = timed(mxq.fp8_quantize_per_tensor_amax, c_pt, c_amax)
    assert torch.equal(cq, cq1) and torch.equal(cs, cs1)   # same codes either way
    nC = c_pt.numel()
    del c_pt, cq, cs, cq1, cs1
    (bx, bsx), t_bx = timed(mxq.fp8_quantize_blockwise_act, X)
    (bwq, bsw), t_bw = timed(mxq.fp8_quantize_blockwise_weight, W)
    _, t_bg = timed(mxq.fp8_gemm_blockwise, bx, bsx, bwq, bsw)
    # the vendor library's per-tensor FP8 GEMM (hipBLASLt through torch) on the
    # same codes and scales: run-only context, and a cross-check of ours
    vendor = None
    try:
        f8 = torch.float8_e4m3fn
        vend = lambda: torch._scaled_mm(px.view(f8), pw.view(f8).t(), scale_a=sx.reshape(()),
                                        scale_b=sw.reshape(()), out_dtype=torch.bfloat16)
        cv, t_v = timed(vend)
        ours = mxq.fp8_gemm_per_tensor(px, sx, pw, sw)
        vendor = {"per_tensor_gemm_fwd_us": t_v * 1e3,
                  "TFLOP_per_s": flops / (t_v * 1e-3) / 1e12,
                  "max_abs_diff_vs_ours_over_max_abs": (
                      (cv.float() - ours.float()).abs().max() / cv.float().abs().max()).item()}
    except (RuntimeError, AttributeError) as ex:        # not built into this torch
        vendor = {"unavailable": str(ex).splitlines()[0][:200]}
    # Each format's whole path (both quantizations and the GEMM) from cold caches:
    # a 1 GiB write before every call evicts the 256 MB last-level cache, which
    # would otherwise hold these inputs (X 34 MB, W 45 MB) between calls.
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=X.device)

    def cold(path):
        ts = []
        for i in range(reps + 1):
            flush.fill_(i & 0xFF)
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            path()
            e.record()
            torch.cuda.synchronize()
            ts.append(s.elapsed_time(e))
        ts = sorted(ts[1:])
        return ts[len(ts) // 2]

    def mx_path():
        a, sa = mxq.mx_quantize_rowwise(X)
        b, sb = mxq.mx_quantize_rowwise(W)
        mxq.mx_gemm(a, sa, b, sb)

    def pt_path():
        a, sa = mxq.fp8_quantize_per_tensor(X)
        b, sb = mxq.fp8_quantize_per_tensor(W)
        mxq.fp8_gemm_per_tensor(a, sa, b, sb)

    def bw_path():
        a, sa = mxq.fp8_quantize_blockwise_act(X)
        b, sb = mxq.fp8_quantize_blockwise_weight(W)
        mxq.fp8_gemm_blockwise(a, sa, b, sb)

    cold_paths = {}
    for name, path in (("mx", mx_path), ("per_tensor", pt_path), ("blockwise", bw_path)):
        ms = cold(path)
        cold_paths[name] = {"us": ms * 1e3, "TFLOP_per_s_incl_quant": flops / (ms * 1e-3) / 1e12}
    del flush
    # output error of each format against the FP32 product of the BF16 inputs
    ref = X.float() @ W.float().t()
    rn = ref.norm().item()
    rel = lambda c: ((c.float() - ref).norm().item() / rn)
    errs = {"mx": rel(mxq.mx_gemm(xq, xs, wq, ws)),
            "per_tensor": rel(mxq.fp8_gemm_per_tensor(px, sx, pw, sw)),
            "blockwise": rel(mxq.fp8_gemm_blockwise(bx, bsx, bwq, bsw))}
    del ref
    gb = lambda n, b, ms: n * b / (ms * 1e-3) / 1e9
    return {
        "shape": "X 8192x2048, W 10944x2048",
        "mx_quant_X": {"us": t_qx * 1e3, "GB_per_s": gb(nX, MX_BYTES_PER_ELT, t_qx)},
        "mx_quant_W": {"us": t_qw * 1e3, "GB_per_s": gb(nW, MX_BYTES_PER_ELT, t_qw)},
        "mx_gemm_fwd": {"us": t_g * 1e3, "TFLOP_per_s": flops / (t_g * 1e-3) / 1e12},
        "per_tensor_quant_X": {"us": t_px * 1e3, "GB_per_s_algorithmic": gb(nX, 3, t_px)},
        "per_tensor_quant_W": {"us": t_pw * 1e3, "GB_per_s_algorithmic": gb(nW, 3, t_pw)},
        "per_tensor_gemm_fwd": {"us": t_pg * 1e3, "TFLOP_per_s": flops / (t_pg * 1e-3) / 1e12},
        "per_tensor_output_quant": {
            "note": "C 8192x10944 quantized per tensor for a next product: amax pass + encode, "
                    "or the amax from the GEMM's epilogue and the encode alone",
            "gemm_us": t_pg * 1e3, "gemm_with_epilogue_amax_us": t_pga * 1e3,
            "quant_two_pass_us": t_cq2 * 1e3, "quant_given_amax_us": t_cq1 * 1e3,
            "chain_two_pass_us": (t_pg + t_cq2) * 1e3,
            "chain_epilogue_amax_us": (t_pga + t_cq1) * 1e3,
            "quant_given_amax_GB_per_s": gb(nC, 3, t_cq1)},
        "blockwise_quant_X_1x128": {"us": t_bx * 1e3, "GB_per_s": gb(nX, 3 + 4 / 128, t_bx)},
        "blockwise_quant_W_128x128": {"us": t_bw * 1e3, "GB_per_s": gb(nW, 3, t_bw)},
        "blockwise_gemm_fwd": {"us": t_bg * 1e3, "TFLOP_per_s": flops / (t_bg * 1e-3) / 1e12},
        "cold_cache_path_median": cold_paths,
        "relative_output_error_vs_fp32_of_bf16_inputs": errs,
        "vendor_hipblaslt_per_tensor_fp8": vendor,
    }


def exact_mode(torch, mxq, workloads, to_dev, seed, X, h, Wgu, Wdn, dY, dGU, offs_d, w_off_gu,
               w_off_dn, flops, fp8_ms):
    """The exact-product accumulation (MXQ_ACC_FP32: E4M3 widened to BF16 with
    the block scale folded in, on the BF16 matrix instruction), which meets
    the contract's |C - Y| <= 1e-5 * S + 1e-6, against the FP8 matrix-unit
    mode: the expert-layer step and the dense FFN forward GEMM in both modes,
    and per configuration the fraction of FP8-mode outputs inside that
    tolerance of the exact-mode output (FP32 outputs; S = |A|·|B|ᵀ from the
    exact mode on the sign-cleared codes with the same scales).  The exact
    mode's own distance from the FP64 product is pinned by the parity tests
    (within the same rule), so this fraction stands in for the FP8 mode's
    fraction inside the rule."""
    ACC = mxq.ACC_FP32

    def step():
        (xq, xs, xT, xTs, poff), (wq, ws, guT, guTs, _) = mxq.mx_quantize_dual_batch(
            [(X, offs_d), (Wgu, w_off_gu)])
        mxq.mx_grouped_gemm(xq, xs, wq.view(E, 2 * FFN, HIDDEN),
                            ws.view(E, 2 * FFN, HIDDEN // 32), offs_d, accum=ACC)
        (hq, hs, hT, hTs, _), (dq, dsc, dnT, dnTs, _) = mxq.mx_quantize_dual_batch(
            [(h, offs_d), (Wdn, w_off_dn)])
        mxq.mx_grouped_gemm(hq, hs, dq.view(E, HIDDEN, FFN), dsc.view(E, HIDDEN, FFN // 32),
                            offs_d, accum=ACC)
        gq, gs, dyT, dyTs, _ = mxq.mx_quantize_dual(dY, offs_d)
        mxq.mx_grouped_gemm(gq, gs, *mxq.expert_view(dnT, dnTs, E, HIDDEN), offs_d, accum=ACC)
        uq, us, duT, duTs, _ = mxq.mx_quantize_dual(dGU, offs_d)
        mxq.mx_grouped_gemm(uq, us, *mxq.expert_view(guT, guTs, E, 2 * FFN), offs_d, accum=ACC)
        mxq.mx_grouped_gemm_wgrad(dyT, dyTs, hT, hTs, poff, accum=ACC)
        mxq.mx_grouped_gemm_wgrad(duT, duTs, xT, xTs, poff, accum=ACC)

    _, ms = _timed(torch, step, reps=5)
    out = {"step": {"ms_per_step": ms, "TFLOP_per_s_incl_quant": flops / (ms * 1e-3) / 1e12,
                    "fp8_mode_ms_per_step": fp8_ms}}

    mag = lambda q: q & 0x7F                          # |code|: the sign bit cleared

    def agree(call, a, sa, b, sb):
        c8 = call(a, sa, b, sb, mxq.ACC_MFMA_FP8)
        cx = call(a, sa, b, sb, ACC)
        sm = call(mag(a), sa, mag(b), sb, ACC)
        ok = (c8 - cx).abs() <= 1e-5 * sm + 1e-6
        fin = torch.isfinite(cx)
        r = (ok & fin).sum().item() / max(1, fin.sum().item())
        del c8, cx, sm, ok, fin
        return r

    fp32 = mxq.OUT_FP32
    dense = lambda a, sa, b, sb, acc: mxq.mx_gemm(a, sa, b, sb, out_dtype=fp32, accum=acc)
    grouped = lambda a, sa, b, sb, acc: mxq.mx_grouped_gemm(a, sa, b, sb, offs_d, out_dtype=fp32,
                                                            accum=acc)
    frac = {}
    t = workloads.tiny_linear(seed)
    frac["tiny_linear_256x256x512"] = agree(dense, *mxq.mx_quantize_rowwise(to_dev(t["A"])),
                                            *mxq.mx_quantize_rowwise(to_dev(t["W"])))
    d = workloads.dense_ffn(seed)
    xq, xs = mxq.mx_quantize_rowwise(to_dev(d["X"]))
    wq, ws = mxq.mx_quantize_rowwise(to_dev(d["W"]))
    frac["dense_ffn_8192x10944x2048"] = agree(dense, xq, xs, wq, ws)
    g8, tg8 = _timed(torch, lambda: mxq.mx_gemm(xq, xs, wq, ws))
    gx, tgx = _timed(torch, lambda: mxq.mx_gemm(xq, xs, wq, ws, accum=ACC))
    f2 = 2 * 8192 * 10944 * 2048
    out["dense_ffn_gemm"] = {"exact_us": tgx * 1e3, "exact_TFLOP_per_s": f2 / (tgx * 1e-3) / 1e12,
                             "fp8_us": tg8 * 1e3, "fp8_TFLOP_per_s": f2 / (tg8 * 1e-3) / 1e12}
    del xq, xs, wq, ws, g8, gx
    xq, xs, xT, xTs, poff = mxq.mx_quantize_dual(X, offs_d)
    wq, ws, guT, guTs, _ = mxq.mx_quantize_dual(Wgu, w_off_gu)
    hq, hs, hT, hTs, _ = mxq.mx_quantize_dual(h, offs_d)
    dq, dsc, dnT, dnTs, _ = mxq.mx_quantize_dual(Wdn, w_off_dn)
    gq, gs, dyT, dyTs, _ = mxq.mx_quantize_dual(dY, offs_d)
    uq, us, duT, duTs, _ = mxq.mx_quantize_dual(dGU, offs_d)
    frac["moe_gate_up_fwd"] = agree(grouped, xq, xs, wq.view(E, 2 * FFN, HIDDEN),
                                    ws.view(E, 2 * FFN, HIDDEN // 32))
    frac["moe_down_fwd"] = agree(grouped, hq, hs, dq.view(E, HIDDEN, FFN),
                                 dsc.view(E, HIDDEN, FFN // 32))
    frac["moe_down_dgrad"] = agree(grouped, gq, gs, *mxq.expert_view(dnT, dnTs, E, HIDDEN))
    frac["moe_gate_up_dgrad"] = agree(grouped, uq, us, *mxq.expert_view(guT, guTs, E, 2 * FFN))
    wg = lambda a, sa, b, sb, acc: mxq.mx_grouped_gemm_wgrad(a, sa, b, sb, poff, out_dtype=fp32,
                                                             accum=acc)
    frac["moe_down_wgrad"] = agree(wg, dyT, dyTs, hT, hTs)
    frac["moe_gate_up_wgrad"] = agree(wg, duT, duTs, xT, xTs)
    out["fp8_mode_fraction_inside_contract"] = frac
    return out


def per_expert_step(torch, mxq, X, h, Wgu, Wdn, dY, dGU, offs_d, w_off_gu, w_off_dn, flops,
                    steps=5):
    """The second format on the same expert-layer step: per-expert current
    scaling (one FP32 scale per expert group of rows and per expert weight),
    every tensor quantized row-major and transposed each step, the six
    products on the per-group-scaled grouped GEMMs."""
    def step():
        # every tensor's row-major and transposed copies from one encoding pass
        xq, xT, xs, poff = mxq.fp8_quantize_per_group_dual(X, offs_d)
        wq, guT, ws, _ = mxq.fp8_quantize_per_group_dual(Wgu, w_off_gu)
        mxq.fp8_grouped_gemm_per_group(xq, xs, wq.view(E, 2 * FFN, HIDDEN), ws, offs_d)
        hq, hT, hs, _ = mxq.fp8_quantize_per_group_dual(h, offs_d)
        dq, dnT, dsc, _ = mxq.fp8_quantize_per_group_dual(Wdn, w_off_dn)
        mxq.fp8_grouped_gemm_per_group(hq, hs, dq.view(E, HIDDEN, FFN), dsc, offs_d)
        gq, dyT, gs, _ = mxq.fp8_quantize_per_group_dual(dY, offs_d)
        mxq.fp8_grouped_gemm_per_group(
            gq, gs, dnT[:, :E * HIDDEN].view(FFN, E, HIDDEN).permute(1, 0, 2), dsc, offs_d)
        uq, duT, us, _ = mxq.fp8_quantize_per_group_dual(dGU, offs_d)
        mxq.fp8_grouped_gemm_per_group(
            uq, us, guT[:, :E * 2 * FFN].view(HIDDEN, E, 2 * FFN).permute(1, 0, 2), ws, offs_d)
        mxq.fp8_grouped_gemm_wgrad_per_group(dyT, gs, hT, hs, poff)
        mxq.fp8_grouped_gemm_wgrad_per_group(duT, us, xT, xs, poff)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        step()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    return {"ms_per_step": ms, "TFLOP_per_s_incl_quant": flops / (ms * 1e-3) / 1e12,
            "quantization": "per-expert FP32 scales, row-major and transposed copies from "
                            "one encoding pass per tensor (fp8_quantize_per_group_dual)"}


def graph_step(torch, step, flops, steps):
    """The same step captured once in a HIP graph (torch.cuda.CUDAGraph; the
    library only enqueues kernels on the current stream) and replayed: the
    host-side launch cost of its 12 launches leaves the step."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"ms_per_step": ms, "TFLOP_per_s_incl_quant": flops / (ms * 1e-3) / 1e12}


def _timed(torch, fn, *a, reps=5):
    """Average milliseconds per call of fn over reps calls (two untimed first)."""
    for _ in range(2):
        r = fn(*a)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        r = fn(*a)
    e.record()
    torch.cuda.synchronize()
    return r, s.elapsed_time(e) / reps


def fused_producer(torch, mxq, X, Wgu, Wdn, dY, dGU, offs_d, w_off_gu, w_off_dn, flops):
    """The gate/up product with SwiGLU and h's MX row and column copies in
    its epilogue, against the unfused chain (the product in BF16, SwiGLU,
    then the dual-axis quantizer on h); and the expert-layer step with the
    fused producer in place of the product and h's quantization (h is then
    the SwiGLU of the product instead of a separate input)."""
    xq, xs, xT, xTs, poff = mxq.mx_quantize_dual(X, offs_d)
    wq, ws, guT, guTs, _ = mxq.mx_quantize_dual(Wgu, w_off_gu)
    wv, wsv = wq.view(E, 2 * FFN, HIDDEN), ws.view(E, 2 * FFN, HIDDEN // 32)
    _, t_fused = _timed(torch, mxq.mx_grouped_gemm_swiglu, xq, xs, wv, wsv, offs_d)
    _, t_fused_nogu = _timed(torch, lambda: mxq.mx_grouped_gemm_swiglu(xq, xs, wv, wsv, offs_d,
                                                                       gu=False))
    gu, t_gemm = _timed(torch, mxq.mx_grouped_gemm, xq, xs, wv, wsv, offs_d)
    silu = torch.nn.functional.silu
    hb, t_swiglu = _timed(torch, lambda: silu(gu[:, :FFN]) * gu[:, FFN:])
    _, t_quant = _timed(torch, mxq.mx_quantize_dual, hb, offs_d)

    def step():
        gu, hq, hs, hT, hTs, poff_h = mxq.mx_grouped_gemm_swiglu(xq_s[0], xq_s[1], *wgu_s, offs_d)
        dq, dsc, dnT, dnTs, _ = mxq.mx_quantize_dual(Wdn, w_off_dn)
        mxq.mx_grouped_gemm(hq, hs, dq.view(E, HIDDEN, FFN), dsc.view(E, HIDDEN, FFN // 32),
                            offs_d)
        gq, gs, dyT, dyTs, _ = mxq.mx_quantize_dual(dY, offs_d)
        bq, bs = mxq.expert_view(dnT, dnTs, E, HIDDEN)
        mxq.mx_grouped_gemm(gq, gs, bq, bs, offs_d)
        uq, us, duT, duTs, _ = mxq.mx_quantize_dual(dGU, offs_d)
        bq2, bs2 = mxq.expert_view(wqT_s[0], wqT_s[1], E, 2 * FFN)
        mxq.mx_grouped_gemm(uq, us, bq2, bs2, offs_d)
        mxq.mx_grouped_gemm_wgrad(dyT, dyTs, hT, hTs, poff_h)
        mxq.mx_grouped_gemm_wgrad(duT, duTs, xq_s[2], xq_s[3], poff_h)

    def full_step():
        # the step's own quantization of X and W_gu, then the rest
        xo, q = mxq.mx_quantize_dual_batch([(X, offs_d), (Wgu, w_off_gu)])
        xq_s[:] = xo[:4]
        wgu_s[:] = [q[0].view(E, 2 * FFN, HIDDEN), q[1].view(E, 2 * FFN, HIDDEN // 32)]
        wqT_s[:] = [q[2], q[3]]
        step()

    xq_s, wgu_s, wqT_s = [None] * 4, [None] * 2, [None] * 2
    _, t_step = _timed(torch, full_step)

    # per-expert current scaling: h's group amaxes from the product's epilogue
    pxq, pxs = mxq.fp8_quantize_per_group(X, offs_d)
    pwq, pws = mxq.fp8_quantize_per_group(Wgu, w_off_gu)
    pwv = pwq.view(E, 2 * FFN, HIDDEN)
    (_, ph, pam), t_pg_fused = _timed(torch, mxq.fp8_grouped_gemm_per_group_swiglu, pxq, pxs,
                                      pwv, pws, offs_d)
    _, t_pg_qa = _timed(torch, mxq.fp8_quantize_per_group_amax, ph, offs_d, pam)
    _, t_pg_qta = _timed(torch, mxq.fp8_quantize_per_group_colwise_amax, ph, offs_d, pam)
    pgu, t_pg_gemm = _timed(torch, mxq.fp8_grouped_gemm_per_group, pxq, pxs, pwv, pws, offs_d)
    _, t_pg_q = _timed(torch, mxq.fp8_quantize_per_group, ph, offs_d)
    _, t_pg_qt = _timed(torch, mxq.fp8_quantize_per_group_colwise, ph, offs_d)
    def pg_step():
        # the per-expert-scaling step with the fused producer: h's group amaxes
        # come from the gate/up epilogue (h's dual quantization has no amax pass)
        xq, xT, xs, poff = mxq.fp8_quantize_per_group_dual(X, offs_d)
        wq, guT, ws, _ = mxq.fp8_quantize_per_group_dual(Wgu, w_off_gu)
        _, hb, ham = mxq.fp8_grouped_gemm_per_group_swiglu(xq, xs, wq.view(E, 2 * FFN, HIDDEN),
                                                          ws, offs_d)
        hq, hT, hs, _ = mxq.fp8_quantize_per_group_dual(hb, offs_d, amax=ham)
        dq, dnT, dsc, _ = mxq.fp8_quantize_per_group_dual(Wdn, w_off_dn)
        mxq.fp8_grouped_gemm_per_group(hq, hs, dq.view(E, HIDDEN, FFN), dsc, offs_d)
        gq, dyT, gs, _ = mxq.fp8_quantize_per_group_dual(dY, offs_d)
        mxq.fp8_grouped_gemm_per_group(
            gq, gs, dnT[:, :E * HIDDEN].view(FFN, E, HIDDEN).permute(1, 0, 2), dsc, offs_d)
        uq, duT, us, _ = mxq.fp8_quantize_per_group_dual(dGU, offs_d)
        mxq.fp8_grouped_gemm_per_group(
            uq, us, guT[:, :E * 2 * FFN].view(HIDDEN, E, 2 * FFN).permute(1, 0, 2), ws, offs_d)
        mxq.fp8_grouped_gemm_wgrad_per_group(dyT, gs, hT, hs, poff)
        mxq.fp8_grouped_gemm_wgrad_per_group(duT, us, xT, xs, poff)

    _, t_pg_step = _timed(torch, pg_step)
    pg = {
        "step_with_fused_producer": {
            "ms_per_step": t_pg_step, "TFLOP_per_s_incl_quant": flops / (t_pg_step * 1e-3) / 1e12},
        "fused_product_us": t_pg_fused * 1e3,
        "quant_h_with_amax_us": {"row": t_pg_qa * 1e3, "transposed": t_pg_qta * 1e3},
        "unfused": {"grouped_gemm_us": t_pg_gemm * 1e3,
                    "quant_h_us": {"row": t_pg_q * 1e3, "transposed": t_pg_qt * 1e3}},
        "producer_plus_quant_us": {
            "fused": (t_pg_fused + t_pg_qa + t_pg_qta) * 1e3,
            "unfused_without_swiglu": (t_pg_gemm + t_pg_q + t_pg_qt) * 1e3},
    }
    return {
        "fused_us": t_fused * 1e3,
        "fused_without_bf16_product_us": t_fused_nogu * 1e3,
        "unfused": {"grouped_gemm_us": t_gemm * 1e3, "torch_swiglu_bf16_us": t_swiglu * 1e3,
                    "dual_quant_h_us": t_quant * 1e3},
        "saving_vs_gemm_plus_quant_us": (t_gemm + t_quant - t_fused) * 1e3,
        "per_expert_scaling": pg,
        "step_with_fused_producer": {
            "ms_per_step": t_step, "TFLOP_per_s_incl_quant": flops / (t_step * 1e-3) / 1e12,
            "note": "h is the SwiGLU of the gate/up product; no separate h input or its "
                    "quantization"},
    }


def step_distribution(torch, step, flops, n=50):
    """Per-step times of the same step over n steps, each between HIP events
    on the launch stream (after the timed region, so the clocks are warm):
    median and 10th / 90th percentiles."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for s, e in ev:
        s.record()
        step()
        e.record()
    torch.cuda.synchronize()
    import numpy as np
    t = np.array([s.elapsed_time(e) for s, e in ev])
    med = float(np.median(t))
    return {"steps": n, "median_ms": med, "p10_ms": float(np.percentile(t, 10)),
            "p90_ms": float(np.percentile(t, 90)),
            "TFLOP_per_s_at_median": flops / (med * 1e-3) / 1e12}


def weights_once_step(torch, mxq, X, h, Wgu, Wdn, dY, dGU, offs_d, w_off_gu, w_off_dn, flops):
    """The expert-layer step with the weights' row and column copies made once
    (weights change once per optimizer step, so their quantization is shared
    by every micro-batch of it); activations and gradients still quantized in
    the step."""
    wq, ws, guT, guTs, _ = mxq.mx_quantize_dual(Wgu, w_off_gu)
    dq, dsc, dnT, dnTs, _ = mxq.mx_quantize_dual(Wdn, w_off_dn)
    bq, bs = mxq.expert_view(dnT, dnTs, E, HIDDEN)
    bq2, bs2 = mxq.expert_view(guT, guTs, E, 2 * FFN)

    def step():
        xq, xs, xT, xTs, poff = mxq.mx_quantize_dual(X, offs_d)
        mxq.mx_grouped_gemm(xq, xs, wq.view(E, 2 * FFN, HIDDEN),
                            ws.view(E, 2 * FFN, HIDDEN // 32), offs_d)
        hq, hs, hT, hTs, _ = mxq.mx_quantize_dual(h, offs_d)
        mxq.mx_grouped_gemm(hq, hs, dq.view(E, HIDDEN, FFN), dsc.view(E, HIDDEN, FFN // 32),
                            offs_d)
        gq, gs, dyT, dyTs, _ = mxq.mx_quantize_dual(dY, offs_d)
        mxq.mx_grouped_gemm(gq, gs, bq, bs, offs_d)
        uq, us, duT, duTs, _ = mxq.mx_quantize_dual(dGU, offs_d)
        mxq.mx_grouped_gemm(uq, us, bq2, bs2, offs_d)
        mxq.mx_grouped_gemm_wgrad(dyT, dyTs, hT, hTs, poff)
        mxq.mx_grouped_gemm_wgrad(duT, duTs, xT, xTs, poff)

    _, ms = _timed(torch, step, reps=10)
    return {"ms_per_step": ms, "TFLOP_per_s_incl_quant": flops / (ms * 1e-3) / 1e12,
            "note": "W_gu and W_dn dual-quantized once outside the step"}


def full_block_step(torch, mxq, workloads, seed):
    """One block at sequence 4096 x batch 4 (16384 tokens): the MLA projection
    and shared-expert Linears and the 64-expert routed products at 98304 rows,
    forward, dgrad and wgrad, every operand MX-quantized in both directions by
    the dual-axis quantizer in the step; and the same with the weights'
    copies made once.  Tensors are drawn on the device with torch's generator
    (N(0,1) activations, N(0,0.02) weights, N(0,1e-3) gradients); expert
    counts as for the expert layer, from 98304 rows."""
    dev = torch.device("cuda:0")
    T = workloads.BLOCK_TOKENS
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)

    def draw(shape, sigma):
        return (torch.randn(shape, device=dev, generator=gen) * sigma).to(torch.bfloat16)

    one = torch.tensor([0, T], dtype=torch.int64, device=dev)
    dense = []
    for name, fin, fout in workloads.BLOCK_DENSE_LINEARS:
        dense.append(dict(X=draw((T, fin), 1.0), W=draw((fout, fin), 0.02),
                          dY=draw((T, fout), 1e-3), fin=fin, fout=fout,
                          woff=torch.tensor([0, fout], dtype=torch.int64, device=dev)))
    counts = workloads.moe_counts(seed, T)
    M = int(counts.sum())
    offs_d = torch.from_numpy(workloads.offsets_from_counts(counts)).to(dev)
    rX, rh = draw((M, HIDDEN), 1.0), draw((M, FFN), 1.0)
    rdY, rdGU = draw((M, HIDDEN), 1e-3), draw((M, 2 * FFN), 1e-3)
    Wgu, Wdn = draw((E * 2 * FFN, HIDDEN), 0.02), draw((E * HIDDEN, FFN), 0.02)
    w_off_gu = torch.arange(E + 1, dtype=torch.int64, device=dev) * (2 * FFN)
    w_off_dn = torch.arange(E + 1, dtype=torch.int64, device=dev) * HIDDEN

    def quant_weights():
        qw = [mxq.mx_quantize_dual(d["W"], d["woff"]) for d in dense]
        return qw, mxq.mx_quantize_dual(Wgu, w_off_gu), mxq.mx_quantize_dual(Wdn, w_off_dn)

    def step(wts=None):
        # in the step, each product's input and weight are quantized in one launch
        qw, qgu, qdn = wts if wts is not None else (None, None, None)
        for i, d in enumerate(dense):
            fout = d["fout"]
            if qw is None:
                (xq, xs, xT, xTs, _), (wq, ws, wT, wTs, _) = mxq.mx_quantize_dual_batch(
                    [(d["X"], one), (d["W"], d["woff"])])
            else:
                wq, ws, wT, wTs, _ = qw[i]
                xq, xs, xT, xTs, _ = mxq.mx_quantize_dual(d["X"], one)
            gq, gs, gT, gTs, _ = mxq.mx_quantize_dual(d["dY"], one)
            mxq.mx_gemm(xq, xs, wq, ws)                                    # Y = X Wᵀ
            mxq.mx_gemm(gq, gs, wT[:, :fout], wTs[:, :fout // 32])         # dX = dY W
            mxq.mx_gemm(gT[:, :T], gTs[:, :T // 32], xT[:, :T], xTs[:, :T // 32])  # dW
        if qgu is None:
            (xq, xs, xT, xTs, poff), (wq, ws, guT, guTs, _) = mxq.mx_quantize_dual_batch(
                [(rX, offs_d), (Wgu, w_off_gu)])
        else:
            wq, ws, guT, guTs, _ = qgu
            xq, xs, xT, xTs, poff = mxq.mx_quantize_dual(rX, offs_d)
        mxq.mx_grouped_gemm(xq, xs, wq.view(E, 2 * FFN, HIDDEN),
                            ws.view(E, 2 * FFN, HIDDEN // 32), offs_d)
        if qdn is None:
            (hq, hs, hT, hTs, _), (dq, dsc, dnT, dnTs, _) = mxq.mx_quantize_dual_batch(
                [(rh, offs_d), (Wdn, w_off_dn)])
        else:
            dq, dsc, dnT, dnTs, _ = qdn
            hq, hs, hT, hTs, _ = mxq.mx_quantize_dual(rh, offs_d)
        mxq.mx_grouped_gemm(hq, hs, dq.view(E, HIDDEN, FFN), dsc.view(E, HIDDEN, FFN // 32),
                            offs_d)
        gq, gs, dyT, dyTs, _ = mxq.mx_quantize_dual(rdY, offs_d)
        bq, bs = mxq.expert_view(dnT, dnTs, E, HIDDEN)
        mxq.mx_grouped_gemm(gq, gs, bq, bs, offs_d)
        uq, us, duT, duTs, _ = mxq.mx_quantize_dual(rdGU, offs_d)
        bq2, bs2 = mxq.expert_view(guT, guTs, E, 2 * FFN)
        mxq.mx_grouped_gemm(uq, us, bq2, bs2, offs_d)
        mxq.mx_grouped_gemm_wgrad(dyT, dyTs, hT, hTs, poff)
        mxq.mx_grouped_gemm_wgrad(duT, duTs, xT, xTs, poff)

    dense_flops = sum(6 * T * fin * fout for _, fin, fout in workloads.BLOCK_DENSE_LINEARS)
    moe_flops = 6 * M * (2 * FFN * HIDDEN + HIDDEN * FFN)
    flops = dense_flops + moe_flops
    _, ms = _timed(torch, step, reps=5)
    wts = quant_weights()
    _, ms_once = _timed(torch, step, wts, reps=5)
    return {"tokens": T, "routed_rows": M, "algorithmic_flops": flops,
            "dense_flops": dense_flops, "routed_flops": moe_flops,
            "ms_per_step": ms, "TFLOP_per_s_incl_quant": flops / (ms * 1e-3) / 1e12,
            "weights_quantized_once": {"ms_per_step": ms_once,
                                       "TFLOP_per_s_incl_quant": flops / (ms_once * 1e-3) / 1e12},
            "data": "device-drawn synthetic tensors (torch generator, seeded)"}


def bf16_sweep(torch, mxq, reps=10):
    """Context, not part of the step: forward Linears of the block in BF16
    through torch.matmul (the ROCm BLAS library) against the MX path over
    token counts, as a per-shape answer to "is MXFP8 at least as fast as
    BF16".  The MX path: row quantization of input and weight in one launch
    (`mx_quantize_rowwise_batch`), then the MX GEMM; with the weight's copy
    made once per optimizer step, only the input is quantized per call.
    Eager times include each call's host-side launch cost (the wrappers
    allocate outputs and go through ctypes), which decides the small shapes;
    the HIP-graph columns replay 10 captured calls and time the GPU alone."""
    g = torch.Generator(device="cuda").manual_seed(0)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps * 1e3

    def graphed(fn, n=10):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(n):
                fn()
        us = timed(graph.replay) / n
        del graph
        return us

    out = []
    for name, fin, fout in (("o_proj", HIDDEN, HIDDEN), ("shared_gate", HIDDEN, 2 * FFN)):
        w = (torch.randn(fout, fin, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        wq, ws = mxq.mx_quantize_rowwise(w)
        for tokens in (1024, 4096, 16384):
            x = torch.randn(tokens, fin, device="cuda", generator=g).to(torch.bfloat16)
            xq, xs = mxq.mx_quantize_rowwise(x)
            bf16 = lambda: torch.matmul(x, w.t())
            gemm = lambda: mxq.mx_gemm(xq, xs, wq, ws)
            act = lambda: mxq.mx_gemm(*mxq.mx_quantize_rowwise(x), wq, ws)

            def both():
                (aq, asc), (bq, bsc) = mxq.mx_quantize_rowwise_batch([x, w])
                return mxq.mx_gemm(aq, asc, bq, bsc)

            r = {"linear": name, "in": fin, "out": fout, "tokens": tokens}
            for key, fn in (("bf16", bf16), ("mx_gemm", gemm), ("mx_incl_act_quant", act),
                            ("mx_incl_quant", both)):
                r[key + "_us"] = timed(fn)
                r[key + "_graph_us"] = graphed(fn)
            for key in ("mx_gemm", "mx_incl_act_quant", "mx_incl_quant"):
                r["speedup_" + key[3:]] = r["bf16_us"] / r[key + "_us"]
                r["speedup_" + key[3:] + "_graph"] = r["bf16_graph_us"] / r[key + "_graph_us"]
            out.append(r)
    return out


def bf16_moe_step(torch, X, h, Wgu, Wdn, dY, dGU, counts, mx_ms, reps=5):
    """Context, not part of the step: the same six expert-layer products in
    BF16 through torch's grouped matmul (no quantization; the transposed
    operand copies it needs are made before timing)."""
    if not hasattr(torch, "_grouped_mm"):
        return {"skipped": "torch._grouped_mm not available"}
    ends = torch.from_numpy(counts.cumsum()).to(torch.int32).cuda()
    wgu = Wgu.view(E, 2 * FFN, HIDDEN)
    wdn = Wdn.view(E, HIDDEN, FFN)
    wguT = wgu.transpose(1, 2).contiguous()          # [E, 2048, 2816]
    wdnT = wdn.transpose(1, 2).contiguous()          # [E, 1408, 2048]
    dYT = dY.t().contiguous()                        # [2048, M]
    dGUT = dGU.t().contiguous()                      # [2816, M]

    def step():
        torch._grouped_mm(X, wguT, offs=ends)        # gate/up forward
        torch._grouped_mm(h, wdnT, offs=ends)        # down forward
        torch._grouped_mm(dY, wdn, offs=ends)        # down data gradient
        torch._grouped_mm(dGU, wgu, offs=ends)       # gate/up data gradient
        torch._grouped_mm(dYT, h, offs=ends)         # down weight gradient [E, 2048, 1408]
        torch._grouped_mm(dGUT, X, offs=ends)        # gate/up weight gradient [E, 2816, 2048]

    try:
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            step()
        e.record()
        torch.cuda.synchronize()
    except Exception as ex:                           # report, do not fail the bench
        return {"skipped": "torch._grouped_mm failed: %s" % repr(ex)[:200]}
    ms = s.elapsed_time(e) / reps
    flops = 3 * 2 * int(counts.sum()) * (2 * FFN * HIDDEN + HIDDEN * FFN)
    return {"ms_per_step": ms, "TFLOP_per_s": flops / (ms * 1e-3) / 1e12,
            "mx_step_speedup": ms / mx_ms}


def cpu_baseline(fw, bw, budget_s):
    """The CPU oracle (unchanged) on a bounded sample of the same step: whole
    experts, smallest first, until about ``budget_s`` seconds of CPU time;
    TFLOP/s = the sample's algorithmic GEMM FLOPs / oracle time.  The
    smallest expert is also timed with the BLAS pool limited to one thread."""
    import numpy as np
    from oracle import gemm, mx

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"), default=1)
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f
                              if ln.startswith("model name")), None)
    except OSError:
        pass

    counts, offs = fw["counts"], fw["offsets"]

    def expert(e):
        """The oracle's forward, dgrad and wgrad of expert e; its GEMM FLOPs."""
        lo, hi = int(offs[e]), int(offs[e + 1])
        xq, xs = mx.mx_quantize_rowwise(fw["X"][lo:hi])
        wq, ws = mx.mx_quantize_rowwise(fw["W_gu"][e])
        gemm.gemm_ref(mx.mx_dequantize(xq, xs), mx.mx_dequantize(wq, ws))
        hq, hs = mx.mx_quantize_rowwise(fw["h"][lo:hi])
        dq, dsc = mx.mx_quantize_rowwise(fw["W_dn"][e])
        gemm.gemm_ref(mx.mx_dequantize(hq, hs), mx.mx_dequantize(dq, dsc))
        gq, gs = mx.mx_quantize_rowwise(bw["dY"][lo:hi])
        bq, bs = mx.mx_quantize_colwise(fw["W_dn"][e])
        gemm.gemm_ref(mx.mx_dequantize(gq, gs), mx.mx_dequantize(bq, bs))
        uq, us = mx.mx_quantize_rowwise(bw["dGU"][lo:hi])
        bq2, bs2 = mx.mx_quantize_colwise(fw["W_gu"][e])
        gemm.gemm_ref(mx.mx_dequantize(uq, us), mx.mx_dequantize(bq2, bs2))
        one = np.array([0, hi - lo], np.int64)
        aT, aTs, p = mx.mx_quantize_grouped_colwise(bw["dY"][lo:hi], one)
        bT, bTs, _ = mx.mx_quantize_grouped_colwise(fw["h"][lo:hi], one)
        gemm.grouped_wgrad_ref(mx.mx_dequantize(aT, aTs), mx.mx_dequantize(bT, bTs), p)
        aT, aTs, p = mx.mx_quantize_grouped_colwise(bw["dGU"][lo:hi], one)
        bT, bTs, _ = mx.mx_quantize_grouped_colwise(fw["X"][lo:hi], one)
        gemm.grouped_wgrad_ref(mx.mx_dequantize(aT, aTs), mx.mx_dequantize(bT, bTs), p)
        return 6 * (hi - lo) * (2 * FFN * HIDDEN + HIDDEN * FFN)

    order = np.argsort(counts, kind="stable")
    done, flops, t_tot = [], 0, 0.0
    for e in order:
        t0 = time.perf_counter()
        flops += expert(e)
        t_tot += time.perf_counter() - t0
        done.append(int(e))
        if t_tot >= budget_s:
            break
    single = None
    if threadpool_limits is not None and len(order):
        with threadpool_limits(limits=1, user_api="blas"):
            t0 = time.perf_counter()
            f1 = expert(order[0])
            t1 = time.perf_counter() - t0
        single = {"value": f1 / t1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                  "sample": "the smallest expert (%d rows), %.1f s" % (int(counts[order[0]]), t1)}
    return {"value": flops / t_tot / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model, "blas_threads": int(threads),
            "sample": "full fwd+dgrad+wgrad oracle path (quant, dequant, FP64 GEMM and "
                      "|A|·|B| magnitudes) for %d whole experts, smallest first (%d rows); "
                      "%.1f s" % (len(done), sum(int(counts[e]) for e in done), t_tot),
            "single_thread": single}


if __name__ == "__main__":
    main()
