"""Seeded synthetic workloads: BF16 tensors and MoE expert routing counts.

This module only draws random inputs; it holds no quantization or GEMM
arithmetic, and both the HIP path's tests/benchmark and the CPU oracle take
their inputs from here.  No datasets or trained weights are used: the tensors
have the shapes of DeepSeek-V3 16B layers ("DeepSeek-V3 16B FSDP2 MXFP8/HiF8
训练设计", §4.1 frozen 16B spec: hidden 2048, dense FFN 10944, MoE FFN 1408,
64 routed experts, 2 shared experts, top-6) and the value distributions listed
below.

Every tensor is drawn from its own generator, seeded by (seed, tensor name), so
any one tensor can be regenerated without the others.  Values are drawn as
float32 normals * sigma; a given fraction of positions, chosen without
replacement, is multiplied by an outlier factor; the result is converted to
BF16 by torch's round-to-nearest-even cast.
"""

import zlib

import numpy as np
import torch

HIDDEN = 2048
DENSE_FFN = 10944
MOE_FFN = 1408
N_EXPERTS = 64
TOP_K = 6
N_SHARED = 2


def _rng(seed, name):
    return np.random.default_rng([int(seed), zlib.crc32(name.encode())])


def bf16_normal(shape, sigma=1.0, *, seed=0, name="x", outlier_frac=0.0,
                outlier_scale=1.0):
    """BF16 bit patterns (uint16 array of ``shape``) of N(0, sigma) values."""
    rng = _rng(seed, name)
    n = int(np.prod(shape))
    x = rng.standard_normal(n, dtype=np.float32)
    x *= np.float32(sigma)
    k = int(round(outlier_frac * n))
    if k > 0:
        pos = rng.choice(n, size=k, replace=False)
        x[pos] *= np.float32(outlier_scale)
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).reshape(shape)


def expert_counts(total_rows, n_experts=N_EXPERTS, zipf_s=1.1, *, seed=0,
                  name="counts"):
    """Rows per expert: multinomial(total_rows, p) with p_e ∝ (e+1)^-s."""
    p = np.arange(1, n_experts + 1, dtype=np.float64) ** (-zipf_s)
    p /= p.sum()
    return _rng(seed, name).multinomial(total_rows, p).astype(np.int64)


def offsets_from_counts(counts):
    counts = np.asarray(counts, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


# --- named workloads -------------------------------------------------------

def tiny_linear(seed=0):
    """Tiny MXFP8 Linear forward: A 256x512 and W 256x512, N(0,1) with 1% of
    entries scaled by 100."""
    return {
        "A": bf16_normal((256, 512), 1.0, seed=seed, name="tiny.A",
                         outlier_frac=0.01, outlier_scale=100.0),
        "W": bf16_normal((256, 512), 1.0, seed=seed, name="tiny.W",
                         outlier_frac=0.01, outlier_scale=100.0),
    }


def dense_ffn(seed=0, tokens=8192):
    """Dense FFN gate/up projection: X [tokens, 2048] N(0,1) with 0.5%
    outliers x50, W [10944, 2048] N(0, 0.02)."""
    return {
        "X": bf16_normal((tokens, HIDDEN), 1.0, seed=seed, name="dense.X",
                         outlier_frac=0.005, outlier_scale=50.0),
        "W": bf16_normal((DENSE_FFN, HIDDEN), 0.02, seed=seed, name="dense.W"),
    }


def moe_counts(seed=0, tokens=8192, top_k=TOP_K, n_experts=N_EXPERTS):
    return expert_counts(tokens * top_k, n_experts, seed=seed)


def moe_forward(seed=0, tokens=8192, top_k=TOP_K, n_experts=N_EXPERTS,
                with_weights=True):
    """Routed-expert layer forward inputs.

    X [T*top_k, 2048] N(0,1) (token copies sorted by expert), h [T*top_k,
    1408] N(0,1) standing in for the SwiGLU output fed to the down
    projection, W_gu [E, 2*1408, 2048] and W_dn [E, 2048, 1408] N(0, 0.02).
    """
    counts = moe_counts(seed, tokens, top_k, n_experts)
    rows = int(counts.sum())
    d = {
        "counts": counts,
        "offsets": offsets_from_counts(counts),
        "X": bf16_normal((rows, HIDDEN), 1.0, seed=seed, name="moe.X"),
        "h": bf16_normal((rows, MOE_FFN), 1.0, seed=seed, name="moe.h"),
    }
    if with_weights:
        d["W_gu"] = bf16_normal((n_experts, 2 * MOE_FFN, HIDDEN), 0.02,
                                seed=seed, name="moe.W_gu")
        d["W_dn"] = bf16_normal((n_experts, HIDDEN, MOE_FFN), 0.02,
                                seed=seed, name="moe.W_dn")
    return d


def moe_backward(seed=0, tokens=8192, top_k=TOP_K, n_experts=N_EXPERTS):
    """Routed-expert layer backward inputs: dY [rows, 2048] N(0, 1e-3) and
    dGU [rows, 2*1408] N(0, 1e-3) standing in for the SwiGLU backward."""
    counts = moe_counts(seed, tokens, top_k, n_experts)
    rows = int(counts.sum())
    return {
        "dY": bf16_normal((rows, HIDDEN), 1e-3, seed=seed, name="moe.dY"),
        "dGU": bf16_normal((rows, 2 * MOE_FFN), 1e-3, seed=seed, name="moe.dGU"),
    }


# Tokens of the full block step: sequence 4096 x batch 4.
BLOCK_TOKENS = 4096 * 4

# MLA projection and shared-expert Linears of one 16B block:
# (name, in_features, out_features).
BLOCK_DENSE_LINEARS = [
    ("q_down", HIDDEN, 512),
    ("kv_up", 512, 3072),
    ("kv_down", HIDDEN, 576),
    ("o_proj", HIDDEN, HIDDEN),
    ("shared_gate", HIDDEN, N_SHARED * MOE_FFN),
    ("shared_up", HIDDEN, N_SHARED * MOE_FFN),
    ("shared_down", N_SHARED * MOE_FFN, HIDDEN),
]


def block_linear(name, in_features, out_features, seed=0, tokens=BLOCK_TOKENS):
    """One dense Linear of the full block step: X [tokens, in] N(0,1), W [out,
    in] N(0, 0.02), dY [tokens, out] N(0, 1e-3)."""
    return {
        "X": bf16_normal((tokens, in_features), 1.0, seed=seed, name=f"blk.{name}.X"),
        "W": bf16_normal((out_features, in_features), 0.02, seed=seed, name=f"blk.{name}.W"),
        "dY": bf16_normal((tokens, out_features), 1e-3, seed=seed, name=f"blk.{name}.dY"),
    }
