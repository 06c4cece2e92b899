"""fp8_quantize_per_group_noalloc (no workspace argument, no allocation: the
row and group maxima live in the library's per-GPU scratch array) against
fp8_quantize_per_group with a workspace, through the C ABI: codes and scales
bit for bit, on two calls in a row, the second on a smaller input with
smaller values, so that the scratch still holds the first call's larger
maxima when the second call runs.  The second call is also checked against
the oracle."""

import numpy as np
import pytest
import torch

from block_quant_gemm_amd import mxq, workloads
from oracle import per_tensor
from tests.gpu_helpers import host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def test_noalloc_per_group_matches_workspace_entry_on_two_calls():
    cases = [([700, 0, 1, 2100, 33, 0, 950], 512, 1.0, 0.01),   # outliers x30
             ([40, 300, 0], 256, 1e-3, 0.0)]
    for i, (counts, K, sigma, frac) in enumerate(cases):
        counts = np.array(counts, np.int64)
        offs = workloads.offsets_from_counts(counts)
        M, E = int(counts.sum()), len(counts)
        say(f"no-alloc per-group call {i + 1}: M={M} K={K} E={E}")
        bits = workloads.bf16_normal((M, K), sigma, seed=40 + i, name="noalloc",
                                     outlier_frac=frac, outlier_scale=30.0)
        x, offs_d = to_dev_bf16(bits), to_dev(offs)
        q = torch.full((M, K), 0xAB, dtype=torch.uint8, device="cuda")
        s = torch.full((E,), -1.0, dtype=torch.float32, device="cuda")
        mxq.fp8_quantize_per_group_noalloc(x, offs_d, q, s)
        rq, rs = mxq.fp8_quantize_per_group(x, offs_d)
        torch.cuda.synchronize()
        assert torch.equal(q, rq), "codes differ from fp8_quantize_per_group"
        assert torch.equal(s.view(torch.int32), rs.view(torch.int32)), "scales differ"
    oq, os_ = per_tensor.pg_quantize(bits, offs)
    assert np.array_equal(host(q), oq) and np.array_equal(host(s).view(np.uint32),
                                                          np.asarray(os_, np.float32).view(np.uint32))
