"""The C-ABI library loads and exports every symbol include/mxq.h declares,
and its host-side argument checks reject bad calls without touching a GPU.
CPU only (no kernel is launched)."""

import ctypes
import os
import re

import pytest

from block_quant_gemm_amd import mxq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "mxq.h"), encoding="utf-8").read()
    return sorted(set(re.findall(r"MXQ_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mxq.LIB_PATH):
        pytest.fail("libmxq.so is not built (run __graft_entry__.build())")
    return mxq.load()


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0        # counts devices without initialising one
    except Exception:
        return False


@pytest.fixture(scope="module")
def host_only_lib(lib):
    """The library, for calls that pass fake device addresses and rely on the
    host-side checks rejecting them before any launch.  Where a GPU is
    visible these never run: a regression in a check would launch a kernel
    on the fake address."""
    if _gpu_visible():
        pytest.skip("passes fake device addresses; runs only where no GPU is visible")
    return lib


def test_every_declared_symbol_is_exported(lib):
    names = declared_symbols()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(mxq.EXPORTS)


def test_version_and_status_strings(lib):
    assert lib.mxq_version() == 10000
    assert lib.mxq_status_string(0) == b"ok"
    assert lib.mxq_status_string(3).startswith(b"misaligned")


def test_host_validation_errors(host_only_lib):
    lib = host_only_lib
    P = 4096  # a fake, never-dereferenced 16-byte-aligned address
    # negative / inconsistent sizes
    assert lib.mx_quantize_rowwise(P, -1, 32, 32, P, 32, P, 1, None) == 2
    assert lib.mx_quantize_rowwise(P, 4, 40, 40, P, 48, P, 2, None) == 2      # K % 32
    assert lib.mx_quantize_rowwise(None, 4, 32, 32, P, 32, P, 1, None) == 1  # NULL
    assert lib.mx_quantize_rowwise(P, 4, 32, 36, P, 32, P, 1, None) == 3     # ldx % 8
    assert lib.mx_quantize_rowwise(P + 2, 4, 32, 32, P, 32, P, 1, None) == 3  # misaligned
    # empty inputs are no-ops that launch nothing
    assert lib.mx_quantize_rowwise(None, 0, 32, 32, None, 32, None, 1, None) == 0
    assert lib.mx_quantize_colwise(P, 64, 20, 24, None, 0, P, 64, 64, P, 2, None, None) == 2
    assert lib.mx_quantize_colwise(P, 64, 32, 32, None, 0, P, 64, 32, P, 1, None, None) == 2
    # with offsets the capacity must hold the padded total's bound M + 31*E (64 + 124)
    assert lib.mx_quantize_colwise(P, 64, 32, 32, P, 4, P, 160, 160, P, 16, P, None) == 2
    assert lib.mx_quantize_dual(P, 64, 32, 32, P, 4, P, 32, P, 16, P, 160, 160, P, 16, P, None) == 2
    assert lib.mx_quantize_dual(P, 64, 32, 32, None, 0, P, 32, P, 16, P, 32, 32, P, 16, P, None) == 2
    assert lib.mx_gemm(P, P, 32, 1, P, P, 32, 1, 4, 4, 33, P, 4, 0, 0, None) == 2
    assert lib.mx_gemm(P, P, 32, 1, P, P, 32, 1, 4, 4, 32, P, 4, 2, 0, None) == 4  # out dtype
    assert lib.mx_gemm(P, P, 32, 1, P, P, 32, 1, 4, 4, 32, P, 4, 0, 7, None) == 4  # accum
    assert lib.mx_gemm(P, P, 32, 1, P, P, 32, 1, 4, 8, 32, P, 4, 0, 0, None) == 2  # ldc < N
    assert lib.mx_gemm(P, P, 24, 1, P, P, 32, 1, 4, 4, 32, P, 4, 0, 0, None) == 2  # lda < K
    assert lib.mx_gemm(None, None, 32, 1, None, None, 32, 1, 0, 4, 32, None, 4, 0, 0, None) == 0
    assert lib.mx_grouped_gemm(P, P, 32, 1, P, P, 32, 1, 256, 8, None, 4, 8, 8, 32, P, 8, 0, 0, None) == 1
    assert lib.mx_grouped_gemm(P, P, 32, 1, P, P, 32, 1, 256, 8, P, 0, 8, 8, 32, P, 8, 0, 0, None) == 2
    assert lib.mx_grouped_gemm(P, P, 32, 1, P, P, 32, 1, 250, 8, P, 4, 8, 8, 32, P, 8, 0, 0, None) == 3
    assert lib.mx_grouped_gemm_wgrad(P, P, 40, 2, P, P, 32, 1, P, 2, 8, 8, P, 8, 0, 0, None) == 3
    assert lib.fp8_quantize_per_tensor(P, -5, P, P, P, 4096, None) == 2
    assert lib.fp8_quantize_per_tensor(P, 100, P, P, P, 4, None) == 5          # workspace
    # given amax: (x, n, amax, q, scale, stream)
    assert lib.fp8_quantize_per_tensor_amax(P, -5, P, P, P, None) == 2
    assert lib.fp8_quantize_per_tensor_amax(P, 100, None, P, P, None) == 1     # amax
    assert lib.fp8_quantize_per_tensor_amax(P, 100, P, P, None, None) == 1     # scale
    assert lib.fp8_quantize_per_tensor_amax(P + 2, 100, P, P, P, None) == 3    # misaligned x
    # GEMM with the output's amax: (a, sa, lda, b, sb, ldb, M, N, K, c, ldc, out, acc, amax, s)
    assert lib.fp8_gemm_per_tensor_amax(P, P, 32, P, P, 32, 4, 4, 32, P, 4, 0, 0, None, None) == 1
    assert lib.fp8_gemm_per_tensor_amax(P, P, 32, P, P, 32, 4, 4, 32, P, 4, 0, 0, P + 2, None) == 3
    assert lib.fp8_gemm_per_tensor_amax(P, P, 32, P, P, 32, 4, 4, 32, P, 4, 2, 0, P, None) == 4
    assert lib.fp8_gemm_per_tensor_amax(P, P, 32, P, P, 32, 4, 4, 33, P, 4, 0, 0, P, None) == 2
    assert lib.mxq_workspace_size(0, 100, 0, 0, 0) > 0
    assert lib.mxq_workspace_size(0, 0, 0, 0, 0) == 0
    assert lib.mxq_validate_offsets(None, 4, 10, None) == 1


def test_rowwise_batch_validation_errors(host_only_lib):
    lib = host_only_lib
    P = 4096
    It = mxq.RowwiseItem

    def call(*items, n=None):
        arr = (It * len(items))(*items)
        return lib.mx_quantize_rowwise_batch(arr, len(items) if n is None else n, None)

    good = It(P, 4, 32, 32, P, 32, P, 1)
    assert call(good, n=0) == 2                                     # n out of range
    assert call(*[good] * 5) == 2                                   # past the batch maximum
    assert lib.mx_quantize_rowwise_batch(None, 1, None) == 1        # NULL items
    assert call(good, It(P, 4, 40, 40, P, 48, P, 2)) == 2           # K % 32 in item 1
    assert call(It(None, 4, 32, 32, P, 32, P, 1), good) == 1        # NULL x in item 0
    assert call(good, It(P + 2, 4, 32, 32, P, 32, P, 1)) == 3       # misaligned x in item 1
    empty = It(None, 0, 32, 32, None, 32, None, 1)
    assert call(empty, empty) == 0                                  # nothing to launch
    assert mxq.ROWWISE_BATCH_MAX == 4


def test_dual_batch_validation_errors(host_only_lib):
    lib = host_only_lib
    P = 4096
    It = mxq.DualItem

    def call(*items, n=None):
        arr = (It * len(items))(*items)
        return lib.mx_quantize_dual_batch(arr, len(items) if n is None else n, None)

    # DualItem(x, M, K, ldx, offsets, E, q, ldq, scale, lds, qT, ldqT, M_cap, scaleT, ldsT, poff)
    good = It(P, 64, 32, 32, P, 4, P, 32, P, 16, P, 192, 192, P, 16, P)
    assert call(good, n=0) == 2                                     # n out of range
    assert call(*[good] * 5) == 2                                   # past the batch maximum
    assert lib.mx_quantize_dual_batch(None, 1, None) == 1           # NULL items
    assert call(good, It(P, 64, 32, 32, P, 4, P, 32, P, 16, P, 160, 160, P, 16, P)) == 2  # M_cap
    assert call(It(P, 64, 40, 40, P, 4, P, 48, P, 16, P, 192, 192, P, 16, P), good) == 2  # K % 32
    assert call(good, It(P, 64, 32, 32, P, 4, P, 32, P, 16, None, 192, 192, P, 16, P)) == 1
    assert call(good, It(P + 2, 64, 32, 32, P, 4, P, 32, P, 16, P, 192, 192, P, 16, P)) == 3
    empty = It(None, 0, 0, 0, None, 0, None, 0, None, 0, None, 0, 0, None, 0, None)
    assert call(empty, empty) == 0                                  # nothing to launch
    assert mxq.DUAL_BATCH_MAX == 4
    assert ctypes.sizeof(It) == 128                                 # mxq_dual_item's layout


def test_per_group_validation_errors(host_only_lib):
    lib = host_only_lib
    P = 4096
    # fp8_quantize_per_group(x, M, K, ldx, offsets, E, q, ldq, scales, ws, ws_bytes, stream)
    ws = lib.mxq_workspace_size(1, 64, 4, 0, 0)
    assert ws == (64 + 4) * 4
    assert lib.fp8_quantize_per_group(P, -1, 32, 32, P, 4, P, 32, P, P, ws, None) == 2
    assert lib.fp8_quantize_per_group(P, 64, 32, 32, P, 0, P, 32, P, P, ws, None) == 2   # E
    assert lib.fp8_quantize_per_group(P, 64, 32, 32, P, 257, P, 32, P, P, ws, None) == 2
    assert lib.fp8_quantize_per_group(P, 64, 32, 32, None, 4, P, 32, P, P, ws, None) == 1
    assert lib.fp8_quantize_per_group(P, 64, 32, 32, P, 4, P, 32, None, P, ws, None) == 1
    assert lib.fp8_quantize_per_group(P, 64, 36, 40, P, 4, P, 48, P, P, ws, None) == 2   # K % 8
    assert lib.fp8_quantize_per_group(P, 64, 32, 36, P, 4, P, 32, P, P, ws, None) == 3   # ldx % 8
    assert lib.fp8_quantize_per_group(P, 64, 32, 32, P, 4, P, 36, P, P, ws, None) == 3   # ldq % 8
    assert lib.fp8_quantize_per_group(P, 64, 32, 32, P, 4, P, 32, P, P, ws - 4, None) == 5
    # fp8_grouped_gemm_per_group(a, sa, lda, b, sb, ldb, b_estride, offsets, E, M, N, K, c, ldc,
    #                            out, accum, stream)
    assert lib.fp8_grouped_gemm_per_group(P, P, 32, P, P, 32, 256, None, 4, 8, 8, 32, P, 8, 0, 0, None) == 1
    assert lib.fp8_grouped_gemm_per_group(P, None, 32, P, P, 32, 256, P, 4, 8, 8, 32, P, 8, 0, 0, None) == 1
    assert lib.fp8_grouped_gemm_per_group(P, P, 32, P, P, 32, 256, P, 0, 8, 8, 32, P, 8, 0, 0, None) == 2
    assert lib.fp8_grouped_gemm_per_group(P, P, 32, P, P, 32, 250, P, 4, 8, 8, 32, P, 8, 0, 0, None) == 3
    assert lib.fp8_grouped_gemm_per_group(P, P, 32, P, P, 32, 256, P, 4, 8, 8, 40, P, 8, 0, 0, None) == 2
    assert lib.fp8_grouped_gemm_per_group(P, P, 32, P, P, 32, 256, P, 4, 8, 8, 32, P, 8, 0, 2, None) == 4


def test_per_group_transposed_and_wgrad_validation_errors(host_only_lib):
    lib = host_only_lib
    P = 4096
    ws = lib.mxq_workspace_size(1, 64, 4, 0, 0)
    # fp8_quantize_per_group_colwise(x, M, K, ldx, offsets, E, qT, ldqT, M_cap, scales,
    #                                offsets_padded, ws, ws_bytes, stream)
    assert lib.fp8_quantize_per_group_colwise(P, -1, 32, 32, P, 4, P, 256, 256, P, P, P, ws, None) == 2
    assert lib.fp8_quantize_per_group_colwise(P, 64, 32, 32, P, 0, P, 256, 256, P, P, P, ws, None) == 2
    assert lib.fp8_quantize_per_group_colwise(P, 64, 36, 40, P, 4, P, 256, 256, P, P, P, ws, None) == 2
    assert lib.fp8_quantize_per_group_colwise(P, 64, 32, 32, P, 4, P, 256, 250, P, P, P, ws, None) == 2
    assert lib.fp8_quantize_per_group_colwise(P, 64, 32, 32, P, 4, P, 200, 256, P, P, P, ws, None) == 2
    assert lib.fp8_quantize_per_group_colwise(P, 64, 32, 32, P, 4, P, 264, 256, P, P, P, ws, None) == 3
    assert lib.fp8_quantize_per_group_colwise(P, 64, 32, 32, None, 4, P, 256, 256, P, P, P, ws, None) == 1
    assert lib.fp8_quantize_per_group_colwise(P, 64, 32, 32, P, 4, P, 256, 256, P, P, P, ws - 4, None) == 5
    assert lib.fp8_quantize_per_group_colwise(P, 64, 32, 32, P, 4, P, 160, 160, P, P, P, ws, None) == 2
    # fp8_quantize_per_group_noalloc(x, M, K, ldx, offsets, E, q, ldq, scales, stream):
    # its scratch holds M + E <= 262144 words
    nf = lib.fp8_quantize_per_group_noalloc
    assert nf(P, 262144, 32, 32, P, 1, P, 32, P, None) == 2
    assert nf(P, 262000, 32, 32, P, 256, P, 32, P, None) == 2
    assert nf(P, 64, 32, 32, P, 0, P, 32, P, None) == 2
    assert nf(P, -1, 32, 32, P, 4, P, 32, P, None) == 2
    assert nf(P, 64, 32, 32, None, 4, P, 32, P, None) == 1
    # fp8_grouped_gemm_wgrad_per_group(at, sa, lda_t, bt, sb, ldb_t, poff, E, N, K, c, ldc,
    #                                  out, accum, stream)
    assert lib.fp8_grouped_gemm_wgrad_per_group(P, P, 40, P, P, 32, P, 2, 8, 8, P, 8, 0, 0, None) == 3
    assert lib.fp8_grouped_gemm_wgrad_per_group(P, None, 32, P, P, 32, P, 2, 8, 8, P, 8, 0, 0, None) == 1
    assert lib.fp8_grouped_gemm_wgrad_per_group(P, P, 32, P, P, 32, P, 0, 8, 8, P, 8, 0, 0, None) == 2
    assert lib.fp8_grouped_gemm_wgrad_per_group(P, P, 32, P, P, 32, P, 2, 8, 8, P, 4, 0, 0, None) == 2
    assert lib.fp8_grouped_gemm_wgrad_per_group(P, P, 32, P, P, 32, P, 2, 8, 8, P, 8, 0, 2, None) == 4


def test_size_limits_rejected(host_only_lib):
    lib = host_only_lib
    """Sizes past what the kernels index with 32-bit offsets are rejected on
    the host (no launch): a 256-row GEMM tile must span < 2^31 bytes, the
    row quantizer's segment count must fit 31 bits."""
    P = 4096
    big_ld = (1 << 31) // 256                         # 256-row tile + K exceeds 2^31
    assert lib.mx_gemm(P, P, big_ld, 64, P, P, 32, 1, 4, 4, 32, P, 4, 0, 0, None) == 2
    assert lib.mx_gemm(P, P, 32, 1, P, P, big_ld, 64, 4, 4, 32, P, 4, 0, 0, None) == 2
    assert lib.mx_grouped_gemm(P, P, big_ld, 64, P, P, 32, 1, 256, 8, P, 4, 8, 8, 32, P, 8,
                               0, 0, None) == 2
    assert lib.mx_grouped_gemm_wgrad(P, P, big_ld, big_ld // 32, P, P, big_ld, big_ld // 32,
                                     P, 2, 8, 8, P, 8, 0, 0, None) == 2
    # strided (non-contiguous) rows: 2^31 segments of 512 elements
    rows = 1 << 29
    assert lib.mx_quantize_rowwise(P, rows, 2048, 2056, P, 2048, P, 64, None) == 2
    # the largest accepted tile stride passes the size check (then fails on alignment)
    ok_ld = ((1 << 31) - 64) // 257 // 16 * 16
    assert lib.mx_gemm(P + 2, P, ok_ld, 64, P, P, 32, 1, 4, 4, 32, P, 4, 0, 0, None) == 3


def test_swiglu_product_validation_errors(host_only_lib):
    lib = host_only_lib
    P = 4096
    f = lib.mx_grouped_gemm_swiglu

    # (a, as, lda, ldsa, b, bs, ldb, ldsb, b_estride, bs_estride, offsets, E, M, F, K,
    #  gu, ldgu, hq, ldhq, hs, ldhs, hqT, ldhqT, hsT, ldhsT, M_cap, poff, stream)
    def call(**kw):
        a = dict(a=P, as_=P, lda=32, ldsa=16, b=P, bs=P, ldb=32, ldsb=16, be=4096, bse=2048,
                 off=P, E=4, M=64, F=64, K=32, gu=P, ldgu=128, hq=P, ldhq=64, hs=P, ldhs=16,
                 hqT=P, ldhqT=256, hsT=P, ldhsT=16, cap=256, poff=P)
        a.update(kw)
        return f(a["a"], a["as_"], a["lda"], a["ldsa"], a["b"], a["bs"], a["ldb"], a["ldsb"],
                 a["be"], a["bse"], a["off"], a["E"], a["M"], a["F"], a["K"], a["gu"],
                 a["ldgu"], a["hq"], a["ldhq"], a["hs"], a["ldhs"], a["hqT"], a["ldhqT"],
                 a["hsT"], a["ldhsT"], a["cap"], a["poff"], None)

    assert call(F=40, ldhq=64) == 2                     # F % 32
    assert call(K=40) == 2                              # K % 32
    assert call(cap=250) == 2                           # M_cap % 32
    assert call(cap=160, ldhqT=160) == 2                # M_cap < M + 31 E
    assert call(off=None) == 1
    assert call(E=0) == 2
    assert call(E=257) == 2
    assert call(hq=None) == 1
    assert call(hsT=None) == 1
    assert call(ldhq=48) == 2                           # ldhq < F
    assert call(ldhq=72) == 3                           # ldhq % 16
    assert call(ldhqT=264) == 3
    assert call(ldhqT=224) == 2                         # ldhqT < M_cap
    assert call(ldgu=96) == 2                           # ldgu < 2F
    assert call(ldgu=132) == 3                          # ldgu % 8
    assert call(gu=P + 8) == 3
    assert call(be=4088) == 3                           # b_estride % 16
    assert call(lda=24) == 2                            # lda < K
    # an expert's 2F weight rows must span < 2^30 bytes
    assert call(F=4096, ldhq=4096, ldgu=8192, ldhs=128, ldb=1 << 17, be=1 << 30) == 2
    assert call(F=0) == 0                               # no-op


def test_fused_per_group_and_blockwise_validation_errors(host_only_lib):
    lib = host_only_lib
    P = 4096
    # fp8_grouped_gemm_per_group_swiglu(a, sa, lda, b, sb, ldb, b_estride, offsets, E, M, F, K,
    #                                   gu, ldgu, h, ldh, h_amax, stream)
    f = lib.fp8_grouped_gemm_per_group_swiglu
    assert f(P, P, 32, P, P, 32, 4096, P, 4, 64, 64, 32, P, 128, P, 64, None, None) == 1  # amax
    assert f(P, P, 32, P, P, 32, 4096, None, 4, 64, 64, 32, P, 128, P, 64, P, None) == 1
    assert f(P, P, 32, P, P, 32, 4096, P, 0, 64, 64, 32, P, 128, P, 64, P, None) == 2     # E
    assert f(P, P, 32, P, P, 32, 4096, P, 4, 64, 40, 32, P, 128, P, 64, P, None) == 2     # F % 32
    assert f(P, P, 32, P, P, 32, 4096, P, 4, 64, 64, 32, P, 128, P, 48, P, None) == 2     # ldh < F
    assert f(P, P, 32, P, P, 32, 4096, P, 4, 64, 64, 32, P, 96, P, 64, P, None) == 2      # ldgu < 2F
    assert f(P, P, 32, P, P, 32, 4096, P, 4, 64, 64, 32, P, 128, P, 68, P, None) == 3     # ldh % 8
    assert f(P, P, 32, P, P, 32, 4088, P, 4, 64, 64, 32, P, 128, P, 64, P, None) == 3     # b_estride
    assert f(P, P, 32, P, P, 32, 4096, P, 4, 64, 64, 32, P, 128, None, 64, P, None) == 1  # h
    # fp8_quantize_per_group_amax(x, M, K, ldx, offsets, E, amax, q, ldq, scales, ws, ws_bytes, s)
    ws = lib.mxq_workspace_size(1, 0, 4, 0, 0)
    assert ws == 16
    g = lib.fp8_quantize_per_group_amax
    assert g(P, 64, 32, 32, P, 4, None, P, 32, P, P, ws, None) == 1                     # amax
    assert g(P, 64, 32, 32, P, 4, P, P, 32, P, P, ws - 4, None) == 5                    # ws
    assert g(P, 64, 32, 36, P, 4, P, P, 32, P, P, ws, None) == 3                        # ldx % 8
    gc = lib.fp8_quantize_per_group_colwise_amax
    assert gc(P, 64, 32, 32, P, 4, None, P, 256, 256, P, P, P, ws, None) == 1
    assert gc(P, 64, 32, 32, P, 4, P, P, 256, 250, P, P, P, ws, None) == 2              # M_cap
    # fp8_quantize_per_group_dual(x, M, K, ldx, offsets, E, amax, q, ldq, qT, ldqT, M_cap,
    #                             scales, offsets_padded, ws, ws_bytes, s)
    d = lib.fp8_quantize_per_group_dual
    assert d(P, 64, 32, 32, P, 4, None, P, 32, P, 256, 256, P, P, P, ws, None) == 5    # row maxima
    assert d(P, 64, 32, 32, P, 4, P, P, 32, P, 256, 256, P, P, P, ws - 4, None) == 5   # amax given
    assert d(P, 64, 32, 32, P, 4, P, P, 32, P, 256, 250, P, P, P, ws, None) == 2       # M_cap
    assert d(P, 64, 32, 32, P, 4, P, P, 32, P, 160, 160, P, P, P, ws, None) == 2       # < M + 31 E
    assert d(P, 64, 32, 32, P, 4, P, P, 32, P, 256, 256, None, P, P, ws, None) == 1    # scales
    # blockwise: fp8_quantize_blockwise_act(x, M, K, ldx, q, ldq, scales, lds, s)
    assert lib.fp8_quantize_blockwise_act(P, 8, 96, 96, P, 96, P, 1, None) == 2          # K % 128
    assert lib.fp8_quantize_blockwise_act(P, 8, 128, 128, P, 128, P, 0, None) == 2       # lds
    assert lib.fp8_quantize_blockwise_act(P, 8, 128, 132, P, 128, P, 1, None) == 3       # ldx % 8
    assert lib.fp8_quantize_blockwise_act(None, 8, 128, 128, P, 128, P, 1, None) == 1
    assert lib.fp8_quantize_blockwise_act(None, 0, 128, 128, None, 128, None, 1, None) == 0
    assert lib.fp8_quantize_blockwise_weight(P, 200, 256, 256, P, 256, P, 1, None) == 2  # lds
    assert lib.fp8_quantize_blockwise_weight(P + 8, 200, 256, 256, P, 256, P, 2, None) == 3
    # fp8_gemm_blockwise(a, sa, lda, ldsa, b, sb, ldb, ldsb, M, N, K, c, ldc, out, accum, s)
    h = lib.fp8_gemm_blockwise
    assert h(P, P, 128, 1, P, P, 128, 1, 4, 4, 96, P, 4, 0, 0, None) == 2                # K % 128
    assert h(P, P, 128, 0, P, P, 128, 1, 4, 4, 128, P, 4, 0, 0, None) == 2               # ldsa
    assert h(P, None, 128, 1, P, P, 128, 1, 4, 4, 128, P, 4, 0, 0, None) == 1
    assert h(P, P, 128, 1, P, P, 128, 1, 4, 4, 128, P, 4, 0, 3, None) == 4               # accum
    # the blockwise GEMM has only the FP8 matrix-unit accumulation
    assert h(P, P, 128, 1, P, P, 128, 1, 4, 4, 128, P, 4, 0, 1, None) == 4
    assert h(P, P, 128, 1, P, P, 128, 1, 0, 4, 128, None, 4, 0, 0, None) == 0            # M = 0
