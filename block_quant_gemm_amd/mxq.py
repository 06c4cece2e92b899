"""ctypes binding of libmxq.so.

Argument marshalling only: every function below checks nothing itself,
allocates its outputs with torch (device memory is the caller's), passes raw
device pointers and the current HIP stream to the C function of the same
name, and raises if the library returns an error.  All arithmetic happens in
the library's HIP kernels; there is no other code path.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxq.so")

OUT_BF16, OUT_FP32 = 0, 1
ACC_MFMA_FP8, ACC_FP32 = 0, 1
WS_PER_TENSOR, WS_PER_GROUP = 0, 1

_i64, _i32, _p, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
ROWWISE_BATCH_MAX = 4
DUAL_BATCH_MAX = 4


class RowwiseItem(ctypes.Structure):
    """mxq_rowwise_item of mxq.h."""
    _fields_ = [("x", _p), ("M", _i64), ("K", _i64), ("ldx", _i64), ("q", _p), ("ldq", _i64),
                ("scale", _p), ("lds", _i64)]


class DualItem(ctypes.Structure):
    """mxq_dual_item of mxq.h."""
    _fields_ = [("x", _p), ("M", _i64), ("K", _i64), ("ldx", _i64), ("offsets", _p),
                ("E", _i32), ("q", _p), ("ldq", _i64), ("scale", _p), ("lds", _i64),
                ("qT", _p), ("ldqT", _i64), ("M_cap", _i64), ("scaleT", _p), ("ldsT", _i64),
                ("offsets_padded", _p)]


_SIGS = {
    "mxq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mxq_version": (ctypes.c_int, []),
    "mx_quantize_rowwise": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p]),
    "mx_quantize_rowwise_batch": (ctypes.c_int, [ctypes.POINTER(RowwiseItem), _i32, _p]),
    "mx_quantize_dual_batch": (ctypes.c_int, [ctypes.POINTER(DualItem), _i32, _p]),
    "mx_quantize_colwise": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _i32, _p, _i64, _i64,
                                           _p, _i64, _p, _p]),
    "mx_quantize_dual": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _i32, _p, _i64, _p, _i64,
                                        _p, _i64, _i64, _p, _i64, _p, _p]),
    "fp8_quantize_per_tensor": (ctypes.c_int, [_p, _i64, _p, _p, _p, _sz, _p]),
    "fp8_quantize_per_tensor_amax": (ctypes.c_int, [_p, _i64, _p, _p, _p, _p]),
    "fp8_quantize_per_group": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _i32, _p, _i64, _p,
                                              _p, _sz, _p]),
    "fp8_quantize_per_group_noalloc": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _i32, _p,
                                                      _i64, _p, _p]),
    "mx_gemm": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p, _i64, _i64, _i64, _i64, _i64,
                               _p, _i64, ctypes.c_int, ctypes.c_int, _p]),
    "fp8_gemm_per_tensor": (ctypes.c_int, [_p, _p, _i64, _p, _p, _i64, _i64, _i64, _i64,
                                           _p, _i64, ctypes.c_int, ctypes.c_int, _p]),
    "fp8_gemm_per_tensor_amax": (ctypes.c_int, [_p, _p, _i64, _p, _p, _i64, _i64, _i64, _i64,
                                                _p, _i64, ctypes.c_int, ctypes.c_int, _p, _p]),
    "mx_grouped_gemm": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p, _i64, _i64, _i64, _i64, _p, _i32,
                                       _i64, _i64, _i64, _p, _i64, ctypes.c_int,
                                       ctypes.c_int, _p]),
    "mx_grouped_gemm_swiglu": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p, _i64, _i64, _i64,
                                              _i64, _p, _i32, _i64, _i64, _i64, _p, _i64, _p,
                                              _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _p,
                                              _p]),
    "fp8_grouped_gemm_per_group_swiglu": (ctypes.c_int, [_p, _p, _i64, _p, _p, _i64, _i64, _p,
                                                         _i32, _i64, _i64, _i64, _p, _i64, _p,
                                                         _i64, _p, _p]),
    "fp8_quantize_per_group_amax": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _i32, _p, _p,
                                                   _i64, _p, _p, _sz, _p]),
    "fp8_quantize_per_group_colwise_amax": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _i32, _p,
                                                           _p, _i64, _i64, _p, _p, _p, _sz,
                                                           _p]),
    "fp8_quantize_blockwise_act": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p]),
    "fp8_quantize_blockwise_weight": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _i64, _p, _i64,
                                                     _p]),
    "fp8_gemm_blockwise": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p, _i64, _i64, _i64, _i64,
                                          _i64, _p, _i64, ctypes.c_int, ctypes.c_int, _p]),
    "fp8_quantize_per_group_dual": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _i32, _p, _p, _i64,
                                                   _p, _i64, _i64, _p, _p, _p, _sz, _p]),
    "fp8_quantize_per_group_colwise": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _i32, _p, _i64,
                                                      _i64, _p, _p, _p, _sz, _p]),
    "fp8_grouped_gemm_wgrad_per_group": (ctypes.c_int, [_p, _p, _i64, _p, _p, _i64, _p, _i32,
                                                        _i64, _i64, _p, _i64, ctypes.c_int,
                                                        ctypes.c_int, _p]),
    "fp8_grouped_gemm_per_group": (ctypes.c_int, [_p, _p, _i64, _p, _p, _i64, _i64, _p, _i32,
                                                  _i64, _i64, _i64, _p, _i64, ctypes.c_int,
                                                  ctypes.c_int, _p]),
    "mx_grouped_gemm_wgrad": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p, _i64, _i64, _p,
                                             _i32, _i64, _i64, _p, _i64, ctypes.c_int,
                                             ctypes.c_int, _p]),
    "mxq_workspace_size": (_sz, [ctypes.c_int, _i64, _i64, _i64, _i64]),
    "mxq_validate_offsets": (ctypes.c_int, [_p, _i32, _i64, _p]),
}

EXPORTS = tuple(_SIGS)

_lib = None


class MxqError(RuntimeError):
    pass


def load(path=LIB_PATH):
    """Load libmxq.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise MxqError(f"{path} is missing: build it with "
                           "`python -m block_quant_gemm_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def _check(status):
    if status != 0:
        msg = load().mxq_status_string(status).decode()
        raise MxqError(f"libmxq error {status}: {msg}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _bf16_bits(x):
    if x.dtype == torch.bfloat16:
        return x
    if x.dtype in (torch.int16, torch.uint16):
        return x
    raise TypeError("expected a bfloat16 tensor (or its 16-bit patterns)")


# ---------------------------------------------------------------------------
# quantization
# ---------------------------------------------------------------------------

def _scale_buffer(rows, cols, device):
    """[rows, cols] uint8 view of storage whose row stride is a multiple of 16
    bytes: the GEMMs read such scales in 16-byte windows (any stride works,
    byte by byte, more slowly)."""
    ld = (cols + 15) // 16 * 16
    return torch.empty((rows, ld), dtype=torch.uint8, device=device)[:, :cols]


def mx_quantize_rowwise(x, q=None, scale=None):
    """Row-wise (1x32) MX quantization of a BF16 [M, K] matrix.

    Returns (codes uint8 [M, K], scales uint8 [M, K/32])."""
    x = _bf16_bits(x)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = _scale_buffer(M, K // 32, x.device)
    _check(load().mx_quantize_rowwise(_ptr(x), M, K, x.stride(0), _ptr(q), q.stride(0),
                                      _ptr(scale), scale.stride(0), _stream()))
    return q, scale


def mx_quantize_rowwise_batch(xs):
    """Row-wise MX quantization of several BF16 matrices in one launch (e.g. a
    Linear's input and weight).  Returns [(codes, scales), ...] as
    mx_quantize_rowwise would for each."""
    xs = [_bf16_bits(x) for x in xs]
    outs, items = [], (RowwiseItem * len(xs))()
    for i, x in enumerate(xs):
        M, K = x.shape
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        scale = _scale_buffer(M, K // 32, x.device)
        items[i] = RowwiseItem(_ptr(x), M, K, x.stride(0), _ptr(q), q.stride(0), _ptr(scale),
                               scale.stride(0))
        outs.append((q, scale))
    _check(load().mx_quantize_rowwise_batch(items, len(xs), _stream()))
    return outs


def colwise_capacity(M, E=None):
    """Output columns that hold any padding of M rows over E groups, rounded
    up to a multiple of 128."""
    need = M + 31 * E if E else (M + 31) // 32 * 32
    return (need + 127) // 128 * 128


def mx_quantize_colwise(x, offsets=None, M_cap=None, qT=None, scaleT=None,
                        offsets_padded=None):
    """Column-wise (32x1) MX quantization, transposed: returns
    (codesT uint8 [K, M_cap], scalesT uint8 [K, M_cap/32], offsets_padded or None).

    With ``offsets`` (int64 [E+1] on the device) each group of rows is padded
    to a multiple of 32 with zeros; ``offsets_padded`` receives the padded
    group starts."""
    x = _bf16_bits(x)
    M, K = x.shape
    E = 0 if offsets is None else offsets.numel() - 1
    if M_cap is None:
        M_cap = colwise_capacity(M, E or None)
    if qT is None:
        qT = torch.empty((K, M_cap), dtype=torch.uint8, device=x.device)
    if scaleT is None:
        scaleT = _scale_buffer(K, M_cap // 32, x.device)
    if offsets is not None and offsets_padded is None:
        offsets_padded = torch.empty(E + 1, dtype=torch.int64, device=x.device)
    _check(load().mx_quantize_colwise(_ptr(x), M, K, x.stride(0), _ptr(offsets), E,
                                      _ptr(qT), qT.stride(0), M_cap, _ptr(scaleT),
                                      scaleT.stride(0), _ptr(offsets_padded), _stream()))
    return qT, scaleT, offsets_padded


def mx_quantize_dual(x, offsets=None, M_cap=None, q=None, scale=None, qT=None, scaleT=None,
                     offsets_padded=None):
    """Row-wise and (grouped) column-wise MX quantization from one read of x.

    Returns (codes [M, K], scales [M, K/32], codesT [K, M_cap],
    scalesT [K, M_cap/32], offsets_padded or None), each equal to what
    mx_quantize_rowwise / mx_quantize_colwise return."""
    x, E, M_cap, q, scale, qT, scaleT, offsets_padded = _dual_outputs(
        x, offsets, M_cap, q, scale, qT, scaleT, offsets_padded)
    M, K = x.shape
    _check(load().mx_quantize_dual(_ptr(x), M, K, x.stride(0), _ptr(offsets), E, _ptr(q),
                                   q.stride(0), _ptr(scale), scale.stride(0), _ptr(qT),
                                   qT.stride(0), M_cap, _ptr(scaleT), scaleT.stride(0),
                                   _ptr(offsets_padded), _stream()))
    return q, scale, qT, scaleT, offsets_padded


def _dual_outputs(x, offsets, M_cap, q, scale, qT, scaleT, offsets_padded):
    x = _bf16_bits(x)
    M, K = x.shape
    E = 0 if offsets is None else offsets.numel() - 1
    if M_cap is None:
        M_cap = colwise_capacity(M, E or None)
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = _scale_buffer(M, K // 32, x.device)
    if qT is None:
        qT = torch.empty((K, M_cap), dtype=torch.uint8, device=x.device)
    if scaleT is None:
        scaleT = _scale_buffer(K, M_cap // 32, x.device)
    if offsets is not None and offsets_padded is None:
        offsets_padded = torch.empty(E + 1, dtype=torch.int64, device=x.device)
    return x, E, M_cap, q, scale, qT, scaleT, offsets_padded


def mx_quantize_dual_batch(items):
    """Dual-axis MX quantization of several BF16 matrices in one launch (e.g.
    an expert product's activation and its stacked weights).  items: a list of
    (x, offsets) pairs, offsets None for one group.  Returns one
    (codes, scales, codesT, scalesT, offsets_padded) tuple per item, as
    mx_quantize_dual would."""
    outs, arr = [], (DualItem * len(items))()
    for i, (x, offsets) in enumerate(items):
        x, E, M_cap, q, scale, qT, scaleT, poff = _dual_outputs(
            x, offsets, None, None, None, None, None, None)
        M, K = x.shape
        arr[i] = DualItem(_ptr(x), M, K, x.stride(0), _ptr(offsets), E, _ptr(q), q.stride(0),
                          _ptr(scale), scale.stride(0), _ptr(qT), qT.stride(0), M_cap,
                          _ptr(scaleT), scaleT.stride(0), _ptr(poff))
        outs.append((x, q, scale, qT, scaleT, poff))
    _check(load().mx_quantize_dual_batch(arr, len(items), _stream()))
    return [o[1:] for o in outs]


def workspace_size(op, n, a1=0, a2=0, a3=0):
    return int(load().mxq_workspace_size(op, n, a1, a2, a3))


def fp8_quantize_per_tensor(x, q=None, scale=None, workspace=None):
    """Per-tensor current-scaling E4M3.  Returns (codes uint8, scale float32 [1])."""
    x = _bf16_bits(x)
    n = x.numel()
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    ws = workspace_size(WS_PER_TENSOR, n)
    if workspace is None:
        workspace = torch.empty(max(ws, 4), dtype=torch.uint8, device=x.device)
    _check(load().fp8_quantize_per_tensor(_ptr(x), n, _ptr(q), _ptr(scale), _ptr(workspace),
                                          workspace.numel(), _stream()))
    return q, scale


def fp8_quantize_per_tensor_amax(x, amax, q=None, scale=None):
    """fp8_quantize_per_tensor with the amax given (float32 [1] on the device),
    e.g. from fp8_gemm_per_tensor_amax.  Returns (codes uint8, scale float32 [1])."""
    x = _bf16_bits(x)
    n = x.numel()
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(load().fp8_quantize_per_tensor_amax(_ptr(x), n, _ptr(amax), _ptr(q), _ptr(scale),
                                               _stream()))
    return q, scale


def fp8_quantize_per_group(x, offsets, q=None, scales=None, workspace=None):
    """Per-group (per-expert) current-scaling E4M3 of a BF16 [M, K] matrix
    whose rows [offsets[e], offsets[e+1]) form group e (offsets int64 [E+1]
    on the device).  Returns (codes uint8 [M, K], scales float32 [E])."""
    x = _bf16_bits(x)
    M, K = x.shape
    E = offsets.numel() - 1
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(E, dtype=torch.float32, device=x.device)
    ws = workspace_size(WS_PER_GROUP, M, E)
    if workspace is None:
        workspace = torch.empty(max(ws, 4), dtype=torch.uint8, device=x.device)
    _check(load().fp8_quantize_per_group(_ptr(x), M, K, x.stride(0), _ptr(offsets), E, _ptr(q),
                                         q.stride(0), _ptr(scales), _ptr(workspace),
                                         workspace.numel(), _stream()))
    return q, scales


def fp8_quantize_per_group_noalloc(x, offsets, q, scales):
    """fp8_quantize_per_group with the library's own per-GPU scratch instead of
    a workspace: q uint8 [M, K] and scales float32 [E] are the caller's."""
    x = _bf16_bits(x)
    M, K = x.shape
    E = offsets.numel() - 1
    _check(load().fp8_quantize_per_group_noalloc(_ptr(x), M, K, x.stride(0), _ptr(offsets), E,
                                                 _ptr(q), q.stride(0), _ptr(scales), _stream()))
    return q, scales


def fp8_quantize_per_group_colwise(x, offsets, M_cap=None, qT=None, scales=None,
                                   offsets_padded=None, workspace=None):
    """Transposed copy of fp8_quantize_per_group: returns (codesT uint8
    [K, M_cap] with each group padded to 32 columns, scales float32 [E],
    offsets_padded int64 [E+1])."""
    x = _bf16_bits(x)
    M, K = x.shape
    E = offsets.numel() - 1
    if M_cap is None:
        M_cap = colwise_capacity(M, E)
    if qT is None:
        qT = torch.empty((K, M_cap), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(E, dtype=torch.float32, device=x.device)
    if offsets_padded is None:
        offsets_padded = torch.empty(E + 1, dtype=torch.int64, device=x.device)
    ws = workspace_size(WS_PER_GROUP, M, E)
    if workspace is None:
        workspace = torch.empty(max(ws, 4), dtype=torch.uint8, device=x.device)
    _check(load().fp8_quantize_per_group_colwise(_ptr(x), M, K, x.stride(0), _ptr(offsets), E,
                                                 _ptr(qT), qT.stride(0), M_cap, _ptr(scales),
                                                 _ptr(offsets_padded), _ptr(workspace),
                                                 workspace.numel(), _stream()))
    return qT, scales, offsets_padded


def fp8_quantize_per_group_dual(x, offsets, amax=None, M_cap=None, q=None, qT=None, scales=None,
                                offsets_padded=None, workspace=None):
    """Both per-group copies in one encoding pass (``amax``: the groups'
    amaxes, float32 [E], to skip the amax pass).  Returns (codes uint8
    [M, K], codesT uint8 [K, M_cap], scales float32 [E], offsets_padded
    int64 [E+1])."""
    x = _bf16_bits(x)
    M, K = x.shape
    E = offsets.numel() - 1
    if M_cap is None:
        M_cap = colwise_capacity(M, E)
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if qT is None:
        qT = torch.empty((K, M_cap), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(E, dtype=torch.float32, device=x.device)
    if offsets_padded is None:
        offsets_padded = torch.empty(E + 1, dtype=torch.int64, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(workspace_size(WS_PER_GROUP, 0 if amax is not None else M, E),
                                    4), dtype=torch.uint8, device=x.device)
    _check(load().fp8_quantize_per_group_dual(
        _ptr(x), M, K, x.stride(0), _ptr(offsets), E, _ptr(amax), _ptr(q), q.stride(0), _ptr(qT),
        qT.stride(0), M_cap, _ptr(scales), _ptr(offsets_padded), _ptr(workspace),
        workspace.numel(), _stream()))
    return q, qT, scales, offsets_padded


def fp8_quantize_per_group_amax(x, offsets, amax, q=None, scales=None, workspace=None):
    """fp8_quantize_per_group with the group amaxes given (float32 [E] on the
    device, e.g. from fp8_grouped_gemm_per_group_swiglu): no pass over x for
    them.  Returns (codes uint8 [M, K], scales float32 [E])."""
    x = _bf16_bits(x)
    M, K = x.shape
    E = offsets.numel() - 1
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(E, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(workspace_size(WS_PER_GROUP, 0, E), 4), dtype=torch.uint8,
                                device=x.device)
    _check(load().fp8_quantize_per_group_amax(_ptr(x), M, K, x.stride(0), _ptr(offsets), E,
                                              _ptr(amax), _ptr(q), q.stride(0), _ptr(scales),
                                              _ptr(workspace), workspace.numel(), _stream()))
    return q, scales


def fp8_quantize_per_group_colwise_amax(x, offsets, amax, M_cap=None, qT=None, scales=None,
                                        offsets_padded=None, workspace=None):
    """fp8_quantize_per_group_colwise with the group amaxes given.  Returns
    (codesT uint8 [K, M_cap], scales float32 [E], offsets_padded int64 [E+1])."""
    x = _bf16_bits(x)
    M, K = x.shape
    E = offsets.numel() - 1
    if M_cap is None:
        M_cap = colwise_capacity(M, E)
    if qT is None:
        qT = torch.empty((K, M_cap), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(E, dtype=torch.float32, device=x.device)
    if offsets_padded is None:
        offsets_padded = torch.empty(E + 1, dtype=torch.int64, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(workspace_size(WS_PER_GROUP, 0, E), 4), dtype=torch.uint8,
                                device=x.device)
    _check(load().fp8_quantize_per_group_colwise_amax(
        _ptr(x), M, K, x.stride(0), _ptr(offsets), E, _ptr(amax), _ptr(qT), qT.stride(0), M_cap,
        _ptr(scales), _ptr(offsets_padded), _ptr(workspace), workspace.numel(), _stream()))
    return qT, scales, offsets_padded


# ---------------------------------------------------------------------------
# GEMMs
# ---------------------------------------------------------------------------

def _out(M, N, out_dtype, device, c):
    if c is not None:
        return c
    dt = torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32
    return torch.empty((M, N), dtype=dt, device=device)


def mx_gemm(a, a_scale, b, b_scale, out_dtype=OUT_BF16, accum=ACC_MFMA_FP8, c=None):
    """C[M, N] = A[M, K] · B[N, K]ᵀ on MX operands (codes + E8M0 scales)."""
    M, K = a.shape
    N = b.shape[0]
    c = _out(M, N, out_dtype, a.device, c)
    _check(load().mx_gemm(_ptr(a), _ptr(a_scale), a.stride(0), a_scale.stride(0),
                          _ptr(b), _ptr(b_scale), b.stride(0), b_scale.stride(0),
                          M, N, K, _ptr(c), c.stride(0), out_dtype, accum, _stream()))
    return c


def fp8_gemm_per_tensor(a, a_scale, b, b_scale, out_dtype=OUT_BF16, accum=ACC_MFMA_FP8,
                        c=None):
    """C = s_a * s_b * (Q_a · Q_bᵀ); a_scale, b_scale: float32 [1] on the device."""
    M, K = a.shape
    N = b.shape[0]
    c = _out(M, N, out_dtype, a.device, c)
    _check(load().fp8_gemm_per_tensor(_ptr(a), _ptr(a_scale), a.stride(0), _ptr(b),
                                      _ptr(b_scale), b.stride(0), M, N, K, _ptr(c),
                                      c.stride(0), out_dtype, accum, _stream()))
    return c


def fp8_gemm_per_tensor_amax(a, a_scale, b, b_scale, out_dtype=OUT_BF16,
                             accum=ACC_MFMA_FP8, c=None, c_amax=None):
    """fp8_gemm_per_tensor that also returns max |C| (float32 [1], from the
    epilogue): (C, amax)."""
    M, K = a.shape
    N = b.shape[0]
    c = _out(M, N, out_dtype, a.device, c)
    if c_amax is None:
        c_amax = torch.empty(1, dtype=torch.float32, device=a.device)
    _check(load().fp8_gemm_per_tensor_amax(_ptr(a), _ptr(a_scale), a.stride(0), _ptr(b),
                                           _ptr(b_scale), b.stride(0), M, N, K, _ptr(c),
                                           c.stride(0), out_dtype, accum, _ptr(c_amax),
                                           _stream()))
    return c, c_amax


def mx_grouped_gemm(a, a_scale, b, b_scale, offsets, out_dtype=OUT_BF16,
                    accum=ACC_MFMA_FP8, c=None):
    """Variable-M grouped GEMM: rows [o_e, o_e+1) of A times B[e]ᵀ.

    a [M, K] codes with scales [M, K/32]; b [E, N, K] codes with scales
    [E, N, K/32], any strides (e.g. a view of column-quantized weights);
    offsets int64 [E+1] on the device."""
    M, K = a.shape
    E, N, _ = b.shape
    c = _out(M, N, out_dtype, a.device, c)
    _check(load().mx_grouped_gemm(_ptr(a), _ptr(a_scale), a.stride(0), a_scale.stride(0),
                                  _ptr(b), _ptr(b_scale), b.stride(1), b_scale.stride(1),
                                  b.stride(0), b_scale.stride(0), _ptr(offsets), E, M, N, K,
                                  _ptr(c), c.stride(0), out_dtype, accum, _stream()))
    return c


def mx_grouped_gemm_swiglu(a, a_scale, b, b_scale, offsets, gu=True, M_cap=None, hq=None,
                           hs=None, hqT=None, hsT=None, offsets_padded=None):
    """Gate/up grouped GEMM with SwiGLU and h's MX copies from the epilogue.

    a [M, K] codes with scales [M, K/32] (row copy of the expert inputs);
    b [E, 2F, K] gate_up codes with scales [E, 2F, K/32] (gate rows first);
    offsets int64 [E+1] on the device.  ``gu``: True allocates the BF16
    gate/up product [M, 2F], a tensor receives it, None/False skips it.
    Returns (gu or None, hq [M, F], hs [M, F/32], hqT [F, M_cap],
    hsT [F, M_cap/32], offsets_padded [E+1])."""
    M, K = a.shape
    E, N2, _ = b.shape
    F = N2 // 2
    dev = a.device
    if M_cap is None:
        M_cap = colwise_capacity(M, E)
    if gu is True:
        gu = torch.empty((M, 2 * F), dtype=torch.bfloat16, device=dev)
    elif gu is False:
        gu = None
    if hq is None:
        hq = torch.empty((M, F), dtype=torch.uint8, device=dev)
    if hs is None:
        hs = _scale_buffer(M, F // 32, dev)
    if hqT is None:
        hqT = torch.empty((F, M_cap), dtype=torch.uint8, device=dev)
    if hsT is None:
        hsT = _scale_buffer(F, M_cap // 32, dev)
    if offsets_padded is None:
        offsets_padded = torch.empty(E + 1, dtype=torch.int64, device=dev)
    _check(load().mx_grouped_gemm_swiglu(
        _ptr(a), _ptr(a_scale), a.stride(0), a_scale.stride(0), _ptr(b), _ptr(b_scale),
        b.stride(1), b_scale.stride(1), b.stride(0), b_scale.stride(0), _ptr(offsets), E, M, F,
        K, _ptr(gu), gu.stride(0) if gu is not None else 0, _ptr(hq), hq.stride(0), _ptr(hs),
        hs.stride(0), _ptr(hqT), hqT.stride(0), _ptr(hsT), hsT.stride(0), M_cap,
        _ptr(offsets_padded), _stream()))
    return gu, hq, hs, hqT, hsT, offsets_padded


def fp8_quantize_blockwise_act(x, q=None, scales=None):
    """1x128 blockwise E4M3 of a BF16 [M, K] matrix (K % 128 == 0).
    Returns (codes uint8 [M, K], scales float32 [M, K/128])."""
    x = _bf16_bits(x)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    _check(load().fp8_quantize_blockwise_act(_ptr(x), M, K, x.stride(0), _ptr(q), q.stride(0),
                                             _ptr(scales), scales.stride(0), _stream()))
    return q, scales


def fp8_quantize_blockwise_weight(w, q=None, scales=None):
    """128x128 blockwise E4M3 of a BF16 [N, K] weight (K % 128 == 0).
    Returns (codes uint8 [N, K], scales float32 [ceil(N/128), K/128])."""
    w = _bf16_bits(w)
    N, K = w.shape
    if q is None:
        q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32, device=w.device)
    _check(load().fp8_quantize_blockwise_weight(_ptr(w), N, K, w.stride(0), _ptr(q), q.stride(0),
                                                _ptr(scales), scales.stride(0), _stream()))
    return q, scales


def fp8_gemm_blockwise(a, a_scales, b, b_scales, out_dtype=OUT_BF16, accum=ACC_MFMA_FP8,
                       c=None):
    """C = A·Bᵀ on blockwise operands (1x128 A blocks, 128x128 B blocks)."""
    M, K = a.shape
    N = b.shape[0]
    c = _out(M, N, out_dtype, a.device, c)
    _check(load().fp8_gemm_blockwise(_ptr(a), _ptr(a_scales), a.stride(0), a_scales.stride(0),
                                     _ptr(b), _ptr(b_scales), b.stride(0), b_scales.stride(0),
                                     M, N, K, _ptr(c), c.stride(0), out_dtype, accum, _stream()))
    return c


def fp8_grouped_gemm_per_group_swiglu(a, a_scales, b, b_scales, offsets, gu=True, h=None,
                                      h_amax=None):
    """Per-group-scaled gate/up grouped GEMM with SwiGLU in the epilogue.

    a [M, K] and b [E, 2F, K] codes from fp8_quantize_per_group (gate rows
    first), scales float32 [E].  Returns (gu BF16 [M, 2F] or None, h BF16
    [M, F], h_amax float32 [E]: each group's largest |h|)."""
    M, K = a.shape
    E, N2, _ = b.shape
    F = N2 // 2
    dev = a.device
    if gu is True:
        gu = torch.empty((M, 2 * F), dtype=torch.bfloat16, device=dev)
    elif gu is False:
        gu = None
    if h is None:
        h = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
    if h_amax is None:
        h_amax = torch.empty(E, dtype=torch.float32, device=dev)
    _check(load().fp8_grouped_gemm_per_group_swiglu(
        _ptr(a), _ptr(a_scales), a.stride(0), _ptr(b), _ptr(b_scales), b.stride(1), b.stride(0),
        _ptr(offsets), E, M, F, K, _ptr(gu), gu.stride(0) if gu is not None else 0, _ptr(h),
        h.stride(0), _ptr(h_amax), _stream()))
    return gu, h, h_amax


def fp8_grouped_gemm_per_group(a, a_scales, b, b_scales, offsets, out_dtype=OUT_BF16,
                               accum=ACC_MFMA_FP8, c=None):
    """Variable-M grouped GEMM with per-group FP32 scales: rows [o_e, o_e+1)
    of C are a_scales[e] * b_scales[e] * (Q_a[rows] · Q_b[e]ᵀ).  a [M, K] and
    b [E, N, K] codes from fp8_quantize_per_group; scales float32 [E]."""
    M, K = a.shape
    E, N, _ = b.shape
    c = _out(M, N, out_dtype, a.device, c)
    _check(load().fp8_grouped_gemm_per_group(_ptr(a), _ptr(a_scales), a.stride(0), _ptr(b),
                                             _ptr(b_scales), b.stride(1), b.stride(0),
                                             _ptr(offsets), E, M, N, K, _ptr(c), c.stride(0),
                                             out_dtype, accum, _stream()))
    return c


def expert_view(qT, sT, E, rows_per_expert):
    """[E, K, rows_per_expert] strided views of column-quantized weights.

    mx_quantize_colwise of a weight stack [E*R, K] with one group per expert
    (R rows each, R % 32 == 0) returns codes [K, E*R]; expert e's transposed
    weight is the column slice [:, e*R:(e+1)*R]."""
    K = qT.shape[0]
    R = rows_per_expert
    q = qT.as_strided((E, K, R), (R, qT.stride(0), 1))
    s = sT.as_strided((E, K, R // 32), (R // 32, sT.stride(0), 1))
    return q, s


def fp8_grouped_gemm_wgrad_per_group(at, a_scales, bt, b_scales, offsets_padded,
                                     out_dtype=OUT_BF16, accum=ACC_MFMA_FP8, c=None):
    """Per-group-scaled weight gradient: dW[e] = s_a[e] s_b[e] Aᵀ[:, group e] ·
    (Bᵀ[:, group e])ᵀ on fp8_quantize_per_group_colwise copies.  Returns dW [E, N, K]."""
    N = at.shape[0]
    K = bt.shape[0]
    E = offsets_padded.numel() - 1
    if c is None:
        dt = torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32
        c = torch.empty((E, N, K), dtype=dt, device=at.device)
    _check(load().fp8_grouped_gemm_wgrad_per_group(_ptr(at), _ptr(a_scales), at.stride(0),
                                                   _ptr(bt), _ptr(b_scales), bt.stride(0),
                                                   _ptr(offsets_padded), E, N, K, _ptr(c),
                                                   c.stride(1), out_dtype, accum, _stream()))
    return c


def mx_grouped_gemm_wgrad(at, at_scale, bt, bt_scale, offsets_padded, out_dtype=OUT_BF16,
                          accum=ACC_MFMA_FP8, c=None):
    """Variable-K grouped GEMM: dW[e] = Aᵀ[:, group e] · (Bᵀ[:, group e])ᵀ.

    at [N, T], bt [K, T] column-quantized codes with scales [N, T/32],
    [K, T/32]; offsets_padded int64 [E+1] (multiples of 32) on the device.
    Returns dW [E, N, K]."""
    N = at.shape[0]
    K = bt.shape[0]
    E = offsets_padded.numel() - 1
    if c is None:
        dt = torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32
        c = torch.empty((E, N, K), dtype=dt, device=at.device)
    _check(load().mx_grouped_gemm_wgrad(_ptr(at), _ptr(at_scale), at.stride(0),
                                        at_scale.stride(0), _ptr(bt), _ptr(bt_scale),
                                        bt.stride(0), bt_scale.stride(0),
                                        _ptr(offsets_padded), E, N, K, _ptr(c),
                                        c.stride(1), out_dtype, accum, _stream()))
    return c


def validate_offsets(offsets, M):
    """Synchronizing check of device offsets (debug aid)."""
    _check(load().mxq_validate_offsets(_ptr(offsets), offsets.numel() - 1, M, _stream()))
