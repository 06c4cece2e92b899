"""MX codes that are valid for values known only to lie in an interval.

A kernel that quantizes values it computed itself (an epilogue that
quantizes FP32 accumulators) cannot match an exact oracle bit for bit: its
values differ from the exact ones by the accumulation and evaluation error.
If every such value is known to lie in [lo, hi], the kernel's block scale
must be one that some amax in the block's amax interval gives, and each code
must lie between the codes of lo and hi at that scale (the shared exponent
and saturating round-to-nearest-even are both monotone).  Where lo == hi
the check is exact equality with the oracle.
"""

import numpy as np

from oracle.codec import E8M0_BIAS, e4m3_decode, e4m3_encode
from oracle.mx import BLOCK, block_shared_exponent


def mx_valid(codes, scales, lo, hi):
    """Check MX codes [R, C] and scales [R, C/32] against value bounds.

    lo, hi: float64 [R, C] with lo <= hi (finite).  Returns
    (ok_codes bool [R, C], ok_scales bool [R, C/32], unique bool [R, C]):
    unique marks elements whose scale and code the bounds fix exactly.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    assert np.all(lo <= hi)
    R, C = codes.shape
    nb = C // BLOCK
    mag_hi = np.maximum(np.abs(lo), np.abs(hi))
    mag_lo = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(lo), np.abs(hi)))
    amax_lo = mag_lo.reshape(R, nb, BLOCK).max(axis=2)
    amax_hi = mag_hi.reshape(R, nb, BLOCK).max(axis=2)
    e_lo, _ = block_shared_exponent(amax_lo)
    e_hi, _ = block_shared_exponent(amax_hi)
    e = scales.astype(np.int64) - E8M0_BIAS
    ok_scales = (scales != 0xFF) & (e >= e_lo) & (e <= e_hi)
    eb = np.repeat(e, BLOCK, axis=1)
    vmin = e4m3_decode(e4m3_encode(np.ldexp(lo, -eb)))
    vmax = e4m3_decode(e4m3_encode(np.ldexp(hi, -eb)))
    v = e4m3_decode(codes)
    with np.errstate(invalid="ignore"):
        ok_codes = (v >= vmin) & (v <= vmax) & ~np.isnan(v)
    unique = np.repeat(e_lo == e_hi, BLOCK, axis=1) & (vmin == vmax)
    return ok_codes, ok_scales, unique
