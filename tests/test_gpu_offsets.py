"""mxq_validate_offsets, the synchronizing check of a device offsets table
that the grouped calls take on trust: a valid table (empty groups included)
passes; a first offset other than 0, a last offset other than M and a
decreasing pair are each reported as MXQ_ERR_OFFSETS, with no kernel run.
Through the C ABI and through the binding."""

import ctypes

import numpy as np
import pytest

from block_quant_gemm_amd import mxq
from tests.gpu_helpers import say, to_dev

pytestmark = pytest.mark.gpu

ERR_OFFSETS = 7


def _status(offs, M, E=None):
    d = to_dev(np.asarray(offs, np.int64))
    E = len(offs) - 1 if E is None else E
    return mxq.load().mxq_validate_offsets(ctypes.c_void_p(d.data_ptr()), E, M, None)


@pytest.mark.parametrize("offs,M", [
    ([0, 300], 300),
    ([0, 0, 5, 5, 129, 129], 129),
    ([0, 0], 0),
    (list(np.cumsum([0] + [7] * 256)), 7 * 256),
])
def test_valid_tables_pass(offs, M):
    say(f"validate offsets E={len(offs) - 1} M={M}")
    assert _status(offs, M) == 0
    mxq.validate_offsets(to_dev(np.asarray(offs, np.int64)), M)


@pytest.mark.parametrize("offs,M", [
    ([1, 300], 300),              # does not start at 0
    ([0, 299], 300),              # does not end at M
    ([0, 10, 9, 300], 300),       # decreasing
    ([0, -1, 300], 300),          # negative
])
def test_bad_tables_reported(offs, M):
    say(f"validate bad offsets {offs} M={M}")
    assert _status(offs, M) == ERR_OFFSETS
    with pytest.raises(mxq.MxqError):
        mxq.validate_offsets(to_dev(np.asarray(offs, np.int64)), M)


def test_only_the_first_E_plus_1_entries_are_read():
    """E = 2 of a longer buffer: the entries past E + 1 are not looked at."""
    assert _status([0, 4, 9, -5, 77], 9, E=2) == 0
