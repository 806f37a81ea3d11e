"""Finishing work-groups of the split engine (per-output k above the
candidate cap, more slices than one wave of work-groups): the slices publish
histograms and leave, one work-group per output placed after every slice in
the grid waits for them and merges.

The wait is bounded; dss_set_spin_limit(0) (a test hook of
include/dss_hooks.h) makes every finisher give up at once and sample its
output with the exact streaming passes instead, so every kernel still exits
normally.  Those outputs must still be valid draws from their kept sets, and
later calls with the normal limit must find the arrival counters and
generations consistent (every output valid, inside its kept set, the same
tokens for the same seeds and offset).
"""

import numpy as np
import pytest

import decode_step_sampling_amd as dss
import synthetic_inputs as si
from oracle import reference as ref
from gpu_util import gpu, host, u64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hetero():
    w = si.hetero()
    w["P"] = gpu(w["probs"])
    return w


def _call(w, sel, offset):
    idx = w["indices"][sel]
    return dss.top_k_top_p_sampling_from_probs(
        w["P"], gpu(w["top_k"][idx]), gpu(w["top_p"][idx]), indices=gpu(idx),
        seed=u64(w["seeds"][sel]), offset=offset, return_valid=True)


def _check(w, sel, s, v, cache):
    assert (v == 1).all()
    for n, out in enumerate(sel):
        row = int(w["indices"][out])
        if row not in cache:
            valid, tau = ref.threshold(w["probs"][row], "top_k_top_p", k=w["top_k"][row],
                                       p=w["top_p"][row])
            assert valid
            cache[row] = ref.support_mask(w["probs"][row], tau)
        assert cache[row][s[n]], (out, row)


def test_finishers_give_up_and_later_calls_stay_consistent(hetero):
    w = hetero
    sel = np.nonzero(w["op_of_output"] == 0)[0]
    assert (w["top_k"][w["indices"][sel]] > 2048).sum() > 100  # most outputs take the path
    lib = dss._lib.load()
    cache = {}
    s0, v0 = _call(w, sel, 7)
    s0, v0 = host(s0), host(v0)
    _check(w, sel, s0, v0, cache)
    try:
        assert lib.dss_set_spin_limit(0) == 0
        s, v = _call(w, sel, 8)
        s, v = host(s), host(v)
    finally:
        lib.dss_set_spin_limit(2**64 - 1)
    _check(w, sel, s, v, cache)
    for off in (9, 7):
        s, v = _call(w, sel, off)
        s, v = host(s), host(v)
        _check(w, sel, s, v, cache)
    # the same seeds and offset as the first call: the same tokens
    assert np.array_equal(s, s0)
