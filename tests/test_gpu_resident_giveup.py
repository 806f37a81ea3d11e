"""The resident engine's bounded wait, forced to give up from the host.

dss_set_spin_limit(0) (a test hook of include/dss_hooks.h) makes every row
barrier give up on arrival, so every kernel still exits normally.  Every
output of that call must come out invalid and every slot it used be marked
broken; later calls with the normal limit must report the outputs on those
slots invalid instead of counting stale arrivals, and zeroing the workspace
makes every output correct again.
"""

import numpy as np
import pytest

import decode_step_sampling_amd as dss
import synthetic_inputs as si
from oracle import reference as ref
from gpu_util import gpu, host, u64

pytestmark = pytest.mark.gpu


def _check(w, s, v, allowed_invalid):
    for r in range(64):
        if v[r] == 0:
            assert s[r] == -1 and r in allowed_invalid, r
        else:
            _, tau = ref.threshold(w["probs"][r], "top_p", p=w["top_p"][r])
            assert ref.support_mask(w["probs"][r], tau)[s[r]], r


def test_resident_wait_gives_up_and_poisons_only_its_blocks():
    w = si.renorm()
    P, p, seeds = gpu(w["probs"]), gpu(w["top_p"]), u64(w["seeds"])
    lib = dss._lib.load()
    dss.reset_workspace()
    # a clean call first (the cached workspace exists and is zero)
    s, v = dss.top_p_sampling_from_probs(P, p, seed=seeds, offset=1, return_valid=True)
    assert host(v).all()
    assert dss.workspace_status() == []
    try:
        assert lib.dss_set_spin_limit(0) == 0
        s, v = dss.top_p_sampling_from_probs(P, p, seed=seeds, offset=2, return_valid=True)
        s, v = host(s), host(v)
    finally:
        lib.dss_set_spin_limit(2**64 - 1)
    broken = dss.workspace_status()
    # outputs 0..63 use slots 0..63 (one launch): every one gave up
    assert broken == list(range(64))
    assert not v.any() and (s == -1).all()
    # default limit again: outputs on broken blocks stay invalid, the rest are correct
    for off in (3, 4):
        s, v = dss.top_p_sampling_from_probs(P, p, seed=seeds, offset=off, return_valid=True)
        s, v = host(s), host(v)
        assert [r for r in range(64) if v[r] == 0] == [r for r in broken if r < 64]
        _check(w, s, v, set(broken))
    assert dss.workspace_status() == broken
    # zeroing the workspace clears the marks
    dss.reset_workspace()
    assert dss.workspace_status() == []
    s, v = dss.top_p_sampling_from_probs(P, p, seed=seeds, offset=5, return_valid=True)
    s, v = host(s), host(v)
    assert v.all()
    _check(w, s, v, set())
