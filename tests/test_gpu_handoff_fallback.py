"""The split engine's hand-off checks, forced to fail from the host.

The split engine trusts same-XCD relaxed atomics and round-robin work-group
placement for its hand-off; each slice's header carries the output's
generation and the slice's XCD, and a merge that finds either wrong must not
use the published lists but compute the output with the in-kernel fallback.
dss_set_handoff_test(1) (a test hook of include/dss_hooks.h) makes every
check fail, so every kernel still exits normally: the outputs must then be
exactly the fallback's (for top-k sampling the exact passes, whose draw is
the oracle's CDF token; renormalisation and selection as the oracle), and
the next calls with normal checks must find the counters and generations
balanced.
"""

import numpy as np
import pytest

import decode_step_sampling_amd as dss
import synthetic_inputs as si
from oracle import philox as ph
from oracle import reference as ref
from gpu_util import gpu, host, u64

pytestmark = pytest.mark.gpu


class _Foreign:
    def __enter__(self):
        assert dss._lib.load().dss_set_handoff_test(1) == 0

    def __exit__(self, *exc):
        dss._lib.load().dss_set_handoff_test(0)


def _cdf_token(row, op, k, p, seed, offset):
    valid, tau = ref.threshold(row, op, k=k, p=p)
    assert valid
    return ref.CdfTable(row, ref.support_mask(row, tau)).draw(ph.draw_bits53(seed, offset, 0, 0))


@pytest.fixture(scope="module")
def headline():
    w = si.renorm()
    w["P"] = gpu(w["probs"])
    return w


def _headline_call(w, offset):
    B = w["probs"].shape[0]
    seeds = (np.arange(B, dtype=np.uint64) + np.uint64(3)) * np.uint64(0x9E3779B97F4A7C15)
    s, v = dss.top_k_top_p_sampling_from_probs(w["P"], gpu(w["top_k"]), gpu(w["top_p"]),
                                               seed=u64(seeds), offset=offset, return_valid=True)
    return host(s), host(v), seeds


def test_headline_shape_fallback_is_exact(headline):
    """B=64, V=151936 (W=4 slices per row, candidate lists): with every
    hand-off foreign, every token is the exact passes' draw, the oracle's CDF
    token over the kept set; afterwards the normal path draws inside the
    kept sets again."""
    w = headline
    with _Foreign():
        s, v, seeds = _headline_call(w, 11)
    assert (v == 1).all()
    for r in range(w["probs"].shape[0]):
        want = _cdf_token(w["probs"][r], "top_k_top_p", int(w["top_k"][r]), w["top_p"][r],
                          int(seeds[r]), 11)
        assert s[r] == want, (r, int(s[r]), want)
    for off in (12, 13):
        s, v, _ = _headline_call(w, off)
        assert (v == 1).all()
        for r in range(w["probs"].shape[0]):
            _, tau = ref.threshold(w["probs"][r], "top_k_top_p", k=int(w["top_k"][r]),
                                   p=w["top_p"][r])
            assert ref.support_mask(w["probs"][r], tau)[s[r]], (r, off)


def test_large_k_finishers_fallback_is_exact():
    """k above the split cap, 72 outputs (finishing work-groups): foreign
    headers make the finishers take the exact passes, and the normal calls
    before and after agree token for token with the oracle as well."""
    rng = np.random.default_rng(41)
    rows, V, n = 8, 32768, 72
    probs = si.softmax_rows(rng, rows, V, 2.0)
    ks = np.array([3000, 2049, 10000, 70000, 5000, 2500, 4096, 30000], dtype=np.int32)
    ps = np.array([0.7, 0.3, 0.95, 0.5, 0.99, 0.8, 0.6, 0.9], dtype=np.float32)
    idx = (np.arange(n) % rows).astype(np.int32)
    seeds = (np.arange(n, dtype=np.uint64) + np.uint64(19)) * np.uint64(0x9E3779B97F4A7C15)
    P = gpu(probs)
    tables = {}
    for i in range(rows):
        valid, tau = ref.threshold(probs[i], "top_k_top_p", k=int(ks[i]), p=ps[i])
        tables[i] = ref.CdfTable(probs[i], ref.support_mask(probs[i], tau))
    for off, foreign in ((1, False), (2, True), (3, False)):
        if foreign:
            with _Foreign():
                s, v = dss.top_k_top_p_sampling_from_probs(P, gpu(ks[idx]), gpu(ps[idx]),
                                                           indices=gpu(idx), seed=u64(seeds),
                                                           offset=off, return_valid=True)
        else:
            s, v = dss.top_k_top_p_sampling_from_probs(P, gpu(ks[idx]), gpu(ps[idx]),
                                                       indices=gpu(idx), seed=u64(seeds),
                                                       offset=off, return_valid=True)
        s, v = host(s), host(v)
        assert (v == 1).all()
        for j in range(n):
            want = tables[int(idx[j])].draw(ph.draw_bits53(int(seeds[j]), off, 0, 0))
            assert s[j] == want, (off, foreign, j, int(s[j]), want)


def test_renorm_and_selection_fallback(headline):
    """Top-k renormalisation and top-k selection with every hand-off
    foreign: the one-work-group fallbacks give the oracle's masks, values
    (1e-6) and selections exactly."""
    w = headline
    with _Foreign():
        out = host(dss.top_k_renorm_probs(w["P"], gpu(w["top_k"])))
        x = si.logits_rows(np.random.default_rng(9), 16, 151936, 2.0)
        vals, ids = dss.top_k(gpu(x), 100)
    for r in range(w["probs"].shape[0]):
        valid, expect = ref.top_k_renorm(w["probs"][r], w["top_k"][r])
        assert valid
        support = expect != 0
        assert np.array_equal(out[r] != 0, support), r
        rel = np.abs(out[r][support].astype(np.float64) - expect[support]) / expect[support]
        assert rel.max(initial=0.0) <= 1e-6, (r, rel.max())
    vals, ids = host(vals), host(ids)
    for r in range(x.shape[0]):
        ok, ev, ei = ref.top_k_select(x[r], 100)
        assert ok
        assert np.array_equal(ids[r], ei), r
        assert np.array_equal(vals[r].view(np.uint32), ev.view(np.uint32)), r
