"""GPU parity of top_k_renorm_probs, top_p_renorm_probs and top_k_mask_logits.

Kept-set masks must match the oracle bit-exactly; renormalised values within
1e-6 relative error (the tolerance the benchmark spec states); masked logits exactly.
"""

import numpy as np
import pytest

import decode_step_sampling_amd as dss
import synthetic_inputs as si
from oracle import reference as ref
from gpu_util import gpu, host

pytestmark = pytest.mark.gpu

RTOL = 1e-6
FLAG_SETS = [0, dss.DSS_FLAG_STREAMING]


def _check_renorm(got, row_in, valid, expect):
    assert valid
    support = expect != 0
    assert np.array_equal(got != 0, support), np.nonzero((got != 0) != support)[0][:10]
    rel = np.abs(got[support].astype(np.float64) - expect[support]) / expect[support]
    assert rel.max(initial=0.0) <= RTOL, rel.max()


@pytest.fixture(scope="module")
def renorm_workload():
    w = si.renorm()
    w["P"] = gpu(w["probs"])
    return w


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_top_p_renorm_full_size(renorm_workload, flags):
    w = renorm_workload
    out, status = dss.top_p_renorm_probs(w["P"], gpu(w["top_p"]), return_status=True,
                                         flags=flags)
    out, status = host(out), host(status)
    assert (status == 0).all()
    margins = []
    for r in range(w["probs"].shape[0]):
        margins.append(ref.top_p_boundary_margin(w["probs"][r], w["top_p"][r]))
        valid, expect = ref.top_p_renorm(w["probs"][r], w["top_p"][r])
        _check_renorm(out[r], w["probs"][r], valid, expect)
    # float64 masses decide every boundary when the margin exceeds ~1e-13
    assert min(margins) > 1e-12


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_top_k_renorm_full_size(renorm_workload, flags):
    w = renorm_workload
    out = host(dss.top_k_renorm_probs(w["P"], gpu(w["top_k"]), flags=flags))
    for r in range(w["probs"].shape[0]):
        valid, expect = ref.top_k_renorm(w["probs"][r], w["top_k"][r])
        _check_renorm(out[r], w["probs"][r], valid, expect)


def test_renorm_small_and_edge_parameters():
    w = si.small()
    probs = w["probs"]
    P = gpu(probs)
    for k in (1, 2, 50, 31999, 32000, 10**6):
        out = host(dss.top_k_renorm_probs(P, k))
        for r in range(probs.shape[0]):
            _check_renorm(out[r], probs[r], *ref.top_k_renorm(probs[r], k))
    for p in (0.0, 1e-6, 0.5, 0.9, 0.999, 1.0, 3.0):
        out = host(dss.top_p_renorm_probs(P, p))
        for r in range(probs.shape[0]):
            _check_renorm(out[r], probs[r], *ref.top_p_renorm(probs[r], p))


@pytest.mark.parametrize("p", [0.3, 0.95])
def test_top_p_dense_boundary_bins(p):
    """Near-uniform and slowly decaying rows put thousands of values into the
    bin where the top-p mass crosses p * Z (more than a work-group's key list
    holds), peaked rows put one: both ways of finding tau, for renormalisation
    and for sampling."""
    w = si.stress(rows=6, vocab=65536)
    probs = w["probs"]
    P = gpu(probs)
    out = host(dss.top_p_renorm_probs(P, p))
    for r in range(probs.shape[0]):
        _check_renorm(out[r], probs[r], *ref.top_p_renorm(probs[r], p))
    n = 2000
    idx = np.repeat(np.arange(probs.shape[0], dtype=np.int32), n)
    s = host(dss.top_p_sampling_from_probs(P, p, indices=gpu(idx), seed=5, offset=1))
    for r in range(probs.shape[0]):
        _, tau = ref.threshold(probs[r], "top_p", k=None, p=np.float32(p), min_p=None)
        support = ref.support_mask(probs[r], tau)
        got = s[r * n:(r + 1) * n]
        assert (got >= 0).all() and support[got].all(), r


@pytest.mark.parametrize("V", [1, 3, 7, 2049, 4101])
def test_renorm_ragged_and_in_place(V):
    rng = np.random.default_rng(V + 5)
    probs = rng.dirichlet(np.full(V, 0.4), size=5).astype(np.float32)
    probs[1, ::2] = 0.0
    if not probs[1].any():
        probs[1, -1] = 1.0
    probs[2, : max(1, V // 4)] = probs[2].max()          # ties
    k = max(1, V // 3)
    P = gpu(probs)
    out = host(dss.top_k_renorm_probs(P, k))
    for r in range(5):
        _check_renorm(out[r], probs[r], *ref.top_k_renorm(probs[r], k))
    P2 = gpu(probs)
    dss.top_p_renorm_probs(P2, 0.6, out=P2)              # in place
    out = host(P2)
    for r in range(5):
        _check_renorm(out[r], probs[r], *ref.top_p_renorm(probs[r], 0.6))


def test_renorm_invalid_rows():
    probs = np.full((5, 100), 0.01, dtype=np.float32)
    probs[1, 3] = np.nan
    probs[2, 4] = -0.5
    probs[3, :] = 0.0
    probs[4, 7] = np.inf
    P = gpu(probs)
    for fn, prm in ((dss.top_k_renorm_probs, 10), (dss.top_p_renorm_probs, 0.5)):
        out, st = fn(P, prm, return_status=True)
        out, st = host(out), host(st)
        assert list(st) == [0, 1, 1, 1, 1]
        assert np.isnan(out[1:]).all() and not np.isnan(out[0]).any()
    out, st = dss.top_k_renorm_probs(P, gpu(np.array([0, 3, 3, 3, 3], np.int32)),
                                     return_status=True)
    assert host(st)[0] == 1 and np.isnan(host(out)[0]).all()


def test_mask_logits():
    rng = np.random.default_rng(31)
    rows, V = 12, 32000
    logits = si.logits_rows(rng, rows, V)
    logits[1, :100] = logits[1].max()                    # ties at the top
    logits[2, ::5] = -np.inf
    logits[3, :] = np.float32(-3.0)
    logits[3, 10] = np.float32(-0.0)
    logits[3, 11] = np.float32(0.0)                      # -0.0 == +0.0
    logits[4, 5] = np.nan                                # invalid row
    logits[5, 9] = np.inf
    ks = np.array([1, 50, 3, 2, 10, 1, 1000, V, V + 5, 31999, 7, 12345], dtype=np.int32)
    L = gpu(logits)
    for flags in FLAG_SETS:
        out, st = dss.top_k_mask_logits(L, gpu(ks), return_status=True, flags=flags)
        out, st = host(out), host(st)
        for r in range(rows):
            valid, expect = ref.mask_logits_row(logits[r], ks[r])
            assert st[r] == (0 if valid else 1)
            if valid:
                assert np.array_equal(out[r], expect), r
            else:
                assert np.isnan(out[r]).all()


# Shapes for the split-row renorm / mask path (V % 4 == 0, V >= 1024): several
# slices per row, one slice per row (W = 1), and more rows than one launch
# chunk takes (2048).
@pytest.mark.parametrize("rows,V", [(3, 8192), (64, 16384), (300, 4096), (2100, 1024)])
def test_split_renorm_and_mask_edges(rows, V):
    rng = np.random.default_rng(rows * 7 + V)
    probs = rng.dirichlet(np.full(V, 0.3), size=rows).astype(np.float32)
    probs[0, : V // 8] = probs[0].max()                  # ties across the top-k boundary
    ks = rng.integers(1, 1500, size=rows).astype(np.int32)
    ks[0] = 200
    special = {}
    if rows > 6:
        probs[1, 5] = np.nan
        probs[2, 7] = -1e-3
        probs[3] = 0.0
        probs[4, 9] = np.inf
        ks[5] = 0                                         # invalid parameter
        ks[6] = 3000                                      # above the split engine's cap
        special = {1, 2, 3, 4, 5}
    P = gpu(probs)
    K = gpu(ks)
    out, st = dss.top_k_renorm_probs(P, K, return_status=True)
    out, st = host(out), host(st)
    P2 = gpu(probs)
    dss.top_k_renorm_probs(P2, K, out=P2)                # in place
    inplace = host(P2)
    for r in range(rows):
        valid, expect = ref.top_k_renorm(probs[r], ks[r])
        assert valid == (r not in special), r
        assert st[r] == (0 if valid else 1), r
        if valid:
            _check_renorm(out[r], probs[r], valid, expect)
            assert np.array_equal(inplace[r], out[r]), r
        else:
            assert np.isnan(out[r]).all() and np.isnan(inplace[r]).all(), r

    logits = si.logits_rows(rng, rows, V)
    logits[0, : V // 8] = logits[0].max()                # ties at the top
    if rows > 6:
        logits[1, 3] = np.nan                             # invalid row
        logits[2, ::3] = -np.inf
        logits[3, 1] = np.inf
        logits[4, :] = np.float32(-2.0)
        logits[4, 10] = np.float32(-0.0)
        logits[4, 11] = np.float32(0.0)                   # -0.0 == +0.0
    L = gpu(logits)
    out, st = dss.top_k_mask_logits(L, K, return_status=True)
    out, st = host(out), host(st)
    for r in range(rows):
        valid, expect = ref.mask_logits_row(logits[r], ks[r])
        assert st[r] == (0 if valid else 1), r
        if valid:
            assert np.array_equal(out[r], expect), r
        else:
            assert np.isnan(out[r]).all(), r
