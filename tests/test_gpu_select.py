"""GPU parity of top-k selection (values and indices) against the oracle:
bit-exact values and exact indices (values descending, equal values by
ascending index, -0.0 equal to +0.0; [Expl] "选择 top-k 值本身").

k <= 2048 on aligned rows of >= 1024 values runs the split engine (its
top-k set sorted); rows whose lists overflow (flat rows, huge tie groups)
fall back inside that kernel to the one-work-group selection, which also
serves k > 2048, unaligned rows and DSS_FLAG_STREAMING."""

import numpy as np
import pytest
import torch

import decode_step_sampling_amd as dss
import synthetic_inputs as si
from oracle import reference as ref
from gpu_util import gpu, host

pytestmark = pytest.mark.gpu


def _check(x, k, vals, idx, status=None):
    for r in range(x.shape[0]):
        ok, ev, ei = ref.top_k_select(x[r], k)
        if not ok:
            assert np.isnan(vals[r]).all() and (idx[r] == -1).all()
            if status is not None:
                assert status[r] == 1
            continue
        assert np.array_equal(idx[r], ei), (r, np.nonzero(idx[r] != ei)[0][:5])
        assert np.array_equal(vals[r].view(np.uint32), ev.view(np.uint32)), r
        if status is not None:
            assert status[r] == 0


@pytest.mark.parametrize("k", [1, 50, 1024, 2048, 2049, 4096])
def test_top_k_full_size_logits(k):
    x = si.logits_rows(np.random.default_rng(k), 64, 151936, 2.0)
    vals, idx = dss.top_k(gpu(x), k)
    _check(x, k, host(vals), host(idx))


@pytest.mark.parametrize("k", [1, 64, 257, 2048])
def test_top_k_split_and_streaming_agree(k):
    """The two engines on the same rows (every tie rule exercised by rows of
    few distinct values), bit for bit, and both against the oracle."""
    rng = np.random.default_rng(40 + k)
    x = (rng.integers(-50, 50, size=(16, 32768)) / 8.0).astype(np.float32)
    a = dss.top_k(gpu(x), k)
    b = dss.top_k(gpu(x), k, flags=dss.DSS_FLAG_STREAMING)
    for u, v in zip(a, b):
        assert np.array_equal(host(u).view(np.uint32), host(v).view(np.uint32))
    _check(x, k, host(a[0]), host(a[1]))


def test_top_k_probabilities():
    w = si.renorm(rows=8)
    vals, idx = dss.top_k(gpu(w["probs"]), 1000)
    _check(w["probs"], 1000, host(vals), host(idx))


@pytest.mark.parametrize("k", [1, 7, 500, 4096])
def test_top_k_ties(k):
    rng = np.random.default_rng(3 + k)
    x = (rng.integers(-4, 5, size=(6, 10000)) / 2.0).astype(np.float32)
    x[1] = 0.25                                   # one flat row: the first k indices
    x[2, ::3] = -0.0                              # signed zeros tie with +0.0
    x[3, 17] = np.inf
    x[3, 18] = -np.inf
    vals, idx, status = dss.top_k(gpu(x), k, return_status=True)
    _check(x, k, host(vals), host(idx), host(status))
    assert list(host(idx)[1][:5]) == list(range(min(k, 5)))


def test_top_k_invalid_rows():
    x = si.logits_rows(np.random.default_rng(1), 3, 2048, 2.0)
    x[1, 100] = np.nan
    vals, idx, status = dss.top_k(gpu(x), 64, return_status=True)
    _check(x, 64, host(vals), host(idx), host(status))
    assert list(host(status)) == [0, 1, 0]


@pytest.mark.parametrize("vocab", [1, 3, 4099])
def test_top_k_ragged_and_unaligned(vocab):
    rng = np.random.default_rng(vocab)
    x = si.logits_rows(rng, 3, vocab, 2.0)
    for k in sorted({1, min(vocab, 4096)}):
        vals, idx = dss.top_k(gpu(x), k)
        _check(x, k, host(vals), host(idx))
    if vocab > 4096:                              # above the selection cap: refused
        with pytest.raises(dss.DssError, match="unsupported"):
            dss.top_k(gpu(x), 4097)
    # rows read from a base one float past a 16-byte boundary
    big = torch.zeros(3 * vocab + 1, dtype=torch.float32, device="cuda:0")
    big[1:] = gpu(x.reshape(-1))
    view = big[1:].view(3, vocab)
    vals, idx = dss.top_k(view, 1)
    _check(x, 1, host(vals), host(idx))
