"""GPU parity of softmax with a temperature and of top-k-then-top-p sampling
from logits (the step before the filters: [Expl] "采样流水线究竟在计算什么").

Both sides compute p_i = float32(exp((z_i - m) / T) / S) with float64
exponentials and sums (oracle: math.fsum; GPU: a fixed-order float64 sum),
so a probability can differ only when e_i / S lies within ~1e-13 relative of
a float32 rounding boundary: at most one ulp, and rarely.
"""

import numpy as np
import pytest

import decode_step_sampling_amd as dss
import synthetic_inputs as si
from oracle import reference as ref
from gpu_util import gpu, host, pooled_chi_square, u64

pytestmark = pytest.mark.gpu


def _ulps(a, b):
    a = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def _check_softmax(got, logits, temps):
    diff_total = 0
    for r in range(logits.shape[0]):
        ok, p = ref.softmax_row(logits[r], temps[r])
        assert ok
        d = _ulps(got[r], p)
        assert d.max() <= 1, (r, int(d.max()))
        diff_total += int((d != 0).sum())
    assert diff_total <= max(2, logits.size // 100000), diff_total


@pytest.mark.parametrize("rows,vocab,sigma", [(4, 32000, 3.0), (64, 151936, 2.0)])
def test_softmax_parity(rows, vocab, sigma):
    rng = np.random.default_rng(7)
    logits = si.logits_rows(rng, rows, vocab, sigma)
    temps = rng.uniform(0.5, 1.5, size=rows).astype(np.float32)
    got = host(dss.softmax(gpu(logits), gpu(temps)))
    _check_softmax(got, logits, temps)
    for T in (0.25, 1.0, 3.0):       # one scalar temperature for every row
        got = host(dss.softmax(gpu(logits), T))
        _check_softmax(got, logits, np.full(rows, T, dtype=np.float32))


@pytest.mark.parametrize("vocab", [1, 3, 1000, 4097, 32000])
def test_softmax_ragged_in_place_and_streaming(vocab):
    rng = np.random.default_rng(vocab)
    logits = si.logits_rows(rng, 3, vocab, 2.0)
    temps = np.array([0.7, 1.0, 2.5], dtype=np.float32)
    for flags in (0, dss.DSS_FLAG_STREAMING):
        _check_softmax(host(dss.softmax(gpu(logits), gpu(temps), flags=flags)), logits, temps)
    x = gpu(logits)
    dss.softmax(x, gpu(temps), out=x)                       # in place
    _check_softmax(host(x), logits, temps)


def test_softmax_invalid_rows_and_temperatures():
    V = 4096
    rng = np.random.default_rng(3)
    base = si.logits_rows(rng, 1, V, 2.0)[0]
    rows = np.stack([base] * 7)
    rows[0, 5] = np.nan
    rows[1, 9] = np.inf
    rows[2, :] = -np.inf
    rows[3, 100:200] = -np.inf                              # valid: those get probability 0
    temps = np.array([1.0, 1.0, 1.0, 1.0, 0.0, -2.0, np.nan], dtype=np.float32)
    for flags in (0, dss.DSS_FLAG_STREAMING):
        out, status = dss.softmax(gpu(rows), gpu(temps), return_status=True, flags=flags)
        out, status = host(out), host(status)
        assert list(status) == [1, 1, 1, 0, 1, 1, 1]
        for r in (0, 1, 2, 4, 5, 6):
            assert np.isnan(out[r]).all()
        assert (out[3, 100:200] == 0).all()
        _check_softmax(out[3:4], rows[3:4], temps[3:4])


@pytest.fixture(scope="module")
def small_logits():
    rng = np.random.default_rng(20261202)
    return si.logits_rows(rng, 4, 32000, 3.0)


@pytest.mark.parametrize("order", ["top_k_first", "joint"])
def test_sampling_from_logits_chi_square(small_logits, order):
    logits = small_logits
    rows, V = logits.shape
    T = 0.7
    draws = 20000
    idx = np.repeat(np.arange(rows, dtype=np.int32), draws)
    s, v = dss.top_k_top_p_sampling_from_logits(gpu(logits), 50, 0.9, T, indices=gpu(idx),
                                                seed=99, offset=4, filter_apply_order=order,
                                                return_valid=True)
    s, v = host(s), host(v)
    assert (v == 1).all()
    op = "top_k_top_p" if order == "top_k_first" else "top_k_top_p_joint"
    for r in range(rows):
        ok, p = ref.softmax_row(logits[r], T)
        valid, tau = ref.threshold(p, op, k=50, p=np.float32(0.9))
        assert ok and valid
        sup = ref.support_mask(p, tau)
        got = s[r * draws:(r + 1) * draws]
        assert sup[got].all(), "draw outside the kept set"
        counts = np.bincount(got, minlength=V)
        pval, tvd, cells = pooled_chi_square(counts[sup], ref.target_distribution(p, tau)[sup])
        assert pval > 1e-3, (r, pval, tvd, cells)


def test_sampling_from_logits_full_size_support():
    """B=64, V=151936 logits N(0, 2^2), per-row k and p, per-row temperatures:
    every draw valid and inside the kept set of the oracle's probabilities."""
    w = si.renorm()
    rng = np.random.default_rng(11)
    logits = si.logits_rows(rng, 64, 151936, 2.0)
    temps = rng.uniform(0.6, 1.4, size=64).astype(np.float32)
    supports = []
    for r in range(64):
        ok, p = ref.softmax_row(logits[r], temps[r])
        valid, tau = ref.threshold(p, "top_k_top_p", k=w["top_k"][r], p=w["top_p"][r])
        assert ok and valid
        supports.append(ref.support_mask(p, tau))
    L, K, Pp, Tt = gpu(logits), gpu(w["top_k"]), gpu(w["top_p"]), gpu(temps)
    seeds = u64(w["seeds"])
    for call in range(10):
        s, v, r_ = dss.top_k_top_p_sampling_from_logits(L, K, Pp, Tt, seed=seeds, offset=call,
                                                        return_valid=True, return_rounds=True)
        s, v = host(s), host(v)
        assert (v == 1).all()
        for r in range(64):
            assert supports[r][s[r]], (call, r)


def test_sampling_from_logits_invalid_rows():
    V = 2048
    rng = np.random.default_rng(5)
    logits = si.logits_rows(rng, 3, V, 2.0)
    logits[1, 7] = np.nan
    temps = np.array([1.0, 1.0, 0.0], dtype=np.float32)
    s, v = dss.top_k_top_p_sampling_from_logits(gpu(logits), 20, 0.8, gpu(temps), seed=1,
                                                return_valid=True)
    s, v = host(s), host(v)
    assert v[0] == 1 and s[0] >= 0
    assert list(v[1:]) == [0, 0] and list(s[1:]) == [-1, -1]


@pytest.mark.parametrize("vocab,flags", [(151936, dss.DSS_FLAG_STREAMING), (50257, 0),
                                         (151936, 0)])
def test_logits_call_leaves_the_shared_workspace_usable(vocab, flags):
    """A from-logits call writes its probabilities into the shared workspace;
    the control words and resident slots that later calls expect at zero
    must survive it (streaming or ragged shapes need no engine area of their
    own).  The fused from-probs call and top-p sampling on the same cached
    workspace afterwards must still give valid draws inside the kept sets."""
    rng = np.random.default_rng(vocab + flags)
    rows = 64
    logits = si.logits_rows(rng, rows, vocab, 2.0)
    kk = rng.integers(1, 1025, size=rows).astype(np.int32)
    pp = rng.uniform(0.5, 0.95, size=rows).astype(np.float32)
    s, v = dss.top_k_top_p_sampling_from_logits(gpu(logits), gpu(kk), gpu(pp), 1.0, seed=5,
                                                offset=0, return_valid=True, flags=flags)
    assert host(v).all()
    w = si.renorm(rows=64, vocab=151936)
    P = gpu(w["probs"])
    for off in range(3):
        s, v = dss.top_k_top_p_sampling_from_probs(P, gpu(w["top_k"]), gpu(w["top_p"]),
                                                   seed=u64(w["seeds"]), offset=off,
                                                   return_valid=True)
        s2, v2 = dss.top_p_sampling_from_probs(P, gpu(w["top_p"]), seed=u64(w["seeds"]),
                                               offset=off, return_valid=True)
        s, v, s2, v2 = host(s), host(v), host(s2), host(v2)
        assert v.all() and v2.all()
        for r in range(0, 64, 7):
            _, tau = ref.threshold(w["probs"][r], "top_k_top_p", k=w["top_k"][r],
                                   p=w["top_p"][r])
            assert ref.support_mask(w["probs"][r], tau)[s[r]]
            _, tau = ref.threshold(w["probs"][r], "top_p", p=w["top_p"][r])
            assert ref.support_mask(w["probs"][r], tau)[s2[r]]
