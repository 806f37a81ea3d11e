"""GPU parity of softmax with a temperature and of top-k-then-top-p sampling
from logits (the step before the filters: [Expl] "采样流水线究竟在计算什么").

The softmax kernel and the oracle compute p_i = float32(exp((z_i - m) / T) /
S) with float64 exponentials and sums (oracle: math.fsum; GPU: a fixed-order
float64 sum), so a probability can differ only when e_i / S lies within
~1e-13 relative of a float32 rounding boundary: at most one ulp, and rarely.
Sampling from logits in the sequential order runs fused: the filters take
the weights w_i = float32(exp((z_i - m) / T)) without the normaliser
(oracle: softmax_weights, reading R21); the joint order, and outputs that
fall back, take the probabilities.
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


def _kept(logits_row, T, op, k, p, fused=True):
    """The oracle's kept set for sampling from logits: on the weights (the
    fused path) or on the probabilities (the joint order, fallbacks)."""
    ok, x = (ref.softmax_weights if fused else ref.softmax_row)(logits_row, T)
    assert ok
    valid, tau = ref.threshold(x, op, k=k, p=p)
    assert valid
    return x, tau, ref.support_mask(x, tau)


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
        p, tau, sup = _kept(logits[r], T, op, 50, np.float32(0.9), fused=order == "top_k_first")
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
    supports = [_kept(logits[r], temps[r], "top_k_top_p", w["top_k"][r], w["top_p"][r])[2]
                for r in range(64)]
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
    """A NaN or +inf logit, no finite logit, or a temperature that is not a
    finite positive number make the output invalid (-1, valid 0)."""
    V = 2048
    rng = np.random.default_rng(5)
    logits = si.logits_rows(rng, 6, V, 2.0)
    logits[1, 7] = np.nan
    logits[3, 99] = np.inf
    logits[4, :] = -np.inf
    temps = np.array([1.0, 1.0, 0.0, 1.0, 1.0, np.inf], dtype=np.float32)
    s, v = dss.top_k_top_p_sampling_from_logits(gpu(logits), 20, 0.8, gpu(temps), seed=1,
                                                return_valid=True)
    s, v = host(s), host(v)
    assert v[0] == 1 and s[0] >= 0
    assert list(v[1:]) == [0] * 5 and list(s[1:]) == [-1] * 5


def test_fused_logits_edge_rows():
    """The fused path (softmax inside the sampling pass) on rows that stress
    it, B=8, V=151936: masked (-inf) entries, a first stretch of -inf in
    every thread's first loads, one logit far above the rest (each thread's
    running reference is raised), a huge spread where most candidates'
    probabilities underflow to zero, a tiny temperature, and k above the
    split engine's cap (that output falls back to probabilities written for
    it, so its kept set is the probabilities').  Twenty calls: every draw
    valid and inside the oracle's kept set."""
    V, rows = 151936, 8
    rng = np.random.default_rng(23)
    logits = si.logits_rows(rng, rows, V, 2.0)
    logits[0, rng.choice(V, 5000, replace=False)] = -np.inf
    logits[1, :65536] = -np.inf
    logits[2, 123] = 300.0
    logits[3] *= 40.0
    temps = np.ones(rows, dtype=np.float32)
    temps[4] = 0.05
    k = np.array([50, 300, 10, 1000, 40, 5000, 2048, 1], dtype=np.int32)
    p = np.array([0.9, 0.95, 0.5, 0.99, 0.8, 0.7, 1.0, 0.3], dtype=np.float32)
    sup = [_kept(logits[r], temps[r], "top_k_top_p", k[r], p[r], fused=k[r] <= 2048)[2]
           for r in range(rows)]
    L, K, Pp, Tt = gpu(logits), gpu(k), gpu(p), gpu(temps)
    for call in range(20):
        s, v = dss.top_k_top_p_sampling_from_logits(L, K, Pp, Tt, seed=5, offset=call,
                                                    return_valid=True)
        s, v = host(s), host(v)
        assert (v == 1).all(), (call, v)
        for r in range(rows):
            assert sup[r][s[r]], (call, r, s[r])


def test_fused_logits_chi_square_full_size():
    """Distribution at the fused path's full-size launch (B=64, V=151936,
    W=4): 4000 calls of the batch, the draws of rows 0-7 (per-row k and p of
    the renorm workload, T = 0.8) against the oracle's p~ on the weights at
    alpha = 1e-3."""
    w = si.renorm()
    rng = np.random.default_rng(13)
    logits = si.logits_rows(rng, 64, 151936, 2.0)
    T = 0.8
    L, K, Pp = gpu(logits), gpu(w["top_k"]), gpu(w["top_p"])
    draws = 4000
    got = np.empty((draws, 8), dtype=np.int64)
    for c in range(draws):
        s = dss.top_k_top_p_sampling_from_logits(L, K, Pp, T, seed=77, offset=c)
        got[c] = host(s)[:8]
    for r in range(8):
        pr, tau, sup = _kept(logits[r], T, "top_k_top_p", w["top_k"][r], w["top_p"][r])
        assert sup[got[:, r]].all(), r
        counts = np.bincount(got[:, r], minlength=151936)
        pval, tvd, cells = pooled_chi_square(counts[sup], ref.target_distribution(pr, tau)[sup])
        assert pval > 1e-3, (r, pval, tvd, cells)


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
