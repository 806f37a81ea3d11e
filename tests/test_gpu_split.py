"""GPU tests aimed at the split-row engine (top-k and top-k-then-top-p).

The engine reads each row once across W work-groups, hands the candidates
to the last one and runs the rejection loop there; it falls back to the
streaming engine when candidates overflow or k is above its cap.  Each test
picks shapes that force one of those paths and checks draws against the
oracle's kept set and distribution.
"""

import numpy as np
import pytest
import torch

import decode_step_sampling_amd as dss
import synthetic_inputs as si
from oracle import reference as ref
from gpu_util import gpu, host, pooled_chi_square, u64

pytestmark = pytest.mark.gpu


def _supports(probs, op, ks, ps):
    out = []
    for r in range(probs.shape[0]):
        k = ks[r] if np.ndim(ks) else ks
        p = ps[r] if np.ndim(ps) else ps
        valid, tau = ref.threshold(probs[r], op, k=k, p=p)
        out.append(ref.support_mask(probs[r], tau) if valid else None)
    return out


def _call(op, P, k, p, **kw):
    if op == "top_k":
        return dss.top_k_sampling_from_probs(P, k, **kw)
    return dss.top_k_top_p_sampling_from_probs(P, k, p, **kw)


@pytest.mark.parametrize("op", ["top_k", "top_k_top_p"])
# 86, 52 and 37 outputs give 3, 5 and 7 slices per row: windows of the
# candidate gather that do not divide the 8192 slots evenly
@pytest.mark.parametrize("rows,vocab", [(64, 151936), (4, 32000), (1, 151936), (3, 8192),
                                        (86, 16384), (52, 50000), (37, 32000)])
def test_split_support_and_validity(op, rows, vocab):
    w = si.renorm(rows=rows, vocab=vocab)
    probs = w["probs"]
    P = gpu(probs)
    sup = _supports(probs, op, w["top_k"], w["top_p"])
    k, p = gpu(w["top_k"]), gpu(w["top_p"])
    seeds = u64(w["seeds"])
    first = None
    for call in range(30):
        s, v, r = _call(op, P, k, p, seed=seeds, offset=call, return_valid=True,
                        return_rounds=True)
        s, v, r = host(s), host(v), host(r)
        assert (v == 1).all() and (r >= 1).all()
        for row in range(rows):
            assert sup[row][s[row]], (op, rows, vocab, call, row)
        if call == 0:
            first = s
    again = host(_call(op, P, k, p, seed=seeds, offset=0))
    assert np.array_equal(first, again)             # deterministic replay


@pytest.mark.parametrize("op", ["top_k", "top_k_top_p"])
def test_split_chi_square_across_calls_w16(op):
    """4 rows per call: 16 slices per row, so every draw crosses the hand-off."""
    w = si.small()
    probs = w["probs"]
    rows, V = probs.shape
    calls = 6000
    k, p = 50, np.float32(0.9)
    P = gpu(probs)
    seeds = u64(np.array([7, 8, 9, 10], dtype=np.uint64))
    out = torch.empty(calls, rows, dtype=torch.int32, device="cuda:0")
    for t in range(calls):
        out[t] = _call(op, P, k, p, seed=seeds, offset=t)
    s = host(out)
    for row in range(rows):
        _, tau = ref.threshold(probs[row], op, k=k, p=p)
        support = ref.support_mask(probs[row], tau)
        assert support[s[:, row]].all()
        counts = np.bincount(s[:, row], minlength=V)
        pval, tvd, _ = pooled_chi_square(counts[support],
                                         ref.target_distribution(probs[row], tau)[support])
        assert pval > 1e-3, (op, row, pval, tvd)


# 4 rows: 16 slices per row; 64 rows: 4 slices, so that large k stays on the
# split path (16 lists of at least k entries would overflow the merge)
@pytest.mark.parametrize("rows,k,p", [(4, 300, 0.95), (4, 50, 0.0), (64, 1000, 0.6),
                                      (64, 2048, 0.3), (64, 700, 0.0), (64, 1024, 0.95)])
def test_split_chi_square_top_p_start(rows, k, p):
    """Top-p cuts far above tau_k: the loop starts from a pivot taken from the
    merge's mass histogram, which must never exclude a kept token."""
    probs = si.small()["probs"] if rows == 4 else si.renorm(rows=rows, vocab=32000)["probs"]
    V = probs.shape[1]
    calls = 4000
    P = gpu(probs)
    seeds = u64(np.arange(11, 11 + rows, dtype=np.uint64))
    out = torch.empty(calls, rows, dtype=torch.int32, device="cuda:0")
    rounds = torch.empty(calls, rows, dtype=torch.int32, device="cuda:0")
    for t in range(calls):
        out[t], _, rounds[t] = dss.top_k_top_p_sampling_from_probs(
            P, k, np.float32(p), seed=seeds, offset=t, return_valid=True, return_rounds=True)
    s, r = host(out), host(rounds)
    assert (r >= 1).all()
    for row in range(4):
        _, tau = ref.threshold(probs[row], "top_k_top_p", k=k, p=np.float32(p))
        support = ref.support_mask(probs[row], tau)
        assert support[s[:, row]].all(), (k, p, row)
        counts = np.bincount(s[:, row], minlength=V)
        if support.sum() > 1:
            pval, tvd, _ = pooled_chi_square(counts[support],
                                             ref.target_distribution(probs[row], tau)[support])
            assert pval > 1e-3, (k, p, row, pval, tvd)


def test_split_adversarial_rows():
    """Flat rows overflow the candidate buffers (streaming fallback); sorted
    rows put the whole top-k in one slice; ties sit at the local bounds."""
    V = 65536
    rng = np.random.default_rng(5)
    flat = (1.0 + rng.uniform(-1e-3, 1e-3, V)) / V
    geo = (1.0 - 1e-4) ** np.arange(V, dtype=np.float64)
    ties = np.repeat(rng.dirichlet(np.ones(V // 64)), 64)     # 64 copies of every value
    peaked = np.full(V, 0.01 / (V - 1))
    peaked[123] = 0.99
    rows = np.stack([r / r.sum() for r in (flat, geo, ties, peaked)]).astype(np.float32)
    P = gpu(rows)
    for op in ("top_k", "top_k_top_p"):
        for k, p in ((1, 0.5), (37, 0.9), (1000, 0.95), (1536, 0.3), (1537, 0.99), (V, 1.0)):
            sup = _supports(rows, op, k, np.float32(p))
            for n_out in (4, 64):           # few outputs: W > 1; many: more rows per call
                idx = gpu((np.arange(n_out) % 4).astype(np.int32))
                s, v = _call(op, P, k, np.float32(p), indices=idx, seed=k, offset=n_out,
                             return_valid=True)
                s, v = host(s), host(v)
                assert (v == 1).all()
                for o in range(n_out):
                    assert sup[o % 4][s[o]], (op, k, p, n_out, o)


def test_split_degenerate_rows():
    V = 16384
    rng = np.random.default_rng(9)
    good = rng.dirichlet(np.ones(V)).astype(np.float32)
    rows = np.stack([good] * 6)
    rows[1, 9000] = np.nan
    rows[2, 15] = -1e-6
    rows[3] = 0.0
    rows[4, 16383] = np.inf
    P = gpu(rows)
    for op in ("top_k", "top_k_top_p"):
        for n_out in (6, 600):
            idx = gpu((np.arange(n_out) % 6).astype(np.int32))
            s, v = _call(op, P, 20, np.float32(0.8), indices=idx, seed=3, return_valid=True)
            s, v = host(s), host(v)
            expect = np.array([1, 0, 0, 0, 0, 1] * (n_out // 6))
            assert np.array_equal(v, expect), (op, n_out)
            assert (s[expect == 0] == -1).all() and (s[expect == 1] >= 0).all()


def test_split_workspace_reuse_across_shapes():
    """The arrival counters must be back at zero after every call."""
    shapes = [(64, 151936), (2, 151936), (16, 50000), (64, 151936), (1, 200000)]
    for rows, vocab in shapes:
        w = si.renorm(rows=rows, vocab=vocab)
        P = gpu(w["probs"])
        sup = _supports(w["probs"], "top_k_top_p", w["top_k"], w["top_p"])
        for call in range(3):
            s, v = dss.top_k_top_p_sampling_from_probs(P, gpu(w["top_k"]), gpu(w["top_p"]),
                                                       seed=u64(w["seeds"]), offset=call,
                                                       return_valid=True)
            s, v = host(s), host(v)
            assert (v == 1).all()
            assert all(sup[r][s[r]] for r in range(rows)), (rows, vocab, call)


def test_workspace_shared_by_renorm_and_sampling():
    """The binding keeps one workspace per device for every op: the per-row
    results of a split renorm or mask of any shape (one slice per row, several
    slices, many rows) must leave the sampler's arrival counters at zero."""
    rng = np.random.default_rng(77)
    w = si.small()
    P = gpu(w["probs"])
    sup = _supports(w["probs"], "top_k_top_p", 50, np.float32(0.9))
    for rows, V in ((2100, 1024), (64, 16384), (3, 8192)):
        probs = rng.dirichlet(np.full(V, 0.3), size=rows).astype(np.float32)
        dss.top_k_renorm_probs(gpu(probs), 100)
        dss.top_k_mask_logits(gpu(np.log(probs)), 100)
        for call in range(3):
            s, v = dss.top_k_top_p_sampling_from_probs(P, 50, np.float32(0.9), seed=5,
                                                       offset=call, return_valid=True)
            s, v = host(s), host(v)
            assert (v == 1).all(), (rows, V, call)
            assert all(sup[r][s[r]] for r in range(4)), (rows, V, call)


@pytest.mark.parametrize("op", ["top_k", "top_k_top_p"])
def test_split_flat_rows_refined_bound(op):
    """Near-uniform and geometric rows with per-output k arrays (so the call
    stays on the split engine): their vector maxima share one or a few
    histogram bins, and the slices narrow their bounds with the next bits
    of those bins.  Every draw valid and inside the oracle's kept set, and
    the draws of one near-uniform row follow p~ (chi-square, alpha = 1e-3)."""
    rng = np.random.default_rng(61)
    rows, V = 8, 151936
    x = np.empty((rows, V), dtype=np.float64)
    x[:4] = 1.0 + rng.uniform(-1e-3, 1e-3, size=(4, V))
    x[4:] = (1.0 - 2e-6) ** np.arange(V, dtype=np.float64)[None, :]
    x /= x.sum(axis=1, keepdims=True)
    probs = np.ascontiguousarray(x.astype(np.float32))
    ks = np.array([200, 1000, 50, 2048, 300, 1000, 20, 2000], dtype=np.int32)
    ps = np.array([0.9, 0.5, 1.0, 0.95, 0.8, 0.99, 0.3, 1.0], dtype=np.float32)
    sup = _supports(probs, op, ks, ps)
    P, K, Pp = gpu(probs), gpu(ks), gpu(ps)
    for call in range(8):
        s, v = _call(op, P, K, Pp, seed=3, offset=call, return_valid=True)
        s, v = host(s), host(v)
        assert (v == 1).all()
        for r in range(rows):
            assert sup[r][s[r]], (call, r)
    # one near-uniform row, 20000 draws in one call
    n = 20000
    idx = np.zeros(n, dtype=np.int32)
    s = host(_call(op, P, gpu(np.full(n, 200, dtype=np.int32)), gpu(np.full(n, 0.9, dtype=np.float32)),
                   indices=gpu(idx), seed=11, offset=0))
    valid, tau = ref.threshold(probs[0], op, k=200, p=np.float32(0.9))
    s0 = ref.support_mask(probs[0], tau)
    assert s0[s].all()
    counts = np.bincount(s, minlength=V)
    pval, tvd, cells = pooled_chi_square(counts[s0], ref.target_distribution(probs[0], tau)[s0])
    assert pval > 1e-3, (pval, tvd, cells)
