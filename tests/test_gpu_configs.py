"""GPU parity at the full sizes of the latency, heterogeneous-batch and
round-count stress workloads, called the way bench.py times them.

Token-for-token equality is not required (RNG consumption differs between
engines); what is checked is what holds at any size: every draw valid and
inside the oracle's kept set for its own row and parameters, per-row
chi-square against the oracle's p~ where enough draws of one row are taken,
and the round counts.
"""

import numpy as np
import pytest
import torch

import decode_step_sampling_amd as dss
import synthetic_inputs as si
from oracle import reference as ref
from gpu_util import gpu, host, pooled_chi_square, u64

pytestmark = pytest.mark.gpu


def _chi_square(row, tau, draws):
    sup = ref.support_mask(row, tau)
    assert (draws >= 0).all() and sup[draws].all(), "draw outside the kept set"
    counts = np.bincount(draws, minlength=row.size)
    pval, tvd, cells = pooled_chi_square(counts[sup], ref.target_distribution(row, tau)[sup])
    assert pval > 1e-3, (pval, tvd, cells)


def test_latency_config_chi_square():
    """B=1, V=151936, k=50, p=0.9 on the split-row path (W=16): 10000 calls
    with offsets 0..9999, the draws against the oracle's p~."""
    w = si.latency()
    probs = w["probs"]
    P = gpu(probs)
    seed = u64(w["seeds"])
    outs = []
    for off in range(10000):
        s, v, r = dss.top_k_top_p_sampling_from_probs(P, 50, 0.9, seed=seed, offset=off,
                                                      return_valid=True, return_rounds=True)
        outs.append(torch.stack([s[0], v[0].to(torch.int32), r[0]]))
    got = host(torch.stack(outs))
    assert (got[:, 1] == 1).all() and (got[:, 2] >= 1).all()
    _, tau = ref.threshold(probs[0], "top_k_top_p", k=50, p=np.float32(0.9))
    _chi_square(probs[0], tau, got[:, 0])


@pytest.fixture(scope="module")
def hetero():
    w = si.hetero()
    w["P"] = gpu(w["probs"])
    return w


HETERO_OPS = ("top_k_top_p", "min_p", "none")


def _hetero_call(w, o, sel, offset, seeds=None, indices=None):
    idx = w["indices"][sel] if indices is None else indices
    I = gpu(idx)
    S = u64(w["seeds"][sel] if seeds is None else seeds)
    if o == 0:
        return dss.top_k_top_p_sampling_from_probs(w["P"], gpu(w["top_k"][idx]), gpu(w["top_p"][idx]),
                                                   indices=I, seed=S, offset=offset,
                                                   return_valid=True, return_rounds=True)
    if o == 1:
        return dss.min_p_sampling_from_probs(w["P"], gpu(w["min_p"][idx]), indices=I, seed=S,
                                             offset=offset, return_valid=True, return_rounds=True)
    return dss.sampling_from_probs(w["P"], indices=I, seed=S, offset=offset, return_valid=True,
                                   return_rounds=True)


def _hetero_tau(w, o, row, cache):
    key = (o, row)
    if key not in cache:
        valid, tau = ref.threshold(w["probs"][row], HETERO_OPS[o], k=w["top_k"][row],
                                   p=w["top_p"][row], min_p=w["min_p"][row])
        assert valid
        cache[key] = ref.support_mask(w["probs"][row], tau)
    return cache[key]


def test_hetero_config_support(hetero):
    """B=256, V=128256 Zipf rows, 512 outputs over the 256 rows, three calls
    per step (top-k-then-top-p with k up to V, min-p, plain) with per-output
    seeds: four steps, every draw valid and inside its own kept set."""
    w = hetero
    cache = {}
    for o in range(3):
        sel = np.nonzero(w["op_of_output"] == o)[0]
        for step in range(4):
            s, v, r = _hetero_call(w, o, sel, step)
            s, v, r = host(s), host(v), host(r)
            assert (v == 1).all() and (r >= 1).all()
            for n, out in enumerate(sel):
                row = int(w["indices"][out])
                assert _hetero_tau(w, o, row, cache)[s[n]], (HETERO_OPS[o], out, row, step)


@pytest.mark.parametrize("o,draws", [(0, 3000), (1, 20000), (2, 20000)])
def test_hetero_config_chi_square(hetero, o, draws):
    """Many draws of one heterogeneous-batch row per op (for top-k-then-top-p
    a row whose k is above the split engine's candidate cap)."""
    w = hetero
    rows = np.nonzero(w["top_k"] > 4096)[0] if o == 0 else np.arange(w["probs"].shape[0])
    row = int(rows[0])
    idx = np.full(draws, row, dtype=np.int32)
    seeds = np.arange(1, draws + 1, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15)
    s, v, _ = _hetero_call(w, o, None, 3, seeds=seeds, indices=idx)
    s, v = host(s), host(v)
    assert (v == 1).all()
    valid, tau = ref.threshold(w["probs"][row], HETERO_OPS[o], k=w["top_k"][row],
                               p=w["top_p"][row], min_p=w["min_p"][row])
    assert valid
    _chi_square(w["probs"][row], tau, s)


def test_stress_config_support_and_rounds():
    """B=512, V=256000: near-uniform, peaked and geometric rows, k=1000,
    p=0.95, per-row seeds: every draw valid and kept; the dual-pivot loop's
    rounds stay small (each rejected round halves (low, high])."""
    w = si.stress()
    probs = w["probs"]
    P = gpu(probs)
    seeds = u64(w["seeds"])
    supports = []
    for row in range(probs.shape[0]):
        valid, tau = ref.threshold(probs[row], "top_k_top_p", k=1000, p=np.float32(0.95))
        assert valid
        supports.append(ref.support_mask(probs[row], tau))
    for offset in (0, 1):
        s, v, r = dss.top_k_top_p_sampling_from_probs(P, 1000, 0.95, seed=seeds, offset=offset,
                                                      return_valid=True, return_rounds=True)
        s, v, r = host(s), host(v), host(r)
        assert (v == 1).all()
        assert (r >= 1).all() and r.max() < 64
        for row in range(probs.shape[0]):
            assert supports[row][s[row]], (offset, row, int(w["groups"][row]))
