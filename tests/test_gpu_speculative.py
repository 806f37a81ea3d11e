"""GPU parity of chain speculative verification against the oracle.

Both sides take the same decisions from the same Philox draws: the
acceptance tests u_j * q_j(d_j) < p_j(d_j) exactly (the GPU with an fma
error term, the oracle in integers), the final draw by inverse transform on
the residual max(0, p - q) (GPU: float64 differences and prefix sums;
oracle: exact integers), so tokens and accepted counts are compared exactly.
A float64 prefix could only disagree for a draw within ~1e-13 relative of a
boundary.
"""

import numpy as np
import pytest

import decode_step_sampling_amd as dss
import synthetic_inputs as si
from oracle import philox as ph
from oracle import reference as ref
from gpu_util import gpu, host, u64

pytestmark = pytest.mark.gpu


def _draws(seed, offset, sid, n):
    return [ph.draw_bits53(int(seed), int(offset), int(sid), j) for j in range(n + 1)]


def _expect(q, ids, p, seeds, offset, per_row_seed=True, rows=None):
    n = ids.shape[1]
    rows = range(q.shape[0]) if rows is None else rows
    out = {}
    for r in rows:
        sid = 0 if per_row_seed else r
        seed = seeds[r] if per_row_seed else seeds
        off = offset[r] if np.ndim(offset) else offset
        out[r] = ref.chain_speculative(q[r], ids[r], p[r], _draws(seed, off, sid, n))
    return out


def _run(q, ids, p, seed, offset=0):
    S = u64(seed) if np.ndim(seed) else int(seed)
    O = u64(offset) if np.ndim(offset) else int(offset)
    t, a, v = dss.chain_speculative_sampling(gpu(q), gpu(ids), gpu(p), seed=S, offset=O,
                                             return_valid=True)
    return host(t), host(a), host(v)


def _compare(exp, t, a, v):
    for r, (ok, tok, acc) in exp.items():
        assert v[r] == (1 if ok else 0), r
        assert list(t[r]) == list(tok), (r, list(t[r]), list(tok))
        assert a[r] == acc, r


@pytest.mark.parametrize("vocab,rows,n", [(32000, 16, 4), (4100, 8, 3), (8, 5, 2), (1024, 3, 7)])
def test_token_exact(vocab, rows, n):
    w = si.speculative(rep=vocab % 97, rows=rows, n=n, vocab=vocab)
    for offset in (0, 5):
        t, a, v = _run(w["q"], w["ids"], w["p"], w["seeds"], offset)
        _compare(_expect(w["q"], w["ids"], w["p"], w["seeds"], offset), t, a, v)
    # one scalar seed: the row index picks the stream
    t, a, v = _run(w["q"], w["ids"], w["p"], 1234567)
    _compare(_expect(w["q"], w["ids"], w["p"], 1234567, 0, per_row_seed=False), t, a, v)


def test_full_size_sampled_rows():
    """B=64, n=4, V=151936 in the bench's launch configuration; the oracle on
    16 of the rows, every row checked for shape (accepted drafts, a token,
    then -1)."""
    w = si.speculative()
    offs = np.arange(64, dtype=np.uint64) * np.uint64(3)
    t, a, v = _run(w["q"], w["ids"], w["p"], w["seeds"], offs)
    assert (v == 1).all()
    for r in range(64):
        k = a[r]
        assert 0 <= k <= 4
        assert list(t[r, :k]) == list(w["ids"][r, :k])
        assert 0 <= t[r, k] < 151936 and (t[r, k + 1:] == -1).all()
    exp = _expect(w["q"], w["ids"], w["p"], w["seeds"], offs, rows=range(0, 64, 4))
    _compare(exp, t, a, v)
    assert 0 < a.sum() < 4 * 64   # both outcomes occur on this workload


def test_no_drafts_and_identical_models():
    w = si.speculative(rep=1, rows=6, n=3, vocab=4096)
    # n = 0: a plain draw from p_0
    p0 = np.ascontiguousarray(w["p"][:, :1])
    q0 = np.zeros((6, 0, 4096), dtype=np.float32)
    ids0 = np.zeros((6, 0), dtype=np.int32)
    t, a, v = _run(q0, ids0, p0, w["seeds"])
    _compare(_expect(q0, ids0, p0, w["seeds"], 0), t, a, v)
    # q = p: every draft accepted, then the bonus token
    qp = np.ascontiguousarray(w["p"][:, :3])
    t, a, v = _run(qp, w["ids"], w["p"], w["seeds"])
    assert (a == 3).all() and (v == 1).all()
    _compare(_expect(qp, w["ids"], w["p"], w["seeds"], 0), t, a, v)


def test_zero_residual_and_zero_target():
    """p = q / 2 (unnormalised): a rejection finds no residual and draws
    from p; p(d) = 0 always rejects."""
    w = si.speculative(rep=2, rows=8, n=2, vocab=2048)
    p = w["p"].copy()
    p[:, :2] = w["q"] * np.float32(0.5)
    p[3, 0, w["ids"][3, 0]] = 0.0
    t, a, v = _run(w["q"], w["ids"], p, w["seeds"])
    _compare(_expect(w["q"], w["ids"], p, w["seeds"], 0), t, a, v)
    assert a[3] == 0


def test_invalid_rows():
    w = si.speculative(rep=3, rows=6, n=3, vocab=4096)
    q, p, ids = w["q"].copy(), w["p"].copy(), w["ids"].copy()
    ids[0, 1] = 4096                        # draft id out of range
    ids[1, 0] = -5
    p[2, 0, ids[2, 0]] = np.nan              # an examined value
    q[3, 0, :] = 0.0                         # row 3 rejects at 0 (q(d) = 0 accepts iff p > 0 ...)
    q[3, 0, ids[3, 0]] = np.float32(1.0)     # ... so make the draft certain and p small
    p[3, 0, ids[3, 0]] = np.float32(1e-30)
    p[3, 0, 7] = -1.0                        # a negative value in the rejected row
    p[4, 3, 11] = np.inf                     # in the bonus row (read only if all accepted)
    q[4, :, :] = p[4, :3, :]                 # identical models: every draft accepted
    t, a, v = _run(q, ids, p, w["seeds"])
    exp = _expect(q, ids, p, w["seeds"], 0)
    _compare(exp, t, a, v)
    assert list(v) == [0, 0, 0, 0, 0, 1]
