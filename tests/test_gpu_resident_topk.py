"""GPU parity of top-k and top-k-then-top-p sampling on the resident engine
(a scalar k above the split engine's cap, or k * W above half of its
candidate capacity): tau_k exactly by counts, the top-p cut inside the top-k
set exactly by masses, then one draw in index order.  That is the oracle's
CDF draw on the kept set, so tokens are compared exactly (up to float64
prefix rounding at a boundary, ~1e-13 relative)."""

import numpy as np
import pytest

import decode_step_sampling_amd as dss
import synthetic_inputs as si
from oracle import philox as ph
from oracle import reference as ref
from gpu_util import gpu, host, u64

pytestmark = pytest.mark.gpu


def _rows(kind, rows, V, rng):
    if kind == "softmax":
        return si.softmax_rows(rng, rows, V, 2.0)
    if kind == "ties":                       # few distinct values, huge tie groups
        x = rng.integers(1, 6, size=(rows, V)).astype(np.float64)
    elif kind == "flat":                     # near-uniform (one level-1 bin)
        x = 1.0 + rng.uniform(-1e-3, 1e-3, size=(rows, V))
    else:                                    # geometric chain in index order
        x = np.tile((1.0 - 1e-5) ** np.arange(V, dtype=np.float64), (rows, 1))
    x /= x.sum(axis=1, keepdims=True)
    return np.ascontiguousarray(x.astype(np.float32))


def _table(row, op, k, p):
    """The oracle's CDF draw on the kept set (``sample_by_cdf``), built once."""
    valid, tau = ref.threshold(row, op, k=k, p=p)
    assert valid
    return ref.CdfTable(row, ref.support_mask(row, tau))


def _call(op, P, k, p, n_per_row, rows, seed, offset):
    idx = np.repeat(np.arange(rows, dtype=np.int32), n_per_row)
    if op == "top_k":
        out = dss.top_k_sampling_from_probs(P, k, indices=gpu(idx), seed=seed, offset=offset,
                                            return_valid=True, return_rounds=True)
    else:
        out = dss.top_k_top_p_sampling_from_probs(P, k, p, indices=gpu(idx), seed=seed,
                                                  offset=offset, return_valid=True,
                                                  return_rounds=True)
    return idx, [host(t) for t in out]


@pytest.mark.parametrize("kind", ["softmax", "ties", "flat", "geometric"])
@pytest.mark.parametrize("op", ["top_k", "top_k_top_p"])
@pytest.mark.parametrize("k", [1000, 3000, 70000])
def test_token_exact(kind, op, k):
    """Four rows of V=32768, one output each (W=16 slices, so k * W > 4096
    even for k=1000), 16 calls with offsets 0..15."""
    rng = np.random.default_rng(sum(map(ord, kind + op)) + k)
    rows, V = 4, 32768
    probs = _rows(kind, rows, V, rng)
    P = gpu(probs)
    p = np.float32(0.8)
    seed = 4242
    tables = [_table(probs[i], op, k, p) for i in range(rows)]
    for offset in range(16):
        idx, (s, v, r) = _call(op, P, k, p, 1, rows, seed, offset)
        assert (v == 1).all() and (r == 1).all()
        for i in range(rows):
            want = tables[i].draw(ph.draw_bits53(seed, offset, i, 0))
            assert s[i] == want, (kind, op, k, offset, i, int(s[i]), want)


def test_extremes_and_invalid():
    rng = np.random.default_rng(9)
    probs = si.softmax_rows(rng, 3, 8192, 2.0)
    P = gpu(probs)
    # k = 1 (the maximum), k = V and above (everything), p = 0 and p = 1
    for k, p in ((1, 0.9), (8192, 0.5), (10**6, 1.0), (2500, 0.0)):
        idx, (s, v, r) = _call("top_k_top_p", P, k, np.float32(p), 8, 3, 77, 0)
        tables = [_table(probs[j], "top_k_top_p", k, np.float32(p)) for j in range(3)]
        for i in range(idx.size):
            assert s[i] == tables[idx[i]].draw(ph.draw_bits53(77, 0, i, 0)), (k, p, i)
    # k <= 0 and a NaN p make the output invalid
    for k, p in ((0, 0.5), (-3, 0.5), (3000, float("nan"))):
        s, v = dss.top_k_top_p_sampling_from_probs(P, k, p, seed=1, return_valid=True)
        assert (host(v) == 0).all() and (host(s) == -1).all()


def test_stress_rows_full_size():
    """The stress workload's near-uniform, peaked and geometric rows at
    B=512, V=256000, p=0.95, with the workload's k=1000 (k * W = 8000) and
    with k=2500 (above the split cap), both on the resident engine (the one
    search on (count, mass) pairs, four slices of 64 values per thread,
    eight launches): one draw per row against the oracle's CDF draw, every
    16th row of each call."""
    w = si.stress()
    probs = w["probs"]
    seeds = w["seeds"]
    P = gpu(probs)
    s, v, r = dss.top_k_top_p_sampling_from_probs(P, 2500, 0.95, seed=u64(seeds),
                                                  offset=5, return_valid=True, return_rounds=True)
    s, v, r = host(s), host(v), host(r)
    assert (v == 1).all() and (r == 1).all()
    for row in range(0, probs.shape[0], 16):
        want = ref.sample_by_cdf(probs[row], "top_k_top_p",
                                 ph.draw_bits53(int(seeds[row]), 5, 0, 0), k=2500,
                                 p=np.float32(0.95))
        assert s[row] == want, (row, int(w["groups"][row]))
    s, v = dss.top_k_top_p_sampling_from_probs(P, 1000, 0.95, seed=u64(seeds), offset=6,
                                               return_valid=True)
    s, v = host(s), host(v)
    assert (v == 1).all()
    for row in range(3, probs.shape[0], 16):
        want = ref.sample_by_cdf(probs[row], "top_k_top_p",
                                 ph.draw_bits53(int(seeds[row]), 6, 0, 0), k=1000,
                                 p=np.float32(0.95))
        assert s[row] == want, (row, int(w["groups"][row]))


@pytest.mark.parametrize("n_out", [8, 72])
@pytest.mark.parametrize("op", ["top_k", "top_k_top_p", "top_k_top_p_joint"])
def test_split_fallback_rows_token_exact(op, n_out):
    """Per-output k arrays keep a call on the split engine; its outputs with
    k above the cap (2048) take the histogram path (exact tau_k, Z_k and top-p
    cut from the slices' histograms and the gathered boundary keys, one draw
    over the tiles in index order), which equals the oracle's CDF draw; the
    other outputs are checked for their kept set only.  8 outputs: the last
    slice to arrive merges (16 slices each); 72 outputs: 288 slices, more
    than one wave of work-groups, so finishing work-groups merge."""
    rng = np.random.default_rng(31)
    rows, V = 8, 32768
    probs = np.concatenate([si.softmax_rows(rng, 6, V, 2.0), _rows("flat", 2, V, rng)])
    ks = np.array([50, 3000, 10, 70000, 2049, 1, 5000, 1000], dtype=np.int32)
    ps = np.array([0.9, 0.7, 0.5, 0.95, 0.3, 1.0, 0.99, 0.6], dtype=np.float32)
    idx = (np.arange(n_out) % rows).astype(np.int32)
    seeds = (np.arange(n_out, dtype=np.uint64) + np.uint64(7)) * np.uint64(0x9E3779B97F4A7C15)
    P = gpu(probs)
    kk, pk = ks[idx], ps[idx]
    tables = {i: _table(probs[i], op, int(ks[i]), ps[i]) for i in range(rows) if ks[i] > 2048}
    for offset in range(8 if n_out == 8 else 3):
        if op == "top_k":
            s, v, r = dss.top_k_sampling_from_probs(P, gpu(kk), indices=gpu(idx), seed=u64(seeds),
                                                    offset=offset, return_valid=True,
                                                    return_rounds=True)
        else:
            order = "joint" if op.endswith("joint") else "top_k_first"
            s, v, r = dss.top_k_top_p_sampling_from_probs(P, gpu(kk), gpu(pk), indices=gpu(idx),
                                                          seed=u64(seeds), offset=offset,
                                                          return_valid=True, return_rounds=True,
                                                          filter_apply_order=order)
        s, v, r = host(s), host(v), host(r)
        assert (v == 1).all()
        for j in range(n_out):
            i = int(idx[j])
            kw = dict(k=int(ks[i]), p=ps[i])
            valid, tau = ref.threshold(probs[i], op, **kw)
            assert ref.support_mask(probs[i], tau)[s[j]], (op, j, offset)
            if ks[i] > 2048:
                want = tables[i].draw(ph.draw_bits53(int(seeds[j]), offset, 0, 0))
                assert s[j] == want and r[j] == 1, (op, j, offset, int(s[j]), want)


@pytest.mark.parametrize("op", ["top_k", "top_k_top_p", "top_k_top_p_joint"])
def test_split_fallback_invalid_rows(op):
    """Outputs with k above the split cap reach the exact fallback before any
    validity check: a NaN, -0.0, a negative value, +inf or an all-zero row
    must come out invalid there; a valid row beside them is unaffected."""
    rng = np.random.default_rng(5)
    V = 8192
    probs = si.softmax_rows(rng, 6, V, 2.0)
    probs[0, 17] = np.nan
    probs[1, 3] = -0.0
    probs[2, 4000] = -1e-3
    probs[3, 9] = np.inf
    probs[4, :] = 0.0
    ks = np.full(6, 3000, dtype=np.int32)
    ps = np.full(6, 0.9, dtype=np.float32)
    P = gpu(probs)
    if op == "top_k":
        s, v = dss.top_k_sampling_from_probs(P, gpu(ks), seed=3, return_valid=True)
    else:
        order = "joint" if op.endswith("joint") else "top_k_first"
        s, v = dss.top_k_top_p_sampling_from_probs(P, gpu(ks), gpu(ps), seed=3, return_valid=True,
                                                   filter_apply_order=order)
    s, v = host(s), host(v)
    assert list(v) == [0, 0, 0, 0, 0, 1], list(v)
    assert list(s[:5]) == [-1] * 5
    want = _table(probs[5], op, 3000, ps[5]).draw(ph.draw_bits53(3, 0, 5, 0))
    assert s[5] == want


# ---- the pair search's branches (scalar k <= 8192 on the resident engine) ----

def _branch(row, k, p):
    """Where the top-p cut of top-k-then-top-p lies relative to the count
    search's path, from the float32 bit patterns (level 1: bits [30:21],
    level 2: [20:10]): ("list" if bin b1 and everything above it hold at
    most 8192 values, else "rows"), ("on", "l1", "l2"), and the number of
    values in the bin that holds the cut when it is off the path."""
    keys = row.view(np.uint32)
    tau_k = np.sort(keys)[::-1][k - 1]
    valid, tau = ref.threshold(row, "top_k_top_p", k=k, p=np.float32(p))
    assert valid
    tp = np.float32(tau).view(np.uint32)
    b1, p1 = tau_k >> 21, tp >> 21
    path = "list" if np.sum(keys >> 21 >= b1) <= 8192 else "rows"
    if p1 != b1:
        return path, "l1", int(np.sum(keys >> 21 == p1))
    if (tp >> 10) != (tau_k >> 10):
        return path, "l2", int(np.sum(keys >> 10 == tp >> 10))
    return path, "on", 0


def _pair_rows(V, rng):
    """Rows built so that the cut takes each branch; (row, k, p, expected)."""
    out = []

    def norm(x):
        x = x / x.sum()
        return np.ascontiguousarray(x.astype(np.float32))

    # a few / many large values above a long flat tail: the cut lies in a
    # level-1 bin above the boundary bin (row histograms for the count search)
    for nbig, big, p in ((20, 1e-2, 0.5), (200, 1e-3, 0.5)):
        x = (1.0 + rng.uniform(-0.3, 0.3, V)) * 1e-6
        x[rng.choice(V, nbig, replace=False)] = big * (1 + np.arange(nbig) * 1e-4)
        out.append((norm(x), 1000, p, ("rows", "l1", nbig)))
    # 1000 values in one level-1 bin, the top few / many of them in a higher
    # level-2 bin, and a tail far below: the count search lists bin b1, the
    # cut is in a level-2 bin above the boundary's
    for ntop, p in ((30, 0.02), (100, 0.05)):
        x = rng.uniform(0.5, 1.5, V) * 1e-9
        pos = rng.choice(V, 1000, replace=False)
        x[pos[:ntop]] = 1.2 * (1 + np.arange(ntop) * 2.5e-7)
        x[pos[ntop:]] = 1.1 * (1 + np.arange(1000 - ntop) * 2.5e-7)
        out.append((norm(x), 1000, p, ("list", "l2", ntop)))
    # a few / many large values above 2000 medium ones and a tail far below:
    # the count search lists bin b1 and everything above it, the cut lies in
    # a level-1 bin above the boundary's
    for nbig, big, p in ((20, 1e-2, 0.5), (200, 1e-3, 0.5)):
        x = rng.uniform(0.5, 1.5, V) * 1e-9
        pos = rng.choice(V, nbig + 2000, replace=False)
        x[pos[:nbig]] = big * (1 + np.arange(nbig) * 1e-4)
        x[pos[nbig:]] = 1e-4 * (1 + np.arange(2000) * 1e-5)
        out.append((norm(x), 1000, p, ("list", "l1", nbig)))
    # the same over a dense level-1 bin (row histograms), the top values in a
    # higher level-2 bin
    for ntop, p in ((30, 0.02), (100, 0.05)):
        x = 1.0 + rng.uniform(0.0, 0.05, V)
        x[rng.choice(V, ntop, replace=False)] = 1.2 * (1 + np.arange(ntop) * 2.5e-7)
        out.append((norm(x), 1000, p, ("rows", "l2", ntop)))
    # on the path
    out.append((norm(1.0 + rng.uniform(-1e-3, 1e-3, V)), 1000, 0.9, ("rows", "on", 0)))
    # fewer positive values than k: tau_k is the zero pattern, every positive
    # value is in the top-k set and the cut lies among them
    x = np.zeros(V)
    x[rng.choice(V, 500, replace=False)] = rng.uniform(0.5, 1.5, 500)
    out.append((norm(x), 1000, 0.7, ("rows", "l1", 50)))
    return out


def test_pair_search_branches_token_exact():
    """Top-k-then-top-p with a scalar k (the one search on (count, mass)
    pairs): rows whose top-p cut lies on the count search's path, in a
    level-1 bin above the top-k boundary bin, or in a level-2 bin above it,
    each with few (at most 64: one wave's exact suffix sums) or many listed
    keys in that bin, with the count search on row histograms or on the
    listed keys.  Every draw equals the oracle's CDF draw, over 8 offsets."""
    rng = np.random.default_rng(79)  # a seed whose rows each take the intended branch
    V = 32768
    cases = _pair_rows(V, rng)
    for row, k, p, want in cases:
        got = _branch(row, k, p)
        assert got[:2] == want[:2] and (got[2] <= 64) == (want[2] <= 64), (want, got)
    probs = np.stack([c[0] for c in cases])
    P = gpu(probs)
    rows = probs.shape[0]
    seed = 99
    tables = [ref.CdfTable(c[0], ref.support_mask(c[0], ref.threshold(c[0], "top_k_top_p", k=c[1],
                                                                         p=np.float32(c[2]))[1]))
              for c in cases]
    ps = np.array([c[2] for c in cases], dtype=np.float32)
    for offset in range(8):
        idx = np.arange(rows, dtype=np.int32)
        s, v, r = dss.top_k_top_p_sampling_from_probs(P, 1000, gpu(ps), indices=gpu(idx), seed=seed,
                                                      offset=offset, return_valid=True,
                                                      return_rounds=True)
        s, v, r = host(s), host(v), host(r)
        assert (v == 1).all() and (r == 1).all()
        for i in range(rows):
            want_tok = tables[i].draw(ph.draw_bits53(seed, offset, i, 0))
            assert s[i] == want_tok, (cases[i][3], offset, int(s[i]), want_tok)


def test_largest_vocab():
    """V = 2^20 - 4 (the pair search's largest rows: sixteen slices of 64
    values per thread) is token-exact against the oracle's CDF draw on a
    near-uniform and a softmax row; at V = 2^20 (DSS_MAX_VOCAB) a bin of a
    near-uniform row would hold 2^20 values, more than a packed pair counts,
    so such calls take another engine: every token there lies in the kept
    set."""
    rng = np.random.default_rng(1234)
    for V, exact in ((2**20 - 4, True), (2**20, False)):
        probs = np.stack([_rows("flat", 1, V, rng)[0], si.softmax_rows(rng, 1, V, 2.0)[0]])
        P = gpu(probs)
        k, p, seed = 1000, np.float32(0.9), 5
        tables = [_table(probs[i], "top_k_top_p", k, p) for i in range(2)]
        for offset in range(4):
            s, v = dss.top_k_top_p_sampling_from_probs(P, k, p, seed=seed, offset=offset,
                                                       return_valid=True)
            s, v = host(s), host(v)
            assert (v == 1).all()
            for i in range(2):
                _, tau = ref.threshold(probs[i], "top_k_top_p", k=k, p=p)
                assert ref.support_mask(probs[i], tau)[s[i]], (V, i, offset)
                if exact:
                    assert s[i] == tables[i].draw(ph.draw_bits53(seed, offset, i, 0)), (V, i, offset)
