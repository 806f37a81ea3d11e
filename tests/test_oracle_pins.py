"""Pins of the CPU oracle to things other than itself (runs without a GPU).

Each test ties one oracle function to the pages' worked examples, to an
independent definition (brute force on tiny vocabularies, the bisection
definition of the F4 note, numpy's own Philox and sort), to a closed form or
to an invariant stated on the pages.  Pages: FlashInfer blog "Sorting-Free
GPU Kernels for LLM Sampling"; gpu-kernel-drills note "F4 讲解：不排序的
top-k / top-p"; charlestar explainer on FlashInfer Sorting-Free Sampling.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

from oracle import philox as ph
from oracle import reference as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def f32(values):
    return np.asarray(values, dtype=np.float32)


# ----------------------------------------------------------------------------
# Philox: numpy ships an independent Philox4x64-10 implementation.  numpy
# increments its 256-bit counter before each block, so its first block for
# counter c is the block for c + 1.
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("key,ctr", [
    ((0, 0), (0, 0, 0, 0)),
    ((123456789, 987654321), (5, 0, 0, 0)),
    ((2**64 - 1, 2**63 + 7), (11, 22, 33, 44)),
    ((42, 0), (2**64 - 1, 0, 0, 0)),            # carry into word 1
    ((7, 9), (2**64 - 1, 2**64 - 1, 3, 0)),     # carry into word 2
])
def test_philox_matches_numpy(key, ctr):
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                          counter=np.array(ctr, dtype=np.uint64))
    got = [int(v) for v in bg.random_raw(8)]
    value = sum(int(c) << (64 * i) for i, c in enumerate(ctr)) + 1
    nxt = [(value >> (64 * i)) & ph.MASK64 for i in range(4)]
    assert got[:4] == list(ph.philox4x64_10(nxt, key))
    value += 1
    nxt = [(value >> (64 * i)) & ph.MASK64 for i in range(4)]
    assert got[4:] == list(ph.philox4x64_10(nxt, key))


def test_draws_are_uniform_and_streams_differ():
    u = np.array([ph.draw_uniform(99, 3, 0, r) for r in range(20000)])
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    assert 0.0 <= u.min() and u.max() < 1.0
    # offset advance and output id give different streams
    a = [ph.draw_bits53(99, 3, 0, r) for r in range(8)]
    b = [ph.draw_bits53(99, 4, 0, r) for r in range(8)]
    c = [ph.draw_bits53(99, 3, 1, r) for r in range(8)]
    assert a != b and a != c and len(set(a)) == 8


# ----------------------------------------------------------------------------
# worked examples printed on the pages
# ----------------------------------------------------------------------------

def test_f4_hand_example_top_p():
    g = golden("f4_hand_example.json")
    row = f32(g["probs"])
    valid, tau = ref.threshold(row, "top_p", p=g["top_p"])
    assert valid and np.float32(tau) == np.float32(g["tau_top_p"])
    assert list(np.nonzero(ref.kept_mask(row, tau))[0]) == g["kept_top_p"]
    valid, tau = ref.threshold(row, "top_k", k=g["top_k"])
    assert valid and np.float32(tau) == np.float32(g["tau_top_k"])
    assert list(np.nonzero(ref.kept_mask(row, tau))[0]) == g["kept_top_k"]


def test_expl_top2_example_law():
    g = golden("expl_top2_example.json")
    row = f32(g["probs"])
    valid, tau = ref.threshold(row, "top_k", k=g["top_k"])
    assert valid
    assert list(np.nonzero(ref.support_mask(row, tau))[0]) == g["support"]
    target = ref.target_distribution(row, tau)
    expect = np.array(g["law_num"]) / g["law_den"]
    # inputs are the float32 roundings of the printed decimals
    assert np.allclose(target[g["support"]], expect, rtol=2e-7, atol=0)
    law, _ = ref.dual_pivot_law(row, "top_k", k=g["top_k"])
    assert set(law) == set(g["support"])
    for j in g["support"]:
        assert abs(float(law[j]) - target[j]) < 1e-15


def test_expl_order_example():
    g = golden("expl_order_example.json")
    row = f32(g["probs"])
    for p, kept in ((g["top_p"], g["kept"]),
                    (g["derived_top_p"], g["derived_kept"])):
        valid, tau = ref.threshold(row, "top_k_top_p", k=g["top_k"], p=p)
        assert valid
        assert list(np.nonzero(ref.kept_mask(row, tau))[0]) == kept
    # the raw-mass reading (raw prefix of the top-3 compared with p itself,
    # i.e. p / Z_k against the top-3 mass) keeps one more token here
    top3 = row[:3]
    valid, tau = ref.threshold(top3, "top_p",
                               p=np.float32(g["derived_top_p"] / float(top3.sum())))
    assert list(np.nonzero(ref.kept_mask(top3, tau))[0]) == g["raw_mass_reading_kept"]
    # the joint order (R17) checks both conditions against the whole row: with
    # p = 0.75 the row prefix .4 + .3 = .7 is still short of .75, so C stays
    # (the raw-mass set); with p = 0.6 the prefix .7 reaches .6 at B, and top-3
    # is looser, so {A, B}.  Derived from the definitions, not printed.
    for p, kept in ((g["derived_top_p"], g["raw_mass_reading_kept"]), (g["top_p"], [0, 1])):
        valid, tau = ref.threshold(row, "top_k_top_p_joint", k=g["top_k"], p=p)
        assert valid
        assert list(np.nonzero(ref.kept_mask(row, tau))[0]) == kept


# ----------------------------------------------------------------------------
# brute force on tiny vocabularies: the F4 note's bisection definition
# ("largest t with count(x >= t) >= k" / "largest t with mass(x >= t) >= p")
# against the explainer's sort-prefix definition used by the oracle
# ----------------------------------------------------------------------------

def _tiny_rows(seed, n_rows=300):
    rng = np.random.default_rng(seed)
    rows = []
    for i in range(n_rows):
        v = int(rng.integers(1, 9))
        if i % 3 == 0:      # tie-heavy: few distinct dyadic values, some zeros
            row = rng.integers(0, 5, size=v).astype(np.float32) / 8
            if not row.any():
                row[0] = 0.25
        else:
            row = rng.dirichlet(np.ones(v)).astype(np.float32)
        rows.append(f32(row))
    return rows


def _brute_top_k(row, k):
    cands = sorted(set(float(x) for x in row))
    ok = [t for t in cands if sum(1 for x in row if x >= t) >= k]
    return max(ok) if ok else min(cands)


def _brute_top_p(row, p, within=None):
    vals = [Fraction(float(x)) for x in row]
    members = [i for i in range(len(row)) if within is None or within[i]]
    z = sum(vals[i] for i in members)
    pf = Fraction(min(max(float(np.float32(p)), 0.0), 1.0))
    cands = sorted(set(vals[i] for i in members))
    ok = [t for t in cands if sum(vals[i] for i in members if vals[i] >= t) >= pf * z]
    return float(max(ok))


def test_tiny_brute_force_thresholds():
    rng = np.random.default_rng(7)
    for row in _tiny_rows(1):
        v = row.size
        k = int(rng.integers(1, v + 2))
        p = float(np.float32(rng.choice([0.0, 0.3, 0.5, 0.77, 0.9, 1.0,
                                         rng.uniform()])))
        mp = float(np.float32(rng.uniform(0, 1)))
        _, tk = ref.threshold(row, "top_k", k=k)
        assert tk == _brute_top_k(row, k)
        _, tp = ref.threshold(row, "top_p", p=p)
        assert tp == _brute_top_p(row, p)
        _, tkp = ref.threshold(row, "top_k_top_p", k=k, p=p)
        assert tkp == _brute_top_p(row, p, within=row >= np.float32(_brute_top_k(row, k)))
        _, tm = ref.threshold(row, "min_p", min_p=mp)
        keep = [Fraction(float(x)) >= Fraction(mp) * Fraction(float(row.max()))
                for x in row]
        assert list(ref.kept_mask(row, tm)) == keep


def test_predicate_equals_threshold_indicator():
    """The rejection predicate f(t) of the blog is the indicator [t >= tau]."""
    rng = np.random.default_rng(11)
    for row in _tiny_rows(2, 120):
        k = int(rng.integers(1, row.size + 1))
        p = float(np.float32(rng.choice([0.0, 0.5, 0.8, 1.0, rng.uniform()])))
        mp = float(np.float32(rng.uniform(0, 1)))
        vals = sorted(set(float(x) for x in row) | {0.0})
        probes = vals + [(a + b) / 2 for a, b in zip(vals, vals[1:])]
        for op in ("top_k", "top_p", "min_p", "top_k_top_p", "top_k_top_p_joint"):
            _, tau = ref.threshold(row, op, k=k, p=p, min_p=mp)
            f = ref.Predicate(row, op, k=k, p=p, min_p=mp)
            for t in probes:
                t32 = np.float32(t)
                assert f(t32) == (float(t32) >= tau), (row, op, k, p, mp, t)


def test_joint_order_special_cases():
    """Joint with k >= V is top-p on the row; with p >= 1 it is top-k; joint
    keeps a superset of top-k-then-top-p (its top-p mass target p * Z_C is at
    least p * Z_k)."""
    rng = np.random.default_rng(21)
    for row in _tiny_rows(5, 150):
        k = int(rng.integers(1, row.size + 1))
        p = float(np.float32(rng.choice([0.0, 0.3, 0.7, 1.0, rng.uniform()])))
        _, tj = ref.threshold(row, "top_k_top_p_joint", k=row.size + 3, p=p)
        assert tj == ref.threshold(row, "top_p", p=p)[1]
        _, tj = ref.threshold(row, "top_k_top_p_joint", k=k, p=1.0)
        assert set(np.nonzero(ref.support_mask(row, tj))[0]) == \
            set(np.nonzero(ref.support_mask(row, ref.threshold(row, "top_k", k=k)[1]))[0])
        _, tj = ref.threshold(row, "top_k_top_p_joint", k=k, p=p)
        _, tf = ref.threshold(row, "top_k_top_p", k=k, p=p)
        assert ref.kept_mask(row, tj)[ref.kept_mask(row, tf)].all()


def test_softmax_row_closed_forms_and_scipy():
    """Probabilities from logits: closed forms, shift invariance, the
    temperature as a scale of the logits, and scipy's softmax."""
    from scipy.special import softmax as sp_softmax
    ok, p = ref.softmax_row(f32([0.0, 0.0]), 1.0)
    assert ok and p.tolist() == [0.5, 0.5]
    ok, p = ref.softmax_row(f32([1.0, 0.0]), 1.0)
    e = np.e
    assert np.allclose(p, [e / (1 + e), 1 / (1 + e)], rtol=2 ** -23, atol=0)
    ok, p = ref.softmax_row(f32([3.0, 1.0, -np.inf]), 2.0)   # -inf has probability 0
    assert p[2] == 0 and np.allclose(p[:2], [np.e / (1 + np.e), 1 / (1 + np.e)], rtol=2 ** -23)
    rng = np.random.default_rng(31)
    for _ in range(50):
        z = f32(rng.normal(0, 3, size=int(rng.integers(2, 300))))
        T = float(np.float32(rng.choice([0.25, 0.5, 1.0, 2.0])))   # powers of two: 1/T exact
        ok, p = ref.softmax_row(z, T)
        assert ok and abs(float(p.astype(np.float64).sum()) - 1.0) < z.size * 2 ** -24
        # integer shift: every difference z_i - m is unchanged, so p is too
        ok2, p2 = ref.softmax_row(z + np.float32(8.0), T) if np.abs(z).max() < 1e3 else (True, p)
        assert ok2 and np.array_equal(p, p2) or not np.array_equal(np.float32(z + 8.0) - 8.0, z)
        q = sp_softmax(z.astype(np.float64) / T)
        # one float32 rounding (absolute below the normal range)
        assert np.allclose(p, q, rtol=2 ** -23, atol=2.0 ** -149)


def test_softmax_weights_closed_forms_and_scale_invariance():
    """The unnormalised weights (R21): closed forms, w = 1 at the maximum,
    w / sum(w) equal to the probabilities within float32 rounding, and the
    kept set of top-k-then-top-p unchanged by the missing normaliser on rows
    with well separated values (the filters compare values only with each
    other and with fractions of their sums)."""
    ok, w = ref.softmax_weights(f32([1.0, 0.0, -np.inf]), 1.0)
    assert ok and w[0] == 1.0 and w[2] == 0.0
    assert w[1] == np.float32(np.exp(-1.0))
    ok, w = ref.softmax_weights(f32([0.0, -2.0]), 0.5)           # exp(-4)
    assert w.tolist() == [1.0, float(np.float32(np.exp(-4.0)))]
    rng = np.random.default_rng(37)
    for _ in range(60):
        z = f32(rng.normal(0, 3, size=int(rng.integers(2, 400))))
        T = float(np.float32(rng.uniform(0.3, 2.0)))
        ok, p = ref.softmax_row(z, T)
        ok2, w = ref.softmax_weights(z, T)
        assert ok and ok2 and w.max() == 1.0
        q = w.astype(np.float64) / w.astype(np.float64).sum()
        assert np.allclose(q, p, rtol=2 ** -21, atol=2.0 ** -140)
        # separated values: no two weights within 1e-4 of each other
        ws = np.sort(w[w > 0].astype(np.float64))
        if ws.size > 1 and np.min(np.diff(ws) / ws[1:]) < 1e-4:
            continue
        k = int(rng.integers(1, z.size + 1))
        pp = np.float32(rng.uniform(0.1, 0.99))
        _, tp = ref.threshold(p, "top_k_top_p", k=k, p=pp)
        _, tw = ref.threshold(w, "top_k_top_p", k=k, p=pp)
        margin = ref.top_p_boundary_margin(p, pp, k=k)
        if margin is not None and abs(margin) < 1e-5:
            continue
        assert np.array_equal(ref.support_mask(p, tp), ref.support_mask(w, tw))
    assert ref.softmax_weights(f32([np.nan, 0.0]), 1.0) == (False, None)
    assert ref.softmax_weights(f32([0.0, 1.0]), 0.0) == (False, None)


def test_softmax_row_invalid_inputs():
    for z, T in ((f32([np.nan, 0.0]), 1.0), (f32([np.inf, 0.0]), 1.0),
                 (f32([-np.inf, -np.inf]), 1.0), (f32([0.0, 1.0]), 0.0),
                 (f32([0.0, 1.0]), -1.0), (f32([0.0, 1.0]), np.nan), (f32([0.0, 1.0]), np.inf)):
        assert ref.softmax_row(z, T) == (False, None)


def test_top_k_select_against_sorted_and_heapq():
    """Top-k selection (R19) against Python's sorted() with an explicit key and
    heapq.nlargest, on rows with ties, signed zeros and infinities."""
    import heapq
    rng = np.random.default_rng(41)
    for trial in range(200):
        v = int(rng.integers(1, 60))
        if trial % 3 == 0:
            row = f32(rng.integers(-3, 4, size=v) / 2.0)       # many ties
            row[rng.integers(0, v)] = -0.0
        else:
            row = f32(rng.normal(0, 2, size=v))
            if trial % 7 == 0:
                row[rng.integers(0, v)] = np.inf
                row[rng.integers(0, v)] = -np.inf
        k = int(rng.integers(1, v + 1))
        ok, vals, idx = ref.top_k_select(row, k)
        assert ok
        want = sorted(range(v), key=lambda i: (-(float(row[i]) + 0.0), i))[:k]
        assert list(idx) == want
        assert [float(x) for x in vals] == [float(row[i]) for i in want]
        big = heapq.nlargest(k, ((float(row[i]) + 0.0, -i) for i in range(v)))
        assert [-b for _, b in big] == want
    assert ref.top_k_select(f32([1.0, np.nan]), 1) == (False, None, None)


def test_k_extremes_and_min_p_closed_form():
    rng = np.random.default_rng(3)
    for _ in range(50):
        row = f32(rng.dirichlet(np.ones(9)))
        _, t1 = ref.threshold(row, "top_k", k=1)
        assert list(np.nonzero(ref.kept_mask(row, t1))[0]) == [int(np.argmax(row))]
        _, tv = ref.threshold(row, "top_k", k=row.size)
        assert ref.kept_mask(row, tv).all()
        _, tv = ref.threshold(row, "top_k", k=10 * row.size)
        assert ref.kept_mask(row, tv).all()
        _, tm = ref.threshold(row, "min_p", min_p=0.5)
        assert np.array_equal(ref.kept_mask(row, tm),
                              row.astype(np.float64) >= 0.5 * float(row.max()))
        _, tp0 = ref.threshold(row, "top_p", p=0.0)
        assert ref.kept_mask(row, tp0).sum() == 1
        _, tp1 = ref.threshold(row, "top_p", p=1.0)
        assert np.array_equal(ref.support_mask(row, tp1), row > 0)


def test_invalid_rows_and_parameters():
    good = f32([0.1, 0.2, 0.7])
    for bad in ([0.1, np.nan, 0.9], [0.1, np.inf, 0.2], [0.5, -0.1, 0.6],
                [0.0, 0.0, 0.0], [0.5, -0.0, 0.5]):
        assert not ref.row_is_valid(f32(bad))
        assert ref.threshold(f32(bad), "none") == (False, None)
    assert ref.threshold(good, "top_k", k=0)[0] is False
    assert ref.threshold(good, "top_k", k=-3)[0] is False
    assert ref.threshold(good, "top_p", p=float("nan"))[0] is False
    assert ref.threshold(good, "min_p", min_p=float("nan"))[0] is False
    assert ref.threshold(good, "top_p", p=7.0) == ref.threshold(good, "top_p", p=1.0)
    assert ref.threshold(good, "min_p", min_p=-1.0)[1] == 0.0


# ----------------------------------------------------------------------------
# distribution: p~ closed form, the blog's theorem (the rejection sampler's
# output law equals p_j / Z), and the round-halving property
# ----------------------------------------------------------------------------

def test_target_distribution_closed_form():
    rng = np.random.default_rng(5)
    for _ in range(30):
        row = f32(rng.dirichlet(np.ones(12)))
        k = int(rng.integers(1, 13))
        _, tau = ref.threshold(row, "top_k", k=k)
        # numpy sort/argsort based top-k on tie-free rows
        top = np.argsort(-row.astype(np.float64), kind="stable")[:k]
        expect = np.zeros(row.size)
        expect[top] = row[top].astype(np.float64) / math.fsum(row[top].astype(np.float64))
        assert np.allclose(ref.target_distribution(row, tau), expect, rtol=1e-14, atol=0)


def test_dual_pivot_law_equals_target():
    """Exact enumeration of the dual-pivot procedure gives p~ exactly."""
    rng = np.random.default_rng(8)
    checked = 0
    for row in _tiny_rows(3, 150):
        if row.size > 7:
            continue
        k = int(rng.integers(1, row.size + 1))
        p = float(np.float32(rng.choice([0.0, 0.4, 0.9, 1.0, rng.uniform()])))
        mp = float(np.float32(rng.uniform(0, 1)))
        for op in ref.OPS:
            _, tau = ref.threshold(row, op, k=k, p=p, min_p=mp)
            law, rounds = ref.dual_pivot_law(row, op, k=k, p=p, min_p=mp)
            units = ref.exact_units(row)
            sup = ref.support_mask(row, tau)
            z = sum(u for u, s in zip(units, sup) if s)
            expect = {i: Fraction(units[i], z) for i in range(row.size) if sup[i]}
            assert law == expect, (row, op, k, p, mp)
            assert rounds >= 1
            checked += 1
    assert checked > 300


def test_single_pivot_law_equals_target():
    """Exact enumeration of the single-pivot procedure also gives p~ exactly
    (every rejection only removes values below the kept set)."""
    rng = np.random.default_rng(9)
    checked = 0
    for row in _tiny_rows(4, 120):
        if row.size > 7:
            continue
        k = int(rng.integers(1, row.size + 1))
        p = float(np.float32(rng.choice([0.0, 0.4, 0.9, 1.0, rng.uniform()])))
        mp = float(np.float32(rng.uniform(0, 1)))
        for op in ref.OPS:
            _, tau = ref.threshold(row, op, k=k, p=p, min_p=mp)
            law, rounds = ref.single_pivot_law(row, op, k=k, p=p, min_p=mp)
            units = ref.exact_units(row)
            sup = ref.support_mask(row, tau)
            z = sum(u for u, s_ in zip(units, sup) if s_)
            assert law == {i: Fraction(units[i], z) for i in range(row.size) if sup[i]}
            assert rounds >= 1
            checked += 1
    assert checked > 200


def test_round_halving():
    """Each rejected round at least halves high - low (blog, Fig. 4 text)."""
    rng = np.random.default_rng(9)
    for i in range(40):
        row = f32(rng.dirichlet(np.full(64, 0.3)))
        k = int(rng.integers(1, 8))
        trace = []
        ref.dual_pivot_sample(row, "top_k", ph.Stream(i, 0, 0), k=k, trace=trace)
        for (l0, h0), (l1, h1) in zip(trace, trace[1:]):
            w0 = float(h0) - float(l0)
            w1 = float(h1) - float(l1)
            assert w1 <= w0 / 2 + 2 * np.spacing(np.float32(h0)), trace


def test_dual_pivot_sampler_matches_target_empirically():
    row = f32(golden("expl_top2_example.json")["probs"])
    counts = np.zeros(row.size)
    for i in range(4000):
        j, _ = ref.dual_pivot_sample(row, "top_k", ph.Stream(1234, i, 0), k=2)
        counts[j] += 1
    assert counts[2:].sum() == 0
    _, tau = ref.threshold(row, "top_k", k=2)
    expect = ref.target_distribution(row, tau)[:2] * counts.sum()
    assert stats.chisquare(counts[:2], expect).pvalue > 1e-3


# ----------------------------------------------------------------------------
# inverse transform: exact quadrature on a dyadic row, boundary convention
# F_{k-1} <= u < F_k (blog "逆变换采样")
# ----------------------------------------------------------------------------

def test_inverse_transform_quadrature_and_boundaries():
    row = f32([1 / 8, 3 / 8, 0.0, 1 / 4, 1 / 4])
    mask = row > 0
    counts = np.zeros(row.size, dtype=int)
    for i in range(64):
        counts[ref.inverse_transform(row, mask, i << 47)] += 1    # u = i / 64
    assert list(counts) == [8, 24, 0, 16, 16]
    assert ref.inverse_transform(row, mask, 1 << 50) == 1          # u = F_0 = 1/8
    assert ref.inverse_transform(row, mask, (1 << 50) - 1) == 0
    assert ref.inverse_transform(row, mask, (1 << 53) - 1) == 4
    # unnormalised row: scaling by the masked total
    assert ref.inverse_transform(row * 4, mask, 1 << 50) == 1


def test_plain_cdf_draw_frequencies():
    rng = np.random.default_rng(21)
    row = f32(rng.dirichlet(np.ones(6)))
    n = 6000
    counts = np.zeros(row.size)
    for i in range(n):
        counts[ref.sample_by_cdf(row, "none", ph.draw_bits53(5, i, 0, 0))] += 1
    expect = row.astype(np.float64) / math.fsum(row.astype(np.float64)) * n
    assert stats.chisquare(counts, expect).pvalue > 1e-3


# ----------------------------------------------------------------------------
# renormalisation, logit masking, exact sums
# ----------------------------------------------------------------------------

def test_exact_units_sum_matches_fsum():
    rng = np.random.default_rng(4)
    for _ in range(20):
        row = f32(rng.dirichlet(np.full(5000, 0.1)))
        exact = sum(ref.exact_units(row))
        assert np.ldexp(float(exact), -ref.SCALE_EXP) == math.fsum(row.astype(np.float64))


def test_renorm_against_numpy_topk():
    rng = np.random.default_rng(6)
    for _ in range(20):
        row = f32(rng.dirichlet(np.ones(200)))
        k = int(rng.integers(1, 201))
        valid, out = ref.top_k_renorm(row, k)
        top = np.argsort(-row.astype(np.float64), kind="stable")[:k]
        expect = np.zeros(row.size, dtype=np.float64)
        expect[top] = row[top] / math.fsum(row[top].astype(np.float64))
        assert valid and np.allclose(out, expect, rtol=1e-6, atol=0)
        assert abs(math.fsum(out.astype(np.float64)) - 1.0) < 1e-5
    g = golden("f4_hand_example.json")
    valid, out = ref.top_p_renorm(f32(g["probs"]), g["top_p"])
    x = np.array(g["probs"], dtype=np.float64)
    expect = np.where(np.isin(np.arange(5), g["kept_top_p"]), x, 0) / x[g["kept_top_p"]].sum()
    assert valid and np.allclose(out, expect, rtol=1e-6, atol=0)


def test_renorm_then_plain_equals_filtered_target():
    """renorm + plain sampling has the fused sampler's target distribution
    (explainer, "当前 FlashInfer API 应怎样选择")."""
    rng = np.random.default_rng(12)
    for _ in range(20):
        row = f32(rng.dirichlet(np.ones(50)))
        p = float(np.float32(rng.uniform(0.3, 0.95)))
        _, tau = ref.threshold(row, "top_p", p=p)
        fused = ref.target_distribution(row, tau)
        _, renormed = ref.top_p_renorm(row, p)
        _, t0 = ref.threshold(renormed, "none")
        assert np.allclose(ref.target_distribution(renormed, t0), fused,
                           rtol=1e-6, atol=1e-12)


def test_mask_logits_against_numpy():
    rng = np.random.default_rng(13)
    for _ in range(30):
        row = f32(rng.standard_normal(300) * 3 - 2)      # many negative logits
        k = int(rng.integers(1, 301))
        valid, out = ref.mask_logits_row(row, k)
        top = np.argpartition(-row, k - 1)[:k]
        expect = np.full(row.size, -np.inf, dtype=np.float32)
        expect[top] = row[top]
        assert valid and np.array_equal(out, expect)
    row = f32([-1.0, -3.0, -1.0, -2.0])
    assert np.array_equal(ref.mask_logits_row(row, 1)[1],
                          f32([-1.0, -np.inf, -1.0, -np.inf]))   # ties kept
    assert np.array_equal(ref.mask_logits_row(row, 9)[1], row)
    assert ref.mask_logits_row(f32([0.0, np.nan]), 1)[0] is False
    assert ref.mask_logits_row(row, 0)[0] is False


def test_batch_thresholds_indices():
    probs = np.stack([f32([0.1, 0.2, 0.7]), f32([0.5, 0.25, 0.25])])
    out = ref.batch_thresholds(probs, "top_k", indices=[1, 0, 2, -1], k=[1, 1, 1, 1],
                               num_outputs=4)
    assert out[0] == (True, 0.5) and out[1] == (True, np.float32(0.7))
    assert out[2] == (False, None) and out[3] == (False, None)


# ----------------------------------------------------------------------------
# chain speculative verification (R20)
# ----------------------------------------------------------------------------

def _emitted_law_grid(q0, p0, p1, N=4096):
    """Law of the first emitted token of a one-draft chain, the draft drawn
    from q0, both uniforms integrated on an N-point midpoint grid: the oracle
    is called as a black box, once per (draft, grid point)."""
    V = q0.size
    grid = [((2 * i + 1) << 52) // N for i in range(N)]  # (i + 1/2) / N * 2**53
    q = q0[None, :]
    p = np.stack([p0, p1])
    law = np.zeros(V)
    for d in range(V):
        if q0[d] == 0:
            continue
        acc = 0
        rej_any = None
        for a in grid:
            ok, tok, n_acc = ref.chain_speculative(q, [d], p, [a, grid[0]])
            assert ok
            if n_acc == 1:
                assert tok[0] == d
                acc += 1
            else:
                rej_any = a
        law[d] += float(q0[d]) * acc / N
        if rej_any is not None:
            res = np.zeros(V)
            for b in grid:
                ok, tok, n_acc = ref.chain_speculative(q, [d], p, [rej_any, b])
                assert ok and n_acc == 0 and tok[1] == -1
                res[tok[0]] += 1.0 / N
            law += float(q0[d]) * (N - acc) / N * res
    return law


@pytest.mark.parametrize("case", range(3))
def test_chain_speculative_preserves_target_law(case):
    """Leviathan, Kalman & Matias 2023 (Theorem / appendix A.1), Chen et al.
    2023 (Theorem 1): with the draft drawn from q, the emitted token is
    distributed exactly as p.  A wrong acceptance test or a residual other
    than max(0, p - q) moves the law by far more than the grid error."""
    rng = np.random.default_rng(500 + case)
    V = 6
    q0 = rng.dirichlet(np.ones(V) * 0.7).astype(np.float32)
    p0 = rng.dirichlet(np.ones(V) * 0.7).astype(np.float32)
    if case == 2:
        q0[3] = 0.0                          # a token the draft never proposes
        p0[5] = 0.0                          # and one the target never emits
        q0 = (q0 / q0.astype(np.float64).sum()).astype(np.float32)
        p0 = (p0 / p0.astype(np.float64).sum()).astype(np.float32)
    p1 = rng.dirichlet(np.ones(V)).astype(np.float32)
    law = _emitted_law_grid(q0, p0, p1)
    target = p0.astype(np.float64) / p0.astype(np.float64).sum()
    # the draft law is q0 / sum(q0), which sums to one up to float32 rounding
    assert np.abs(law / law.sum() - target).max() < 3.0 / 4096, (law, target)


def test_chain_speculative_identical_models_accept_everything():
    """q = p: u * q < p for every u < 1, so every draft is accepted and the
    bonus token is the inverse-transform draw from p_n."""
    rng = np.random.default_rng(7)
    n, V = 5, 40
    p = rng.dirichlet(np.ones(V), size=n + 1).astype(np.float32)
    ids = rng.integers(0, V, size=n)
    for a_fin in (0, 1 << 52, (1 << 53) - 1):
        a53s = [int(x) for x in rng.integers(0, 1 << 53, size=n, dtype=np.uint64)] + [a_fin]
        ok, tok, acc = ref.chain_speculative(p[:n], ids, p, a53s)
        assert ok and acc == n
        assert list(tok[:n]) == list(ids)
        assert tok[n] == ref.CdfTable(p[n], p[n] > 0).draw(a_fin)


def test_chain_speculative_one_hot_draft():
    """q_0 = e_d: the draft is accepted iff u < p(d); on rejection the
    residual max(0, p - e_d) is p without token d (closed form)."""
    p0 = np.array([0.125, 0.5, 0.25, 0.125], dtype=np.float32)
    p = np.stack([p0, p0])
    q = np.zeros((1, 4), dtype=np.float32)
    d = 1
    q[0, d] = 1.0
    half = 1 << 52                                    # u = 1/2 = p(d)
    assert ref.chain_speculative(q, [d], p, [half - 1, 0])[2] == 1
    ok, tok, acc = ref.chain_speculative(q, [d], p, [half, 0])
    assert ok and acc == 0
    without = p0.copy()
    without[d] = 0
    for a in (0, 1 << 51, 3 << 51, (1 << 53) - 1):
        tok = ref.chain_speculative(q, [d], p, [half, a])[1]
        assert tok[0] == ref.CdfTable(without, without > 0).draw(a)
        assert tok[0] != d


def test_chain_speculative_zero_target_and_zero_residual():
    """p(d) = 0 rejects for every u (even u = 0); a residual that is zero
    everywhere (p <= q, an unnormalised p) falls back to a draw from p."""
    q = np.array([[0.25, 0.25, 0.5]], dtype=np.float32)
    p = np.array([[0.0, 0.5, 0.5], [1.0, 0.0, 0.0]], dtype=np.float32)
    ok, tok, acc = ref.chain_speculative(q, [0], p, [0, 0])
    assert ok and acc == 0 and tok[0] in (1, 2)
    ph_ = np.array([[0.125, 0.125, 0.25]], dtype=np.float32)   # p = q / 2
    pp = np.concatenate([ph_, p[1:]])
    ok, tok, acc = ref.chain_speculative(q, [2], pp, [1 << 52, 1 << 52])  # u = 1/2: rejected
    assert ok and acc == 0
    assert tok[0] == ref.CdfTable(ph_[0], ph_[0] > 0).draw(1 << 52)
    assert ref.chain_speculative(q, [2], pp, [(1 << 52) - 1, 0])[2] == 1


def test_chain_speculative_two_positions_monte_carlo():
    """A chain of two drafts with the drafts drawn from q: the token emitted
    at position 1, given position 0 accepted its draft, follows p_1; the
    bonus, given both accepted, follows p_2 (chi-square, 20000 chains)."""
    rng = np.random.default_rng(11)
    V = 5
    q = rng.dirichlet(np.ones(V), size=2).astype(np.float32)
    p = rng.dirichlet(np.ones(V), size=3).astype(np.float32)
    pos1, bonus = np.zeros(V), np.zeros(V)
    cq = np.cumsum(q.astype(np.float64), axis=1)
    for _ in range(20000):
        ids = [min(int(np.searchsorted(cq[j], rng.random() * cq[j, -1], side="right")), V - 1)
               for j in range(2)]
        a53s = [int(x) for x in rng.integers(0, 1 << 53, size=3, dtype=np.uint64)]
        ok, tok, acc = ref.chain_speculative(q, ids, p, a53s)
        assert ok
        if acc >= 1:
            pos1[tok[1]] += 1
        if acc == 2:
            bonus[tok[2]] += 1
    for counts, row in ((pos1, p[1]), (bonus, p[2])):
        expect = counts.sum() * row.astype(np.float64) / row.astype(np.float64).sum()
        assert stats.chisquare(counts, expect).pvalue > 1e-3


def test_chain_speculative_invalid_rows():
    q = np.array([[0.5, 0.5, 0.0]], dtype=np.float32)
    p = np.array([[0.25, 0.75, 0.0], [0.5, 0.5, 0.0]], dtype=np.float32)
    for ids in ([-1], [3]):                                  # draft id outside [0, V)
        assert not ref.chain_speculative(q, ids, p, [0, 0])[0]
    pn = p.copy()
    pn[0, 2] = np.nan                                        # in the rejected row
    assert not ref.chain_speculative(q, [0], pn, [(1 << 53) - 1, 0])[0]
    assert ref.chain_speculative(q, [0], pn, [0, 0])[0]      # accepted: row not read
    pz = p.copy()
    pz[1, 2] = -0.0                                          # in the bonus row
    assert not ref.chain_speculative(q, [0], pz, [0, 0])[0]
    p0 = p.copy()
    p0[1] = 0.0                                              # bonus row with no mass
    ok, tok, acc = ref.chain_speculative(q, [0], p0, [0, 0])
    assert not ok and list(tok) == [-1, -1] and acc == 0


# ----------------------------------------------------------------------------
# pivot2 = (pivot1 + high) / 2 (blog "双枢轴拒绝采样"), traced on the A..E
# top-2 row of the explainer ("一个简化的 top-k 例子").  The output law does
# not depend on where pivot2 sits, so only the trace of (low, high) can tell
# the pages' midpoint from another one (e.g. (low + high) / 2).
# ----------------------------------------------------------------------------

class _Scripted:
    """A draw stream that returns the given uniforms u as 53-bit integers."""

    def __init__(self, us):
        self.a53 = [int(u * 2.0**53) for u in us]

    def next(self):
        return self.a53.pop(0)


def _mid(a, b):
    return np.float32((np.float64(np.float32(a)) + np.float64(np.float32(b))) / 2)


def test_dual_pivot_trace_first_draw_d():
    """k = 2, first draw D (u = .87 lies in [F_C, F_D) = [.81, .93)):
    pivot1 = .12 is rejected (three values exceed it); pivot2 = (.12 + .35) / 2
    = .235 is rejected too (#{x > .235} = 2 is not below k), so low moves to
    .235 and high stays .35; then A (u = .1 among A, B) is accepted."""
    row = f32(golden("expl_top2_example.json")["probs"])
    trace = []
    j, rounds = ref.dual_pivot_sample(row, "top_k", _Scripted([0.87, 0.1]), k=2, trace=trace)
    assert (j, rounds) == (0, 2)
    assert trace == [(np.float32(0), np.float32(0.35)), (_mid(0.12, 0.35), np.float32(0.35))]
    assert abs(float(trace[1][0]) - 0.235) < 1e-7


def test_dual_pivot_trace_second_case():
    """k = 3 (tau = .18), first draw E (u = .96): pivot1 = .07 is rejected
    (four values exceed it) but pivot2 = (.07 + .35) / 2 = .21 passes
    (#{x > .21} = 2 < 3), so (low, high) becomes (.07, .21).  The next draw
    D (.12, u = .9 of the mass above .07) is rejected and pivot2 =
    (.12 + .21) / 2 = .165 fails (#{x > .165} = 3), so low moves to .165;
    then A is accepted."""
    row = f32(golden("expl_top2_example.json")["probs"])
    trace = []
    j, rounds = ref.dual_pivot_sample(row, "top_k", _Scripted([0.96, 0.9, 0.05]), k=3,
                                      trace=trace)
    assert (j, rounds) == (0, 3)
    assert trace[0] == (np.float32(0), np.float32(0.35))
    assert trace[1] == (np.float32(0.07), _mid(0.07, 0.35))
    assert trace[2] == (_mid(0.12, _mid(0.07, 0.35)), _mid(0.07, 0.35))
    assert abs(float(trace[1][1]) - 0.21) < 1e-7 and abs(float(trace[2][0]) - 0.165) < 1e-7


# ----------------------------------------------------------------------------
# the law of the round count, worked by hand on the A..E row of the explainer
# ("一个简化的 top-k 例子") with the update of the blog ("双枢轴拒绝采样")
# ----------------------------------------------------------------------------

def test_rounds_law_top2_by_hand():
    """k = 2: A or B is accepted at once (mass .63).  C, D or E is rejected,
    and its pivot2 (.265, .235 or .21) still has two values above it, so low
    moves to pivot2 with only A and B left: exactly two rounds (mass .37)."""
    row = f32(golden("expl_top2_example.json")["probs"])
    u = ref.exact_units(row)
    z = sum(u)
    law = ref.dual_pivot_rounds_law(row, "top_k", k=2)
    assert law == {1: Fraction(u[0] + u[1], z), 2: Fraction(u[2] + u[3] + u[4], z)}
    assert abs(float(law[2]) - 0.37) < 1e-7


def test_rounds_law_top3_by_hand():
    """k = 3: A, B, C accepted at once (.81).  D: pivot2 = .235 passes, so
    (low, high) = (.12, .235) and A, B or C is taken next: two rounds.  E:
    pivot2 = .21 passes, (low, high) = (.07, .21); next A, B, C (mass .81 of
    .93) end at two rounds, D (.12 of .93) is rejected again, pivot2 = .165
    fails, low = .165, and the third round accepts."""
    row = f32(golden("expl_top2_example.json")["probs"])
    u = ref.exact_units(row)
    z = sum(u)
    above07 = u[0] + u[1] + u[2] + u[3]
    law = ref.dual_pivot_rounds_law(row, "top_k", k=3)
    p_e = Fraction(u[4], z)
    assert law == {1: Fraction(u[0] + u[1] + u[2], z),
                   2: Fraction(u[3], z) + p_e * Fraction(u[0] + u[1] + u[2], above07),
                   3: p_e * Fraction(u[3], above07)}
    assert abs(float(law[3]) - 0.07 * 0.12 / 0.93) < 1e-7


def test_rounds_law_sums_to_one_and_matches_expectation():
    """On random tiny rows the round law is a probability law whose mean is
    the expected round count of the exact output-law enumeration."""
    rng = np.random.default_rng(17)
    checked = 0
    for row in _tiny_rows(5, 60):
        if row.size > 7:
            continue
        k = int(rng.integers(1, row.size + 1))
        p = float(np.float32(rng.uniform(0.2, 0.95)))
        for op in ("top_k", "top_p", "top_k_top_p"):
            law = ref.dual_pivot_rounds_law(row, op, k=k, p=p)
            _, mean = ref.dual_pivot_law(row, op, k=k, p=p)
            if not law:
                continue
            assert sum(law.values()) == 1
            assert sum(r * q for r, q in law.items()) == mean
            checked += 1
    assert checked > 50
