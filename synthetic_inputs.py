"""Seeded synthetic workloads for the sampling ops.

This module only generates inputs (probability rows, per-output parameters,
seeds, index maps).  It holds none of the filtering or sampling arithmetic,
so both the oracle tests and the GPU tests/bench can use it without sharing
any of the method's code.  All math is float64, cast once to float32 with
round-to-nearest; every array is C-contiguous.

Workloads (shapes, value distributions and parameter mixes as named):

  small     B=4,   V=32000,  probs = softmax(z), z ~ N(0, 3^2); top_k=50,
            top_p=0.9 on every row
  renorm    B=64,  V=151936, probs = softmax(N(0, 2^2)); per row
            top_p ~ U[0.5, 0.95], top_k ~ U{1..1024}   (also the headline
            fused top-k-then-top-p sampling workload)
  latency   B=1,   V=151936, softmax(N(0, 2^2)); top_k=50, top_p=0.9
  hetero    B=256, V=128256, Zipf-shaped weights rank^-1.1 x lognormal(0, 0.5)
            noise, randomly permuted; per row k ~ U{1..V}, p ~ U[0.1, 1],
            min_p ~ U[0, 0.2]; 512 outputs (each row twice, shuffled), each
            assigned one of {top_k_top_p, min_p, plain}
  stress    B=512, V=256000 in three groups (171/171/170 rows): near-uniform
            (1 + U[-1e-3, 1e-3]) / V; peaked (0.99 at one random id, the rest
            equal); geometric chain p_i ~ (1 - 1e-6)^i; top_k=1000, top_p=0.95
  speculative  B=64, n=4 draft tokens, V=151936: draft logits z_j ~ N(0, 2^2),
            target logits z_j + N(0, 0.5^2) (position n: fresh N(0, 2^2)),
            q_j = softmax(draft), p_j = softmax(target); draft tokens drawn
            from q_j with numpy's generator (an input, not the verifier);
            per-row seeds
"""

import numpy as np

BASE_SEED = 20261202
CFG_IDS = {"small": 1, "renorm": 2, "latency": 3, "hetero": 4, "stress": 5,
           "speculative": 6}


def rng_for(cfg, rep=0):
    return np.random.default_rng(BASE_SEED + 100 * CFG_IDS[cfg] + rep)


def softmax_rows(rng, rows, vocab, sigma):
    """float32 rows of softmax(z), z ~ N(0, sigma^2) iid (float64 math)."""
    z = rng.standard_normal((rows, vocab)) * sigma
    z -= z.max(axis=1, keepdims=True)
    e = np.exp(z)
    e /= e.sum(axis=1, keepdims=True)
    return np.ascontiguousarray(e.astype(np.float32))


def seeds_for(rng, n):
    return rng.integers(0, np.iinfo(np.uint64).max, size=n, dtype=np.uint64,
                        endpoint=True)


def small(rep=0):
    rng = rng_for("small", rep)
    probs = softmax_rows(rng, 4, 32000, 3.0)
    return dict(probs=probs, top_k=50, top_p=np.float32(0.9),
                seeds=seeds_for(rng, 4), offset=0)


def renorm(rep=0, rows=64, vocab=151936):
    rng = rng_for("renorm", rep)
    probs = softmax_rows(rng, rows, vocab, 2.0)
    top_p = rng.uniform(0.5, 0.95, size=rows).astype(np.float32)
    top_k = rng.integers(1, 1024, size=rows, endpoint=True).astype(np.int32)
    return dict(probs=probs, top_p=top_p, top_k=top_k,
                seeds=seeds_for(rng, rows), offset=0)


def latency(rep=0):
    rng = rng_for("latency", rep)
    probs = softmax_rows(rng, 1, 151936, 2.0)
    return dict(probs=probs, top_k=50, top_p=np.float32(0.9),
                seeds=seeds_for(rng, 1), offset=0)


def hetero(rep=0, rows=256, vocab=128256):
    rng = rng_for("hetero", rep)
    rank = np.arange(1, vocab + 1, dtype=np.float64)
    w = rank[None, :] ** -1.1 * rng.lognormal(0.0, 0.5, size=(rows, vocab))
    for r in range(rows):
        w[r] = w[r, rng.permutation(vocab)]
    probs = np.ascontiguousarray((w / w.sum(axis=1, keepdims=True))
                                 .astype(np.float32))
    top_k = rng.integers(1, vocab, size=rows, endpoint=True).astype(np.int32)
    top_p = rng.uniform(0.1, 1.0, size=rows).astype(np.float32)
    min_p = rng.uniform(0.0, 0.2, size=rows).astype(np.float32)
    n_out = 2 * rows
    indices = rng.permutation(np.repeat(np.arange(rows, dtype=np.int32), 2))
    op_of_output = rng.integers(0, 3, size=n_out)       # 0 top_k_top_p, 1 min_p, 2 plain
    return dict(probs=probs, top_k=top_k, top_p=top_p, min_p=min_p,
                indices=indices.astype(np.int32), op_of_output=op_of_output,
                seeds=seeds_for(rng, n_out), offset=0)


def stress(rep=0, rows=512, vocab=256000):
    rng = rng_for("stress", rep)
    g1 = (rows + 2) // 3
    g2 = (rows + 1) // 3
    out = np.empty((rows, vocab), dtype=np.float64)
    out[:g1] = (1.0 + rng.uniform(-1e-3, 1e-3, size=(g1, vocab))) / vocab
    peaked = np.full((g2, vocab), 0.01 / (vocab - 1))
    peaked[np.arange(g2), rng.integers(0, vocab, size=g2)] = 0.99
    out[g1:g1 + g2] = peaked
    out[g1 + g2:] = (1.0 - 1e-6) ** np.arange(vocab, dtype=np.float64)[None, :]
    out /= out.sum(axis=1, keepdims=True)
    groups = np.repeat(np.array([0, 1, 2]), [g1, g2, rows - g1 - g2])
    return dict(probs=np.ascontiguousarray(out.astype(np.float32)),
                top_k=1000, top_p=np.float32(0.95), groups=groups,
                seeds=seeds_for(rng, rows), offset=0)


def logits_rows(rng, rows, vocab, sigma=2.0):
    """float32 logits z ~ N(0, sigma^2) for the logit-masking op."""
    return np.ascontiguousarray((rng.standard_normal((rows, vocab)) * sigma)
                                .astype(np.float32))


def speculative(rep=0, rows=64, n=4, vocab=151936, sigma=2.0, noise=0.5):
    """Draft / target distributions and draft tokens for chain verification."""
    rng = rng_for("speculative", rep)
    zq = rng.standard_normal((rows, n, vocab)) * sigma
    zp = np.empty((rows, n + 1, vocab))
    zp[:, :n] = zq + rng.standard_normal((rows, n, vocab)) * noise
    zp[:, n] = rng.standard_normal((rows, vocab)) * sigma

    def sm(z):
        z = z - z.max(axis=-1, keepdims=True)
        e = np.exp(z)
        return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)
    q, p = sm(zq), sm(zp)
    del zq, zp
    cq = np.cumsum(q.astype(np.float64), axis=-1)
    u = rng.random((rows, n, 1)) * cq[:, :, -1:]
    ids = np.minimum((cq <= u).sum(axis=-1), vocab - 1).astype(np.int32)
    return dict(q=np.ascontiguousarray(q), p=np.ascontiguousarray(p),
                ids=np.ascontiguousarray(ids), seeds=seeds_for(rng, rows), offset=0)

