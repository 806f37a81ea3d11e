"""Throughput of fused top-k-then-top-p sampling on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--engine auto|streaming|from_zero]

One step = one call of top_k_top_p_sampling_from_probs over a batch of
B=64 rows of V=151936 float32 probabilities (softmax of N(0, 2^2) logits),
per-row top_k ~ U{1..1024} and top_p ~ U[0.5, 0.95], one sampled token per
row.  Inputs are resident in HBM before the timed region; the headline is
cold-cache: 16 distinct input buffers (622 MB, beyond the 256 MB Infinity
Cache) are used round-robin.

Two timed loops on the same stream:
  * steps: K calls back to back between two HIP events -> ms_per_step and
    `value` (sampled rows per second, launch gaps included);
  * kernel: K more calls with the library's dispatch-event hook
    (dss_set_timing_events, hipExtLaunchKernel start/stop events on the
    kernel itself) -> the average kernel duration, the figure a kernel-trace
    profiler reports, from which roofline.achieved is computed.
Beside the headline: a plain read of the same cold batch (the achievable
read rate), the other workloads (warm: one resident buffer; cold: 16
rotating buffers), the latency row at 4, 8 and 16 slices per row, and the
oracle timed on the host's cores (a process pool forked before the first GPU
call).  ``--phase-stamps`` instead prints the per-phase timeline of the
headline kernel from the measurement build libdss_stamps.so.
Prints one JSON line on stdout; details go to stderr.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sampled rows/s + achieved HBM GB/s, fused top-k/top-p, B=64 V=151936 fp32"
HBM_PEAK_GBS = 8000.0
N_BUFFERS = 16
KERNEL_SOURCES = ["decode_step_sampling_amd/csrc/split_kernels.hip",
                  "decode_step_sampling_amd/csrc/split_device.h",
                  "decode_step_sampling_amd/csrc/stream_device.h",
                  "decode_step_sampling_amd/csrc/dss_device.h",
                  "decode_step_sampling_amd/csrc/dss_internal.h"]
TRAFFIC_FILE = "profiles/split_sample_topk_topp_B64_V151936_traffic.md"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel sources have changed since the counters were taken."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel source hash:\s*`?([0-9a-f]+)", text)
    val = re.search(r"traffic bytes per launch:\s*`?([0-9.e+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


# ----------------------------------------------------------------------------
# the oracle on the host's cores
# ----------------------------------------------------------------------------

_CPU = {}   # workload arrays, set before the pool forks (shared copy-on-write)


def _oracle_rows(task):
    """Worker: the oracle on `count` outputs of one workload, starting at
    output `start` (cycling); returns the number of outputs done."""
    from oracle import philox as ph
    from oracle import reference as ref
    name, start, count, rep = task
    d = _CPU[name]
    n = d["n"]
    for t in range(start, start + count):
        i = t % n
        if name == "renorm":       # top-p and top-k renormalisation of one row
            ref.top_p_renorm(d["probs"][i], d["top_p"][i])
            ref.top_k_renorm(d["probs"][i], d["top_k"][i])
            continue
        row = d["probs"][d["row_of"][i]]
        a53 = ph.draw_bits53(int(d["seeds"][i]), rep, 0, 0)
        op = d["op"][i]
        ref.sample_by_cdf(row, op, a53, k=d["k"][i], p=d["p"][i], min_p=d["mp"][i])
    return count


def cpu_workloads(si, names):
    """The host arrays of each workload the oracle is timed on (output-major)."""
    out = {}
    for name in names:
        if name == "headline":
            w = si.renorm()
            n = w["probs"].shape[0]
            out[name] = dict(n=n, probs=w["probs"], row_of=np.arange(n), seeds=w["seeds"],
                             op=["top_k_top_p"] * n, k=w["top_k"], p=w["top_p"], mp=[None] * n,
                             vocab=w["probs"].shape[1], what="fused top-k/top-p draw per row")
        elif name == "renorm":
            w = si.renorm()
            n = w["probs"].shape[0]
            out[name] = dict(n=n, probs=w["probs"], top_p=w["top_p"], top_k=w["top_k"],
                             vocab=w["probs"].shape[1],
                             what="top_p_renorm + top_k_renorm of one row")
        elif name == "latency":
            w = si.latency()
            out[name] = dict(n=1, probs=w["probs"], row_of=[0], seeds=w["seeds"],
                             op=["top_k_top_p"], k=[w["top_k"]], p=[w["top_p"]], mp=[None],
                             vocab=w["probs"].shape[1], what="fused top-k/top-p draw (k=50, p=0.9)")
        elif name == "hetero":
            w = si.hetero()
            idx = w["indices"]
            ops = [("top_k_top_p", "min_p", "none")[o] for o in w["op_of_output"]]
            out[name] = dict(n=len(idx), probs=w["probs"], row_of=idx, seeds=w["seeds"], op=ops,
                             k=w["top_k"][idx], p=w["top_p"][idx], mp=w["min_p"][idx],
                             vocab=w["probs"].shape[1],
                             what="one output of the mixed top-k/top-p, min-p, plain batch")
        elif name == "stress":
            w = si.stress()
            n = w["probs"].shape[0]
            out[name] = dict(n=n, probs=w["probs"], row_of=np.arange(n), seeds=w["seeds"],
                             op=["top_k_top_p"] * n, k=[w["top_k"]] * n, p=[w["top_p"]] * n,
                             mp=[None] * n, vocab=w["probs"].shape[1],
                             what="fused top-k/top-p draw (k=1000, p=0.95)")
    return out


def cpu_pool():
    """Worker processes for the oracle: one per core of the machine's CPU share
    (at most 16), forked now, before any GPU call."""
    import multiprocessing as mp
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    n = max(1, min(16, avail))
    return mp.get_context("fork").Pool(n, initializer=_one_thread), n


def _one_thread():
    """Each oracle process runs single-threaded (no hidden thread pools)."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(pool, ncores, names, per_core=(("headline", 48), ("renorm", 8),
                                                ("latency", 32), ("hetero", 24),
                                                ("stress", 16))):
    """The oracle as it stands (sort-based filter + exact CDF draw, or the
    renormalisation), timed on the host: for every workload, five runs on all
    `ncores` worker processes (each doing `count` outputs) and five on one,
    the median of each; outputs per second and the equivalent GB/s of one
    read of each output's row."""
    import statistics
    res = {}
    pool.map(_oracle_rows, [("latency", 0, 1, 0)] * ncores, chunksize=1)   # imports in every worker
    for name, count in per_core:
        if name not in names:
            continue
        d = _CPU[name]
        row_bytes = 4 * d["vocab"] * (2 if name == "renorm" else 1)

        def timed(ntasks, rep):
            tasks = [(name, (rep * 7919 + j * count) % d["n"], count, rep) for j in range(ntasks)]
            t0 = time.perf_counter()
            done = sum(pool.map(_oracle_rows, tasks, chunksize=1))
            return done / (time.perf_counter() - t0)

        multi = statistics.median(timed(ncores, r) for r in range(5))
        single = statistics.median(timed(1, r) for r in range(5))
        res[name] = {"all_cores": {"value": multi, "GBps": multi * row_bytes / 1e9},
                     "one_core": {"value": single, "GBps": single * row_bytes / 1e9},
                     "unit": "outputs/s", "sample": f"{count} outputs per process per run, "
                     f"median of 5 runs ({d['what']})"}
    return res


QUICK = [False]   # --quick: a few calls per workload (for counter runs under a profiler)


def kernel_times(lib, fn, reps, warm=2):
    """Per-call kernel time in us of fn() (dispatch-event hook), reps calls."""
    import torch
    if QUICK[0]:
        reps, warm = min(reps, 4), min(warm, 1)
    for _ in range(warm):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        b.record()
    torch.cuda.synchronize()
    for a, b in ev:
        lib.dss_set_timing_events(a.cuda_event, b.cuda_event)
        fn()
    lib.dss_set_timing_events(None, None)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) * 1e3 for a, b in ev])


def reference_points(lib, bufs, steps):
    """Context beside the headline, on the same cold rotating buffers: a plain
    HIP streaming read of the batch (dss_stream_read_reference: one pass,
    38.9 MB per step, five 16-byte loads in flight per thread) as the read
    rate this GPU reaches at this size, and torch.sort of one batch (the sort
    the sorting-free method avoids)."""
    import torch
    nb = len(bufs)
    out = torch.zeros(1, dtype=torch.int32, device=bufs[0].device)
    stream = torch.cuda.current_stream(bufs[0].device).cuda_stream
    n = bufs[0].numel()

    def read(i):
        if lib.dss_stream_read_reference(bufs[i % nb].data_ptr(), n, out.data_ptr(), stream) != 0:
            raise RuntimeError("stream read reference failed")

    # kernel time through the dispatch-event hook, like the headline's kernel_us
    # (back-to-back calls from Python would be launch-bound for a read this short)
    cnt = [0]

    def step():
        read(cnt[0])
        cnt[0] += 1

    us = float(kernel_times(lib, step, steps, warm=10).mean())
    nbytes = n * 4
    for _ in range(3):
        torch.sort(bufs[0], dim=-1, descending=True)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for i in range(10):
        torch.sort(bufs[i % nb], dim=-1, descending=True)
    s1.record()
    torch.cuda.synchronize()
    return {"stream_read": {"op": "dss_stream_read_reference over the batch, cold rotating buffers",
                            "kernel_us": us, "GBps": nbytes / (us * 1e-6) / 1e9,
                            "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS},
            "torch_sort_us": s0.elapsed_time(s1) * 1e3 / 10}


def extra_configs(dss, si, lib, dev):
    """The other workloads of the sampling path, one line each: kernel time
    per call (mean, and p50/p99 where the workload is a latency case) and the
    fraction of the 8 TB/s roofline for the op's algorithmic bytes (one read
    of each output's row; read + write for renorm and masking)."""
    import torch

    def g(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def entry(t, nbytes, **kw):
        d = {"kernel_us": float(t.mean()), "algorithmic_bytes": int(nbytes),
             "hbm_frac": nbytes / (t.mean() * 1e-6) / (HBM_PEAK_GBS * 1e9)}
        d.update(kw)
        return d

    out = {}
    w = si.small()
    P = g(w["probs"])
    B, V = P.shape
    t = kernel_times(lib, lambda: dss.top_k_top_p_sampling_from_probs(P, 50, 0.9, seed=1, offset=0),
                     200)
    out["small B=4 V=32000 top_k_top_p (k=50, p=0.9)"] = entry(
        t, B * V * 4, p50_us=float(np.percentile(t, 50)), p99_us=float(np.percentile(t, 99)))
    w = si.renorm()
    P = g(w["probs"])
    B, V = P.shape
    k, p = g(w["top_k"]), g(w["top_p"])
    out["renorm B=64 V=151936 top_p_renorm_probs"] = entry(
        kernel_times(lib, lambda: dss.top_p_renorm_probs(P, p), 10), 2 * B * V * 4)
    out["renorm B=64 V=151936 top_k_renorm_probs"] = entry(
        kernel_times(lib, lambda: dss.top_k_renorm_probs(P, k), 50), 2 * B * V * 4)
    # the same two ops cold: 16 rotating input buffers, 16 output buffers
    Pc = [P.clone() for _ in range(N_BUFFERS)]
    Oc = [torch.empty_like(P) for _ in range(N_BUFFERS)]
    cnt = [0]

    def rot(fn):
        def step():
            j = cnt[0] % N_BUFFERS
            cnt[0] += 1
            fn(Pc[j], Oc[j])
        return step
    out["renorm B=64 V=151936 top_p_renorm_probs, cold (16 buffers)"] = entry(
        kernel_times(lib, rot(lambda x, o: dss.top_p_renorm_probs(x, p, out=o)), 50, 4),
        2 * B * V * 4)
    out["renorm B=64 V=151936 top_k_renorm_probs, cold (16 buffers)"] = entry(
        kernel_times(lib, rot(lambda x, o: dss.top_k_renorm_probs(x, k, out=o)), 50, 4),
        2 * B * V * 4)
    del Pc, Oc
    L = g(si.logits_rows(np.random.default_rng(1), B, V))
    out["logits B=64 V=151936 top_k_mask_logits"] = entry(
        kernel_times(lib, lambda: dss.top_k_mask_logits(L, k), 50), 2 * B * V * 4)
    out["probs B=64 V=151936 sampling_from_probs"] = entry(
        kernel_times(lib, lambda: dss.sampling_from_probs(P, seed=1, offset=0), 50), B * V * 4)
    out["probs B=64 V=151936 top_p_sampling_from_probs"] = entry(
        kernel_times(lib, lambda: dss.top_p_sampling_from_probs(P, p, seed=1, offset=0), 10),
        B * V * 4)
    out["probs B=64 V=151936 min_p_sampling_from_probs (0.05)"] = entry(
        kernel_times(lib, lambda: dss.min_p_sampling_from_probs(P, 0.05, seed=1, offset=0), 10),
        B * V * 4)
    Lg = g(si.logits_rows(np.random.default_rng(2), B, V, 2.0))
    out["logits B=64 V=151936 softmax (T=0.8)"] = entry(
        kernel_times(lib, lambda: dss.softmax(Lg, 0.8), 50), 2 * B * V * 4)
    out["logits B=64 V=151936 top_k_top_p_sampling_from_logits (T=0.8; softmax fused into the sampling kernel)"] = entry(
        kernel_times(lib, lambda: dss.top_k_top_p_sampling_from_logits(Lg, k, p, 0.8, seed=1, offset=0), 50),
        B * V * 4)
    Lc = [Lg.clone() for _ in range(N_BUFFERS)]
    cnt = [0]

    def logits_cold():
        x = Lc[cnt[0] % N_BUFFERS]
        cnt[0] += 1
        dss.top_k_top_p_sampling_from_logits(x, k, p, 0.8, seed=1, offset=0)
    out["logits B=64 V=151936 top_k_top_p_sampling_from_logits (T=0.8; fused), cold (16 buffers)"] = entry(
        kernel_times(lib, logits_cold, 50, 4), B * V * 4)
    del Lc
    for kk in (50, 1024):
        out[f"logits B=64 V=151936 top_k selection (k={kk}; values + indices)"] = entry(
            kernel_times(lib, lambda: dss.top_k(Lg, kk), 50), B * V * 4 + B * kk * 8)
    # chain speculative verification: one read of the two rows a rejection
    # draws from (p_j*, q_j*), or of p_n for the bonus token, per row
    w = si.speculative()
    Q, Ids, Pt = g(w["q"]), g(w["ids"]), g(w["p"])
    Sd = g(w["seeds"].view(np.int64))
    t = kernel_times(lib, lambda: dss.chain_speculative_sampling(Q, Ids, Pt, seed=Sd, offset=0), 50)
    _, acc = dss.chain_speculative_sampling(Q, Ids, Pt, seed=Sd, offset=0)
    acc = acc.cpu().numpy()
    nd = w["ids"].shape[1]
    Vs = w["p"].shape[2]
    nbytes = int(sum(8 * Vs if a < nd else 4 * Vs for a in acc))
    out["speculative B=64 n=4 V=151936 chain_speculative_sampling"] = entry(
        t, nbytes, mean_accepted=float(acc.mean()), rejected_rows=int((acc < nd).sum()))
    del Q, Pt
    w = si.latency()
    P = g(w["probs"])
    t = kernel_times(lib, lambda: dss.top_k_top_p_sampling_from_probs(P, 50, 0.9, seed=3,
                                                                       offset=0), 1000, 20)
    out["latency B=1 V=151936 top_k_top_p (k=50, p=0.9), 1000 calls"] = entry(
        t, 151936 * 4, p50_us=float(np.percentile(t, 50)), p95_us=float(np.percentile(t, 95)),
        p99_us=float(np.percentile(t, 99)), slices=16)
    # the same row at other slice counts (dss_set_split_slices; the engine's
    # own choice is 16, its largest; 32 slices of one row do not exist)
    sweep = {}
    for W in (4, 8, 16):
        lib.dss_set_split_slices(W)
        try:
            t = kernel_times(lib, lambda: dss.top_k_top_p_sampling_from_probs(
                P, 50, 0.9, seed=3, offset=0), 1000, 20)
        finally:
            lib.dss_set_split_slices(0)
        sweep[str(W)] = {"p50_us": float(np.percentile(t, 50)), "p95_us": float(np.percentile(t, 95)),
                         "p99_us": float(np.percentile(t, 99)), "mean_us": float(t.mean())}
    best = min(sweep, key=lambda x: sweep[x]["p50_us"])
    out["latency B=1 V=151936 slices per row sweep (p50/p95/p99 over 1000 calls)"] = {
        "slices": sweep, "best": int(best), "32": "not available (at most 16 slices per row)"}
    w = si.hetero()
    P = g(w["probs"])
    B, V = P.shape
    idx, op, seeds = w["indices"], w["op_of_output"], w["seeds"]
    step, parts = 0.0, {}
    for o, name in enumerate(("top_k_top_p", "min_p", "plain")):
        sel = np.nonzero(op == o)[0]
        I, S = g(idx[sel]), g(seeds[sel].view(np.int64))
        K, Pp, M = g(w["top_k"][idx[sel]]), g(w["top_p"][idx[sel]]), g(w["min_p"][idx[sel]])
        fn = {0: lambda: dss.top_k_top_p_sampling_from_probs(P, K, Pp, indices=I, seed=S, offset=0),
              1: lambda: dss.min_p_sampling_from_probs(P, M, indices=I, seed=S, offset=0),
              2: lambda: dss.sampling_from_probs(P, indices=I, seed=S, offset=0)}[o]
        t = kernel_times(lib, fn, 5, 1)
        parts[name] = {"outputs": int(len(sel)), "kernel_us": float(t.mean())}
        step += float(t.mean())
    out["hetero B=256 V=128256, 512 outputs, three calls per step"] = {
        "kernel_us": step, "algorithmic_bytes": 512 * V * 4,
        "hbm_frac": 512 * V * 4 / (step * 1e-6) / (HBM_PEAK_GBS * 1e9), "calls": parts}
    # cold: every call of a step on the next of 16 rotating copies of the batch
    Pc = [P.clone() for _ in range(N_BUFFERS)]
    step, parts = 0.0, {}
    for o, name in enumerate(("top_k_top_p", "min_p", "plain")):
        sel = np.nonzero(op == o)[0]
        I, S = g(idx[sel]), g(seeds[sel].view(np.int64))
        K, Pp, M = g(w["top_k"][idx[sel]]), g(w["top_p"][idx[sel]]), g(w["min_p"][idx[sel]])
        cnt = [o * 5]

        def fn(o=o, I=I, S=S, K=K, Pp=Pp, M=M, cnt=cnt):
            X = Pc[cnt[0] % N_BUFFERS]
            cnt[0] += 1
            if o == 0:
                dss.top_k_top_p_sampling_from_probs(X, K, Pp, indices=I, seed=S, offset=0)
            elif o == 1:
                dss.min_p_sampling_from_probs(X, M, indices=I, seed=S, offset=0)
            else:
                dss.sampling_from_probs(X, indices=I, seed=S, offset=0)
        t = kernel_times(lib, fn, 16, 1)
        parts[name] = {"outputs": int(len(sel)), "kernel_us": float(t.mean())}
        step += float(t.mean())
    out["hetero B=256 V=128256, 512 outputs, three calls per step, cold (16 buffers)"] = {
        "kernel_us": step, "algorithmic_bytes": 512 * V * 4,
        "hbm_frac": 512 * V * 4 / (step * 1e-6) / (HBM_PEAK_GBS * 1e9), "calls": parts}
    del Pc
    w = si.stress()
    P = g(w["probs"])
    B, V = P.shape
    seeds = g(w["seeds"].view(np.int64))
    t = kernel_times(lib, lambda: dss.top_k_top_p_sampling_from_probs(P, 1000, 0.95, seed=seeds,
                                                                       offset=0), 3, 1)
    _, _, r = dss.top_k_top_p_sampling_from_probs(P, 1000, 0.95, seed=seeds, offset=7,
                                                  return_valid=True, return_rounds=True)
    r = r.cpu().numpy()
    hist = {}
    for gi, name in enumerate(("near-uniform", "peaked", "geometric")):
        x = r[w["groups"] == gi]
        hist[name] = {"mean": float(x.mean()), "p95": float(np.percentile(x, 95)),
                      "p99": float(np.percentile(x, 99)), "max": int(x.max())}
    out["stress B=512 V=256000 top_k_top_p (k=1000, p=0.95)"] = entry(t, B * V * 4,
                                                                      rounds=hist)
    Pc = [P.clone() for _ in range(N_BUFFERS)]
    cnt = [0]

    def cold_stress():
        X = Pc[cnt[0] % N_BUFFERS]
        cnt[0] += 1
        dss.top_k_top_p_sampling_from_probs(X, 1000, 0.95, seed=seeds, offset=0)
    out["stress B=512 V=256000 top_k_top_p (k=1000, p=0.95), cold (16 buffers)"] = entry(
        kernel_times(lib, cold_stress, 16, 1), B * V * 4)
    del Pc
    # the pages' tail argument: rounds of the loop run from low = 0 with the
    # second pivot (dual) and without it (single), same rows, same streams
    cmp = {}
    for name, fl in (("dual_pivot", dss.DSS_FLAG_FROM_ZERO), ("single_pivot", dss.DSS_FLAG_SINGLE_PIVOT)):
        _, _, r = dss.top_k_top_p_sampling_from_probs(P, 1000, 0.95, seed=seeds, offset=7,
                                                      return_valid=True, return_rounds=True,
                                                      flags=fl)
        r = r.cpu().numpy()
        cmp[name] = {}
        for gi, gname in enumerate(("near-uniform", "peaked", "geometric")):
            x = r[w["groups"] == gi]
            cmp[name][gname] = {"mean": float(x.mean()), "p99": float(np.percentile(x, 99)),
                                "max": int(x.max())}
    out["stress rounds from low = 0: dual vs single pivot"] = cmp
    return out


PHASES = [(1, "slice loads issued, histogram cleared"), (2, "provisional bound from 30% sample"),
          (3, "slice landed (thread 0)"), (4, "certified slice bound"),
          (6, "candidates extracted to LDS"), (7, "list + header stored, drained"),
          (8, "arrival counted"), (9, "last arriver: headers read"),
          (10, "last arriver: lists placed"), (11, "tau_k histogram"), (12, "tau_k bin found"),
          (13, "top-k set partitioned"), (14, "tau_k in the boundary bin"),
          (15, "top-p start certified"), (16, "dual-pivot loop done")]


def phase_stamps(si, steps):
    """Per-phase timeline of the headline kernel: the measurement build
    libdss_stamps.so (DSS_PHASE_STAMPS: thread 0 of every work-group stores
    the 100 MHz constant clock at each phase boundary) on the cold rotating
    buffers; times from the kernel's first work-group start, averaged over
    `steps` launches.  The stamps themselves cost about 0.1 us each."""
    import ctypes
    import torch
    from decode_step_sampling_amd import _lib, build
    path = build.STAMPS_LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m decode_step_sampling_amd.build --stamps`")
    lib = ctypes.CDLL(path)
    for name, (a, r) in _lib.SIGNATURES.items():
        f = getattr(lib, name)
        f.argtypes, f.restype = a, r
    lib.dss_debug_set_stamps.argtypes = [ctypes.c_void_p]
    dev = torch.device("cuda:0")
    w = si.renorm()
    B, V = w["probs"].shape
    base = torch.from_numpy(w["probs"]).to(dev)
    bufs = [base.clone() for _ in range(N_BUFFERS)]
    k = torch.from_numpy(w["top_k"]).to(dev)
    p = torch.from_numpy(w["top_p"]).to(dev)
    seeds = torch.from_numpy(w["seeds"].view(np.int64)).to(dev)
    samples = torch.empty(B, dtype=torch.int32, device=dev)
    wsb = lib.dss_workspace_size(4, B, V, B, 0)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    st = torch.zeros(4096 * 32, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def call(i):
        r = lib.dss_top_k_top_p_sampling_from_probs(
            bufs[i % N_BUFFERS].data_ptr(), B, V, None, B, seeds.data_ptr(), 0, None, i,
            k.data_ptr(), 0, p.data_ptr(), 0.0, samples.data_ptr(), None, None, 0, ws.data_ptr(),
            wsb, stream)
        if r != 0:
            raise RuntimeError(_lib.strerror(r))
    for i in range(20):
        call(i)
    torch.cuda.synchronize()
    rel = []
    for rep in range(steps):
        st.zero_()
        lib.dss_debug_set_stamps(ctypes.c_void_p(st.data_ptr()))
        call(100 + rep)
        torch.cuda.synchronize()
        lib.dss_debug_set_stamps(None)
        a = st.cpu().numpy().reshape(-1, 32)[:256].astype(np.float64)
        t0 = a[:, 0][a[:, 0] > 0].min()
        rel.append(np.where(a > 0, (a - t0) * 0.01, np.nan))
    R = np.stack(rel)
    print("| phase (thread 0 of each work-group, after the step) | all work-groups, mean us "
          "| last arriver (64), mean us |")
    print("|---|---|---|")
    last = ~np.isnan(R[:, :, 9])
    for j, name in PHASES:
        x = R[:, :, j]
        lx = np.where(last, x, np.nan)
        print(f"| {j:2d} {name} | {np.nanmean(x):.2f} | "
              f"{np.nanmean(lx):.2f} |" if not np.all(np.isnan(lx)) else
              f"| {j:2d} {name} | {np.nanmean(x):.2f} | - |")
    ends = np.nanmax(R[:, :, 16], axis=1)
    print(f"\nlast loop end (kernel end less the sample store), mean over {steps} launches: "
          f"{ends.mean():.2f} us")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--engine", default="auto", choices=["auto", "streaming", "from_zero"])
    ap.add_argument("--warm-cache", action="store_true", help="time one buffer only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (other_configs)")
    ap.add_argument("--quick", action="store_true",
                    help="four timed calls per other workload (for counter runs under a profiler)")
    ap.add_argument("--phase-stamps", action="store_true",
                    help="print the headline kernel's phase timeline (libdss_stamps.so) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "rows shard across GPUs with no exchange, so per-GPU throughput is the figure.",
              file=sys.stderr)
        sys.exit(2)

    QUICK[0] = args.quick
    import synthetic_inputs as si
    if args.phase_stamps:
        phase_stamps(si, args.steps)
        return
    # the oracle's worker processes are forked before anything touches the GPU
    pool = None
    cpu_names = ("headline", "renorm", "latency", "hetero", "stress")
    if not args.no_cpu:
        _CPU.update(cpu_workloads(si, cpu_names))
        pool, ncores = cpu_pool()

    import torch
    import decode_step_sampling_amd as dss

    flags = {"auto": 0, "streaming": dss.DSS_FLAG_STREAMING,
             "from_zero": dss.DSS_FLAG_FROM_ZERO}[args.engine]
    dev = torch.device("cuda:0")
    w = si.renorm()
    B, V = w["probs"].shape
    base = torch.from_numpy(w["probs"]).to(dev)
    nbuf = 1 if args.warm_cache else N_BUFFERS
    bufs = [base.clone() for _ in range(nbuf)]
    k = torch.from_numpy(w["top_k"]).to(dev)
    p = torch.from_numpy(w["top_p"]).to(dev)
    seeds = torch.from_numpy(w["seeds"].view(np.int64)).to(dev)
    samples = torch.empty(B, dtype=torch.int32, device=dev)
    lib = dss._lib.load()
    ws_bytes = lib.dss_workspace_size(dss.OP_IDS["top_k_top_p_sampling_from_probs"], B, V, B,
                                      flags)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)   # zero-filled once
    fn = lib.dss_top_k_top_p_sampling_from_probs
    stream = torch.cuda.current_stream(dev).cuda_stream
    ptrs = [b.data_ptr() for b in bufs]

    def launch(i):
        # the C ABI directly: per-row seed array, scalar offset i (new stream per call)
        st = fn(ptrs[i % nbuf], B, V, None, B, seeds.data_ptr(), 0, None, i, k.data_ptr(), 0,
                p.data_ptr(), 0.0, samples.data_ptr(), None, None, flags, ws.data_ptr(),
                ws_bytes, stream)
        if st != 0:
            raise RuntimeError(dss._lib.strerror(st))

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()

    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(K):
        launch(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = e0.elapsed_time(e1)
    ms_per_step = total_ms / K

    # kernel durations: dispatch events attached to each call's kernel
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for ev in starts + ends:
        ev.record()                     # creates the HIP event behind the handle
    torch.cuda.synchronize()
    for i in range(K):
        st = lib.dss_set_timing_events(starts[i].cuda_event, ends[i].cuda_event)
        if st != 0:
            raise RuntimeError(dss._lib.strerror(st))
        launch(args.warmup + K + i)
    lib.dss_set_timing_events(None, None)
    torch.cuda.synchronize()
    per_launch_ms = float(np.mean([s.elapsed_time(e) for s, e in zip(starts, ends)]))

    bytes_per_launch = B * V * 4
    achieved = bytes_per_launch / (per_launch_ms * 1e-3) / 1e9

    # round histogram of the rejection loop on this workload (untimed)
    hist = {}
    for i in range(20):
        s, v, r = dss.top_k_top_p_sampling_from_probs(bufs[0], k, p, seed=seeds, offset=10_000 + i,
                                                      return_valid=True, return_rounds=True,
                                                      flags=flags)
        assert bool((v == 1).all())
        for x in r.cpu().numpy().tolist():
            hist[x] = hist.get(x, 0) + 1
    log(f"engine={args.engine} cache={'warm' if args.warm_cache else 'cold'} "
        f"kernel {per_launch_ms * 1e3:.2f} us, per-step {ms_per_step * 1e3:.2f} us, "
        f"wall {wall * 1e6 / K:.1f} us/step; rounds histogram {dict(sorted(hist.items()))}")

    traffic = measured_traffic() if args.engine == "auto" and not args.warm_cache else None
    out = {
        "metric": METRIC,
        "value": B / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "fused top_k_top_p_sampling_from_probs, B=64, V=151936, fp32 "
                        "softmax(N(0,2^2)), per-row top_k~U{1..1024}, top_p~U[0.5,0.95]",
            "batch": B, "vocab": V, "engine": args.engine, "workspace_bytes": ws_bytes,
            "cache": "warm (1 buffer)" if args.warm_cache else f"cold ({nbuf} rotating buffers)",
        },
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "traffic_source": (f"{TRAFFIC_FILE} (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                        f"kernel source hash {kernel_source_hash()})")
                     if traffic is not None else None,
                     "kernel_us": per_launch_ms * 1e3,
                     "algorithmic_bytes": bytes_per_launch},
        "rounds_histogram": {str(kk): vv for kk, vv in sorted(hist.items())},
    }
    if not args.no_extra and args.engine == "auto" and not args.warm_cache:
        out["reference"] = reference_points(lib, bufs, K)
        del bufs
        torch.cuda.empty_cache()
        out["other_configs"] = extra_configs(dss, si, lib, dev)
    if pool is not None:
        res = cpu_baseline(pool, ncores, cpu_names)
        pool.close()
        pool.join()
        h = res["headline"]
        out["cpu_baseline"] = {
            "value": h["all_cores"]["value"], "unit": "rows/s", "cores": ncores, "kind": "oracle",
            "sample": f"{h['sample']}; the sort-based Python/numpy oracle in {ncores} worker "
                      "processes (one per core of the box's CPU share, at most 16)",
            "one_core": h["one_core"]["value"], "GBps": h["all_cores"]["GBps"],
            "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "configs": {n: res[n] for n in res if n != "headline"}}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
