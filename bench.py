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


def cpu_baseline(w, budget_s=10.0):
    """The oracle as it stands (sort-based filter + exact CDF draw), one core.

    Cycles over the 64 headline rows (a new stream per pass) for about
    ``budget_s`` seconds of CPU work and reports draws per second.
    """
    from oracle import philox as ph
    from oracle import reference as ref
    probs, ks, ps, seeds = w["probs"], w["top_k"], w["top_p"], w["seeds"]
    rows = probs.shape[0]
    t0 = time.perf_counter()
    done = 0
    while done < rows or time.perf_counter() - t0 < budget_s:
        r = done % rows
        ref.sample_by_cdf(probs[r], "top_k_top_p",
                          ph.draw_bits53(int(seeds[r]), done // rows, 0, 0), k=ks[r], p=ps[r])
        done += 1
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} sampled rows cycling over the 64 headline rows (sort + exact "
                      f"prefix + CDF draw per row), {dt:.1f} s single-threaded Python/numpy"}


def kernel_times(lib, fn, reps, warm=2):
    """Per-call kernel time in us of fn() (dispatch-event hook), reps calls."""
    import torch
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
    out["logits B=64 V=151936 top_k_top_p_sampling_from_logits (T=0.8; softmax + sampling kernels)"] = entry(
        kernel_times(lib, lambda: dss.top_k_top_p_sampling_from_logits(Lg, k, p, 0.8, seed=1, offset=0), 50),
        B * V * 4)
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
        p99_us=float(np.percentile(t, 99)))
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
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "rows shard across GPUs with no exchange, so per-GPU throughput is the figure.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_step_sampling_amd as dss
    import synthetic_inputs as si

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
                     "traffic": measured_traffic() if args.engine == "auto" and not args.warm_cache
                     else None,
                     "kernel_us": per_launch_ms * 1e3,
                     "algorithmic_bytes": bytes_per_launch},
        "rounds_histogram": {str(kk): vv for kk, vv in sorted(hist.items())},
    }
    if not args.no_extra and args.engine == "auto" and not args.warm_cache:
        out["reference"] = reference_points(lib, bufs, K)
        del bufs
        torch.cuda.empty_cache()
        out["other_configs"] = extra_configs(dss, si, lib, dev)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
