"""The allocation-free entry point (dss_top_k_top_p_sampling_from_probs_noalloc,
scratch in the library's static device array) against the workspace entry
point, called through the C ABI: the same kernels and Philox streams, so
tokens, valid flags and round counts must be equal, on consecutive calls
with different shapes (the static scratch keeps the previous call's
contents) and on both engines (split for per-row k, resident for a scalar k
above the split cap)."""

import numpy as np
import pytest
import torch

import decode_step_sampling_amd as dss
import synthetic_inputs as si
from gpu_util import gpu, host, u64

pytestmark = pytest.mark.gpu


def _noalloc(P, k, p, seeds, offset):
    lib = dss._lib.load()
    B, V = P.shape
    samples = torch.full((B,), -7, dtype=torch.int32, device=P.device)
    valid = torch.full((B,), 7, dtype=torch.uint8, device=P.device)
    rounds = torch.full((B,), -7, dtype=torch.int32, device=P.device)
    karr = k if isinstance(k, torch.Tensor) else None
    parr = p if isinstance(p, torch.Tensor) else None
    st = lib.dss_top_k_top_p_sampling_from_probs_noalloc(
        P.data_ptr(), B, V, None, B, seeds.data_ptr(), 0, None, offset,
        None if karr is None else karr.data_ptr(), 0 if karr is not None else int(k),
        None if parr is None else parr.data_ptr(), 0.0 if parr is not None else float(p),
        samples.data_ptr(), valid.data_ptr(), rounds.data_ptr(), 0,
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, dss._lib.strerror(st)
    return host(samples), host(valid), host(rounds)


def _with_workspace(P, k, p, seeds, offset):
    s, v, r = dss.top_k_top_p_sampling_from_probs(P, k, p, seed=seeds, offset=offset,
                                                  return_valid=True, return_rounds=True)
    return host(s), host(v), host(r)


def test_noalloc_matches_workspace_entry_point():
    big = si.renorm()
    small = si.renorm(rep=1, rows=8, vocab=32000)
    cases = [
        (gpu(big["probs"]), gpu(big["top_k"]), gpu(big["top_p"]), u64(big["seeds"])),
        (gpu(small["probs"]), 50, 0.9, u64(small["seeds"])),
        (gpu(big["probs"]), 3000, 0.9, u64(big["seeds"])),      # resident engine
        (gpu(small["probs"]), gpu(small["top_k"]), gpu(small["top_p"]), u64(small["seeds"])),
    ]
    for n, (P, k, p, seeds) in enumerate(cases):
        for offset in (0, 1):
            a = _noalloc(P, k, p, seeds, 10 * n + offset)
            b = _with_workspace(P, k, p, seeds, 10 * n + offset)
            assert np.array_equal(a[1], b[1]) and a[1].all(), (n, offset)
            assert np.array_equal(a[0], b[0]), (n, offset)
            assert np.array_equal(a[2], b[2]), (n, offset)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    lib = dss._lib.load()
    P = torch.zeros(4, dtype=torch.float32, device="cuda:0")
    out = torch.zeros(4096, dtype=torch.int32, device="cuda:0")
    # 4096 rows of 151936 need more than the 64 MiB static scratch
    st = lib.dss_top_k_top_p_sampling_from_probs_noalloc(
        P.data_ptr(), 4096, 151936, None, 4096, None, 1, None, 0, None, 50, None, 0.9,
        out.data_ptr(), None, None, 0, torch.cuda.current_stream().cuda_stream)
    assert st == dss._lib.DSS_ERR_WORKSPACE
