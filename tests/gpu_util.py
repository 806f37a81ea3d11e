"""Helpers shared by the GPU tests (device transfers, statistics)."""

import numpy as np
import torch
from scipy import stats

DEV = "cuda:0"


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def u64(values):
    """uint64 numbers as an int64 GPU tensor with the same bit pattern."""
    return gpu(np.asarray(values, dtype=np.uint64).view(np.int64))


def host(t):
    return t.detach().cpu().numpy()


def pooled_chi_square(counts, target):
    """Chi-square p-value of observed counts against a target law.

    Cells whose expected count is below 5 are pooled into one cell (merged
    with the smallest remaining cell if the pool itself stays below 5).
    Returns (p_value, total variation distance, number of cells).
    """
    counts = np.asarray(counts, dtype=np.float64)
    target = np.asarray(target, dtype=np.float64)
    n = counts.sum()
    expected = target * n
    big = expected >= 5
    obs = list(counts[big])
    exp = list(expected[big])
    rest_o, rest_e = counts[~big].sum(), expected[~big].sum()
    if rest_e > 0:
        if rest_e >= 5 or not obs:
            obs.append(rest_o)
            exp.append(rest_e)
        else:
            j = int(np.argmin(exp))
            obs[j] += rest_o
            exp[j] += rest_e
    tvd = 0.5 * np.abs(counts / n - target).sum()
    if len(obs) < 2:
        return 1.0, tvd, len(obs)
    exp = np.asarray(exp) * (np.sum(obs) / np.sum(exp))
    return float(stats.chisquare(obs, exp).pvalue), float(tvd), len(obs)
