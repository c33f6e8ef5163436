"""Process pool for the float64 oracle work of the GPU parity tests.

Planting margins and running the oracle take about half a second per
selection pass on a 64K-token head, and the full-size tests visit 32 heads
or more, so they run in worker processes.  Workers are started with the
"spawn" method (a fresh interpreter, never a fork of a process that holds a
GPU context) and import only numpy and the oracle.  Head data crosses the
process boundary as its raw stored bits (bfloat16 as uint16), and each
worker widens them to the exact float64 values the oracle reads.
"""

import multiprocessing as mp
import os

import numpy as np

MAX_WORKERS = 16  # the host CPU share of one GPU


def decode(arr, dtype):
    """Exact float64 values of stored bfloat16 bits (uint16) or float32 data."""
    if dtype == "bf16":
        return (np.asarray(arr, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def plant_job(job):
    """Margin planting for one head: returns (key, ops, converged)."""
    from oracle.planting import plant_margins

    key, dtype, q, kp, budgets, levels, agg, wavelet, max_iter = job
    _, ops, ok = plant_margins(decode(q, dtype), decode(kp, dtype), budgets, levels, agg=agg, wavelet=wavelet,
                               max_iter=max_iter)
    return key, ops, ok


def oracle_job(job):
    """The oracle's selection and output for one head, without the stored
    bands (returned: key, O, sel, cand, scores, gap)."""
    from oracle import select_attend

    key, dtype, q, k, v, n_prompt, gen, budgets, levels, agg, wavelet = job
    out, res = select_attend(decode(q, dtype), decode(k, dtype), decode(v, dtype), n_prompt, gen, budgets, levels,
                             agg, wavelet)
    return key, out, res.sel, res.cand, res.scores, res.gap


def validity_job(job):
    """Level sets of a device selection checked as a valid Top-K under the
    oracle's float64 scores (see ``_parity.check_validity``)."""
    from oracle import attend, dwt_pyramid, level_scores

    key, dtype, q, k, v, n_prompt, gen, budgets, levels, agg, wavelet, dev_levels, band = job
    qf, kf, vf = decode(q, dtype), decode(k, dtype), decode(v, dtype)
    approx, _ = dwt_pyramid(kf[:n_prompt], levels, wavelet)
    worst = np.inf  # smallest relative margin of a kept over a dropped candidate
    for j in range(levels, -1, -1):
        kj = budgets[levels - j]
        sel = np.asarray(dev_levels[j], dtype=np.int64)
        if j == levels:
            cand = np.arange(approx[levels].shape[0])
        else:
            par = np.asarray(dev_levels[j + 1], dtype=np.int64)
            cand = np.sort(np.concatenate([2 * par, 2 * par + 1]))
        if len(sel) != kj or len(np.unique(sel)) != kj or not np.all(np.isin(sel, cand)):
            return key, f"level {j}: not {kj} distinct candidates", None
        if kj < len(cand):
            s = level_scores(qf, approx[j][cand], agg)
            kept = np.isin(cand, sel)
            lo, hi = s[kept].min(), s[~kept].max()
            scale = max(abs(lo), abs(hi), 1e-300)
            margin = (lo - hi) / scale
            worst = min(worst, margin)
            if margin < -band:
                return key, f"level {j}: a dropped candidate beats a kept one by {-margin:.3g} (relative)", None
    rows = np.concatenate([np.asarray(dev_levels[0], dtype=np.int64), np.asarray(gen, dtype=np.int64)])
    out = attend(qf, kf[rows], vf[rows])
    return key, None, (out, worst)


def workers(n_jobs):
    return max(1, min(MAX_WORKERS, len(os.sched_getaffinity(0)), n_jobs))


def run(fn, jobs):
    """fn over jobs, in a spawn pool when there is more than one."""
    if len(jobs) <= 1:
        return [fn(j) for j in jobs]
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers(len(jobs))) as pool:
        return pool.map(fn, jobs, chunksize=1)
