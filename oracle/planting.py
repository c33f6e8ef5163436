"""Margin planting for exact-index parity tests.

TEST INFRASTRUCTURE ONLY.  Near-ties at a Top-K boundary make more than one
selection correct, and a float32 device computation may resolve such a tie
differently from the float64 oracle.  To make the selected index sets
comparable bit for bit, the test harness pushes every near-boundary region
that the oracle did *not* keep away from the boundary, by scaling that
region's prompt keys by exactly 0.5 (or 2.0 when its score is negative).

The region score is positively homogeneous in the region's keys (the
approximation coefficient is linear in them and the maximum over query rows
commutes with a positive scale), so the scale moves that score by a factor
of two.  Scaling by a power of two is exact in float32 and bfloat16, so the
rounded inputs stay exactly what the oracle sees.

This is harness code: it changes the synthetic inputs, never the method.
"""

import numpy as np

from .wavefilter import select


def plant_margins(q, k_prompt, budgets, levels, min_gap=2e-3, band=3e-3, max_iter=64, agg="max", wavelet="haar"):
    """Scale near-boundary losing regions until every level's gap exceeds ``min_gap``.

    Works from the coarsest level whose gap is too small: every candidate
    that was not kept there and whose score lies within ``band`` (relative)
    below the k-th best score has its ``2**j`` prompt keys scaled.  Repeats,
    since a change at one level can move the selection at others.

    Returns ``(k_new, ops, converged)`` where ``ops`` lists the applied
    ``(row_begin, row_end, factor)`` edits in order, so that the same edits
    can be replayed on another copy of the keys.
    """
    k = np.array(k_prompt, dtype=np.float64, copy=True)
    ops = []
    for _ in range(max_iter):
        res = select(q, k, budgets, levels, agg, wavelet)
        low = [j for j in range(levels, -1, -1) if res.gap[j] <= min_gap]
        if not low:
            return k, ops, True
        j = low[0]
        cand = res.cand[j]
        s = res.scores[j]
        kept = set(int(c) for c in res.sel[j])
        k_j = budgets[levels - j]
        s_kth = np.sort(s)[::-1][k_j - 1]
        threshold = s_kth - band * abs(s_kth)
        changed = False
        for c, sc in zip(cand, s):
            if int(c) in kept or not sc > threshold:
                continue
            factor = 0.5 if sc > 0 else 2.0
            r0, r1 = int(c) << j, (int(c) + 1) << j
            k[r0:r1] *= factor
            ops.append((r0, r1, factor))
            changed = True
        if not changed:
            break
    res = select(q, k, budgets, levels, agg, wavelet)
    ok = all(res.gap[j] > min_gap for j in range(levels + 1))
    return k, ops, ok
