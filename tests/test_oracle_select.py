"""Pins of the oracle's coarse-to-fine selection (WaveFilter Figure 2 (c)-(d)).

Independent checks: scores by explicit loops over tokens (not through the
pyramid), brute-force flat top-B when the coarse levels keep everything,
the union-of-coarse-blocks special case, exhaustive subset search on tiny
inputs, exact ties, and invariances.
"""

import itertools
import math

import numpy as np
import pytest

from oracle import level_scores, top_k, select, haar_pyramid
from workloads.configs import check_budgets


def block_score_loop(q, k_prompt, j, c):
    """max_i q_i . (2^{-j/2} sum_{t in block c} k_t) / sqrt(d), by explicit loops."""
    n_q, d = q.shape
    w = 1 << j
    best = -math.inf
    for i in range(n_q):
        acc = 0.0
        for t in range(c * w, (c + 1) * w):
            acc += float(np.dot(q[i], k_prompt[t]))
        best = max(best, acc * 2 ** (-j / 2) / math.sqrt(d))
    return best


def rank_key(score, idx):
    return (-score, idx)


def test_level_scores_loop():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((7, 6))
    kp = rng.standard_normal((32, 6))
    approx, _ = haar_pyramid(kp, 3)
    for j in range(4):
        s = level_scores(q, approx[j])
        for c in range(32 >> j):
            assert abs(s[c] - block_score_loop(q, kp, j, c)) < 1e-12


def test_top_k_ties_and_gap():
    cand = np.array([10, 3, 7, 5, 1])
    sc = np.array([2.0, 5.0, 2.0, 2.0, -1.0])
    chosen, gap = top_k(cand, sc, 2)
    # best is 3 (5.0); then among the three 2.0 ties the lowest index, 5
    assert list(chosen) == [3, 5]
    assert gap == 0.0
    chosen, gap = top_k(cand, sc, 4)
    assert list(chosen) == [3, 5, 7, 10]
    assert abs(gap - (2.0 - (-1.0)) / 2.0) < 1e-15
    chosen, gap = top_k(cand, sc, 5)
    assert gap == math.inf and list(chosen) == [1, 3, 5, 7, 10]
    with pytest.raises(ValueError):
        top_k(cand, sc, 6)


@pytest.mark.parametrize("levels,n_p,B", [(1, 32, 5), (3, 64, 9), (4, 256, 37)])
def test_flat_top_b_when_coarse_levels_keep_all(levels, n_p, B):
    rng = np.random.default_rng(levels)
    d = 8
    q = rng.standard_normal((5, d))
    kp = rng.standard_normal((n_p, d))
    budgets = [n_p >> j for j in range(levels, 0, -1)] + [B]
    res = select(q, kp, budgets, levels)
    tok = [max(float(np.dot(q[i], kp[t])) for i in range(5)) / math.sqrt(d) for t in range(n_p)]
    brute = sorted(range(n_p), key=lambda t: rank_key(tok[t], t))[:B]
    assert list(res.sel[0]) == sorted(brute)


def test_union_of_coarse_blocks_on_full_expansion():
    rng = np.random.default_rng(7)
    levels, n_p, d = 3, 256, 8
    q = rng.standard_normal((4, d))
    kp = rng.standard_normal((n_p, d))
    k_top = 5
    budgets = [k_top << i for i in range(levels + 1)]
    res = select(q, kp, budgets, levels)
    blocks = sorted(range(n_p >> levels),
                    key=lambda c: rank_key(block_score_loop(q, kp, levels, c), c))[:k_top]
    want = sorted(t for c in blocks for t in range(c << levels, (c + 1) << levels))
    assert list(res.sel[0]) == want


def brute_select(q, kp, budgets, levels):
    """Level by level, the kept set is the k-subset of the candidates with the
    largest score sum (exhaustive search over all subsets); candidates are
    the children of the kept parents; scores by explicit loops."""
    n_top = kp.shape[0] >> levels
    cand = list(range(n_top))
    out = {}
    for j in range(levels, -1, -1):
        if j < levels:
            cand = sorted([2 * p for p in out[j + 1]] + [2 * p + 1 for p in out[j + 1]])
        sc = {c: block_score_loop(q, kp, j, c) for c in cand}
        k = budgets[levels - j]
        best = max(itertools.combinations(cand, k), key=lambda sub: sum(sc[c] for c in sub))
        out[j] = sorted(best)
    return out


def test_exhaustive_tiny():
    rng = np.random.default_rng(11)
    checked = 0
    for levels, n_p in [(1, 8), (2, 16), (3, 16), (2, 32)]:
        schedules = []
        n_top = n_p >> levels

        def grow(prefix):
            if len(prefix) == levels + 1:
                schedules.append(list(prefix))
                return
            j = levels - len(prefix)
            for k in range(1, min(2 * prefix[-1], n_p >> j) + 1):
                grow(prefix + [k])

        for k_top in range(1, n_top + 1):
            grow([k_top])
        # keep the exhaustive search small: at most a few thousand subsets per level
        schedules = [s for s in schedules
                     if math.comb(n_top, s[0]) <= 3000
                     and all(math.comb(2 * s[i - 1], s[i]) <= 3000 for i in range(1, len(s)))]
        picks = rng.choice(len(schedules), size=min(12, len(schedules)), replace=False)
        for p in picks:
            budgets = schedules[p]
            assert check_budgets(n_p, levels, budgets)
            q = rng.standard_normal((3, 4))
            kp = rng.standard_normal((n_p, 4))
            res = select(q, kp, budgets, levels)
            want = brute_select(q, kp, budgets, levels)
            for j in range(levels + 1):
                assert list(res.sel[j]) == want[j], (levels, n_p, budgets, j)
            checked += 1
    assert checked >= 30


def test_full_budgets_select_everything():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 8))
    kp = rng.standard_normal((128, 8))
    budgets = [128 >> j for j in range(4, -1, -1)]
    res = select(q, kp, budgets, 4)
    assert list(res.sel[0]) == list(range(128))
    assert all(res.gap[j] == math.inf for j in range(5))


def test_exact_tie_goes_to_lower_index():
    rng = np.random.default_rng(9)
    d, levels = 8, 2
    kp = rng.standard_normal((32, d)) * 0.01
    q = rng.standard_normal((3, d))
    big = rng.standard_normal((4, d))
    kp[20:24] = big + 5 * q.mean(axis=0)   # block 5 at level 2
    kp[8:12] = kp[20:24]                   # block 2: identical keys, exactly equal score
    res = select(q, kp, [1, 2, 4], levels)
    assert list(res.sel[2]) == [2]
    assert res.gap[2] == 0.0


def test_invariances():
    rng = np.random.default_rng(4)
    levels, n_p, d = 4, 512, 16
    q = rng.standard_normal((6, d))
    kp = rng.standard_normal((n_p, d))
    budgets = [6, 10, 17, 30, 50]
    base = select(q, kp, budgets, levels)
    scaled = select(3.5 * q, kp, budgets, levels)
    perm = select(q[rng.permutation(6)], kp, budgets, levels)
    for j in range(levels + 1):
        assert list(base.sel[j]) == list(scaled.sel[j]) == list(perm.sel[j])
    # scaling one level-2 region's keys by c > 0 scales its level-2 score by c
    c_reg, factor = 9, 0.37
    kp2 = kp.copy()
    kp2[c_reg * 4:(c_reg + 1) * 4] *= factor
    a1, _ = haar_pyramid(kp, 2)
    a2, _ = haar_pyramid(kp2, 2)
    s1 = level_scores(q, a1[2][c_reg:c_reg + 1])[0]
    s2 = level_scores(q, a2[2][c_reg:c_reg + 1])[0]
    assert abs(s2 - factor * s1) < 1e-12


# -- the "mean" aggregation variant (the query rows' scores averaged) --------

def test_mean_scores_are_the_mean_query_loop():
    """Mean aggregation, written out as a double loop over rows and columns."""
    rng = np.random.default_rng(21)
    q = rng.standard_normal((5, 8))
    a = rng.standard_normal((7, 8))
    got = level_scores(q, a, "mean")
    for c in range(7):
        acc = 0.0
        for i in range(5):
            acc += sum(q[i, t] * a[c, t] for t in range(8))
        assert abs(got[c] - acc / 5 / math.sqrt(8)) < 1e-12


def test_mean_selection_is_the_averaged_query_selection():
    """By linearity the mean of the rows' scores is the score of the mean
    query row, and with one row every aggregation agrees: the mean selection
    of a block equals the selection of its single averaged row, at every level."""
    rng = np.random.default_rng(22)
    for levels, n_p, budgets in [(3, 256, [5, 9, 16, 30]), (4, 512, [6, 10, 17, 30, 50]), (0, 64, [20])]:
        q = rng.standard_normal((6, 16))
        kp = rng.standard_normal((n_p, 16))
        mean = select(q, kp, budgets, levels, "mean")
        single = select(q.mean(axis=0, keepdims=True), kp, budgets, levels, "max")
        for j in range(levels + 1):
            assert list(mean.sel[j]) == list(single.sel[j])


def test_max_and_mean_pick_different_tokens():
    """Hand-worked: rows (1, 0) and (0, 1); token 0 = (3, -3) scores 3/sqrt2
    for one row and -3/sqrt2 for the other, token 1 = (1, 1) scores 1/sqrt2
    for both.  The maximum keeps token 0 (3/sqrt2 > 1/sqrt2), the mean keeps
    token 1 (0 < 1/sqrt2)."""
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    kp = np.array([[3.0, -3.0], [1.0, 1.0]])
    s_max = level_scores(q, kp, "max")
    s_mean = level_scores(q, kp, "mean")
    assert np.allclose(s_max, [3 / math.sqrt(2), 1 / math.sqrt(2)])
    assert np.allclose(s_mean, [0.0, 1 / math.sqrt(2)])
    assert list(select(q, kp, [1], 0, "max").sel[0]) == [0]
    assert list(select(q, kp, [1], 0, "mean").sel[0]) == [1]


def test_duplicated_row_moves_the_mean_not_the_max():
    rng = np.random.default_rng(23)
    q = rng.standard_normal((4, 8))
    a = rng.standard_normal((9, 8))
    q_dup = np.concatenate([q, q[1:2]])
    assert np.array_equal(level_scores(q_dup, a, "max"), level_scores(q, a, "max"))
    per_row = q @ a.T / math.sqrt(8)
    want = (per_row.sum(axis=0) + per_row[1]) / 5
    assert np.allclose(level_scores(q_dup, a, "mean"), want, atol=1e-12)
    with pytest.raises(ValueError):
        level_scores(q, a, "median")


# -- the softmax-probability aggregations ------------------------------------
# p_i[c] = exp(l_ic) / sum over the level's candidates c' of exp(l_ic'),
# l_ic = q_i . a_c / sqrt(d); the score is max_i p_i[c] or mean_i p_i[c].

def test_softmax_scores_are_the_direct_loop():
    """Both softmax aggregations written out with scalar exp and sums, the
    normaliser taken over the candidates (columns), not over the rows."""
    rng = np.random.default_rng(31)
    n_q, m, d = 4, 6, 8
    q = rng.standard_normal((n_q, d))
    a = rng.standard_normal((m, d))
    p = [[0.0] * m for _ in range(n_q)]
    for i in range(n_q):
        logit = [sum(q[i, t] * a[c, t] for t in range(d)) / math.sqrt(d) for c in range(m)]
        z = sum(math.exp(x) for x in logit)
        for c in range(m):
            p[i][c] = math.exp(logit[c]) / z
    got_max = level_scores(q, a, "softmax_max")
    got_mean = level_scores(q, a, "softmax_mean")
    for c in range(m):
        assert abs(got_max[c] - max(p[i][c] for i in range(n_q))) < 1e-14
        assert abs(got_mean[c] - sum(p[i][c] for i in range(n_q)) / n_q) < 1e-14
    # every row's probabilities sum to one, so the mean scores do too
    assert abs(got_mean.sum() - 1.0) < 1e-12


def test_one_row_softmax_max_selects_what_the_logit_max_selects():
    """With one query row the softmax is a monotone map of the row's logits
    over the candidates, so both aggregations keep the same regions at every
    level (the candidates of a level depend only on the previous choice)."""
    rng = np.random.default_rng(32)
    for levels, n_p, budgets in [(3, 256, [5, 9, 16, 30]), (4, 512, [6, 10, 17, 30, 50]), (0, 64, [20])]:
        q = rng.standard_normal((1, 16))
        kp = rng.standard_normal((n_p, 16))
        for agg in ("softmax_max", "softmax_mean"):
            soft = select(q, kp, budgets, levels, agg)
            hard = select(q, kp, budgets, levels, "max")
            for j in range(levels + 1):
                assert list(soft.sel[j]) == list(hard.sel[j])


def test_softmax_mean_and_logit_mean_pick_different_regions():
    """Hand-worked, d = 2, rows q_1 = (1, 0) and q_2 = (0, 1); coefficient
    c = sqrt2 (x_c, y_c), so the logits are exactly x_c (row 1) and y_c
    (row 2).  x = (ln 8, 0, 0), y = (0, ln 20, ln 29):
      row 1 probabilities 8/10, 1/10, 1/10; row 2 1/50, 20/50, 29/50;
      softmax mean (0.41, 0.25, 0.34) and softmax max (0.8, 0.4, 0.58) keep c0;
      logit mean (ln 8/2, ln 20/2, ln 29/2) and logit max keep c2."""
    r2 = math.sqrt(2.0)
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    a = r2 * np.array([[math.log(8), 0.0], [0.0, math.log(20)], [0.0, math.log(29)]])
    assert np.allclose(level_scores(q, a, "softmax_mean"), [0.41, 0.25, 0.34], atol=1e-14)
    assert np.allclose(level_scores(q, a, "softmax_max"), [0.8, 0.4, 0.58], atol=1e-14)
    assert np.allclose(level_scores(q, a, "mean"), [math.log(8) / 2, math.log(20) / 2, math.log(29) / 2])
    assert list(select(q, a, [1], 0, "softmax_mean").sel[0]) == [0]
    assert list(select(q, a, [1], 0, "softmax_max").sel[0]) == [0]
    assert list(select(q, a, [1], 0, "mean").sel[0]) == [2]
    assert list(select(q, a, [1], 0, "max").sel[0]) == [2]


def test_a_constant_added_to_one_rows_logits_changes_nothing():
    """Shift invariance of each row's softmax: an extra coordinate that is 1
    in every coefficient and t in one query row adds t/sqrt(d) to that row's
    logits of every candidate.  The softmax scores do not move (the logit
    scores do, which shows the change reaches the logits)."""
    rng = np.random.default_rng(33)
    n_q, m, d = 5, 7, 9
    q = rng.standard_normal((n_q, d))
    q[:, -1] = 0.0
    a = rng.standard_normal((m, d))
    a[:, -1] = 1.0
    q_shift = q.copy()
    q_shift[2, -1] = 4.0
    for agg in ("softmax_max", "softmax_mean"):
        assert np.allclose(level_scores(q_shift, a, agg), level_scores(q, a, agg), rtol=0, atol=1e-14)
    assert not np.allclose(level_scores(q_shift, a, "mean"), level_scores(q, a, "mean"))
