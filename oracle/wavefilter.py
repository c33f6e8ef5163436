"""Float64 oracle of the WaveFilter selection + sparse attention path.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Parity pins: every
function below is pinned by a CPU test against something other than itself
(closed forms, the textbook Haar matrix, invariants, a library attention
routine, exhaustive brute force on tiny inputs); none is "parity unpinned".

Sources (WaveFilter: Enhancing the Long-Context Capability of Diffusion LLMs
via Wavelet-Guided KV Cache Filtering, arXiv 2606.00724):

* section 2.2, equation 5 and the paragraph after it -- one analysis level of
  a two-channel filter bank with downsampling by two, iterated on the
  approximation band to give the pyramid {A_L, D_L, ..., D_1};
* section 3.1 -- the DWT is taken along the token axis of the cached *prompt*
  keys only, giving the low-frequency keys;
* Figure 2 (c) -- queries are scored against the low-frequency keys and a
  Top-K picks candidate regions;
* Figure 2 (d) and section 1 -- the candidate regions are refined recursively
  across scales down to single tokens, which form the sparse KV;
* section 2.1, equation 3 -- attention of the current queries over the cached
  keys/values with a 1/sqrt(d) scaled softmax, here restricted to the
  selected prompt tokens plus the generated positions.

Readings where the pages are silent (each is also listed in the design
notes): orthonormal Haar filters; the pair (x[2n], x[2n+1]) forms coefficient
n, so level-j coefficient n covers tokens [n 2^j, (n+1) 2^j) and has exactly
the children 2n, 2n+1; the score of a region is the maximum over the query
rows of the scaled dot product with its approximation coefficient (or, as
the variant "mean", its average over the rows; or the maximum or average of
the rows' softmax probabilities over the level's candidates); only the
two children of a selected region become candidates at the next finer level;
ties go to the lower index; the generated positions are always attended and
never scored; no mask.
"""

from dataclasses import dataclass, field
import math

import numpy as np

# Orthonormal Haar analysis filters (low-pass g, high-pass h).  The pages name
# only a generic wavelet basis (section 3.1) and generic g, h (equation 5).
HAAR_G = np.array([1.0, 1.0]) / math.sqrt(2.0)
HAAR_H = np.array([1.0, -1.0]) / math.sqrt(2.0)

# Daubechies' orthonormal four-tap filters (two vanishing moments), from their
# closed form (1 + s, 3 + s, 3 - s, 1 - s) / (4 sqrt2) with s = sqrt3; the
# high-pass filter is the quadrature mirror h[m] = (-1)^m g[3 - m].  A longer
# basis psi than Haar, for the variant of section 3.1's generic wavelet.
_S3 = math.sqrt(3.0)
DB2_G = np.array([1.0 + _S3, 3.0 + _S3, 3.0 - _S3, 1.0 - _S3]) / (4.0 * math.sqrt(2.0))
DB2_H = np.array([DB2_G[3], -DB2_G[2], DB2_G[1], -DB2_G[0]])
WAVELETS = ("haar", "db2")


def analysis_step(x, g=HAAR_G, h=HAAR_H):
    """One level of the two-channel analysis filter bank (section 2.2, eq. 5).

    ``x`` is ``[N, ...]`` with the signal along axis 0.  The filters are
    applied in polyphase (correlation) alignment,
    ``A[n] = sum_m g[m] x[2n + m]`` and ``D[n] = sum_m h[m] x[2n + m]``, i.e.
    output n is built from the input pair starting at 2n and the output is
    the input downsampled by two.  Requires N to be a multiple of the filter
    length (no boundary extension).
    """
    x = np.asarray(x, dtype=np.float64)
    n_in = x.shape[0]
    taps = len(g)
    if n_in % 2 != 0 or n_in % taps != 0:
        raise ValueError("signal length must be even and a multiple of the filter length")
    n_out = n_in // 2
    a = np.zeros((n_out,) + x.shape[1:], dtype=np.float64)
    dd = np.zeros_like(a)
    for m in range(taps):
        phase = x[m::2][:n_out]
        a += g[m] * phase
        dd += h[m] * phase
    return a, dd


def analysis_step_periodic(x, g, h):
    """One analysis level (eq. 5) with the signal extended periodically.

    ``A[n] = sum_m g[m] x[(2n + m) mod N]`` and likewise D with h: the same
    alignment as ``analysis_step`` (output n starts at input 2n), with the
    filter wrapping around the end of the signal.  For two-tap filters it
    equals ``analysis_step``.
    """
    x = np.asarray(x, dtype=np.float64)
    n_in = x.shape[0]
    if n_in % 2 != 0:
        raise ValueError("signal length must be even")
    n_out = n_in // 2
    a = np.zeros((n_out,) + x.shape[1:], dtype=np.float64)
    dd = np.zeros_like(a)
    for n in range(n_out):
        for m in range(len(g)):
            a[n] += g[m] * x[(2 * n + m) % n_in]
            dd[n] += h[m] * x[(2 * n + m) % n_in]
    return a, dd


def dwt_pyramid(x, levels, wavelet="haar"):
    """L-level pyramid with the named basis: "haar" (``haar_pyramid``) or
    "db2" (Daubechies' four-tap filters, periodic extension at every level).
    Same return convention as ``haar_pyramid``."""
    if wavelet == "haar":
        return haar_pyramid(x, levels)
    if wavelet != "db2":
        raise ValueError("unknown wavelet")
    x = np.asarray(x, dtype=np.float64)
    if levels < 0 or x.shape[0] % (1 << levels) != 0:
        raise ValueError("token count must be a multiple of 2**levels")
    approx = [x]
    detail = [None]
    for _ in range(levels):
        a, dd = analysis_step_periodic(approx[-1], DB2_G, DB2_H)
        approx.append(a)
        detail.append(dd)
    return approx, detail


def synthesis_step(a, dd):
    """Inverse of one orthonormal Haar analysis level.

    Undoes ``A = (x0 + x1)/sqrt2, D = (x0 - x1)/sqrt2`` pairwise:
    ``x[2n] = (A[n] + D[n])/sqrt2`` and ``x[2n+1] = (A[n] - D[n])/sqrt2``.
    """
    a = np.asarray(a, dtype=np.float64)
    dd = np.asarray(dd, dtype=np.float64)
    x = np.empty((2 * a.shape[0],) + a.shape[1:], dtype=np.float64)
    x[0::2] = (a + dd) / math.sqrt(2.0)
    x[1::2] = (a - dd) / math.sqrt(2.0)
    return x


def haar_pyramid(x, levels):
    """L-level pyramid by iterating eq. 5 on the approximation band (section 2.2).

    Returns ``(A, D)`` where ``A[j]`` is the level-j approximation
    (``A[0] = x``) and ``D[j]`` the level-j detail (``D[0] is None``), for
    j = 0..levels.  The signal axis is axis 0 (the token axis, section 3.1).
    """
    x = np.asarray(x, dtype=np.float64)
    if levels < 0 or x.shape[0] % (1 << levels) != 0:
        raise ValueError("token count must be a multiple of 2**levels")
    approx = [x]
    detail = [None]
    for _ in range(levels):
        a, dd = analysis_step(approx[-1])
        approx.append(a)
        detail.append(dd)
    return approx, detail


def haar_reconstruct(a_top, details):
    """Rebuild the signal from ``{A_L, D_L, ..., D_1}`` (``details[j]`` = D_j, j >= 1)."""
    x = np.asarray(a_top, dtype=np.float64)
    for j in range(len(details) - 1, 0, -1):
        x = synthesis_step(x, details[j])
    return x


AGGREGATIONS = ("max", "mean", "softmax_max", "softmax_mean")


def refresh_top(a_top, k_prompt_new, blocks, levels):
    """Incremental refresh of the level-L approximation of a head's pyramid.

    The cached prompt keys change on the cache's own schedule (section 2.1,
    eq. 4, for the positions a step recomputes); the low-frequency keys of
    section 3.1 are the DWT of the current cache.  Rows ``blocks`` of the
    old ``a_top`` (``[n_L, d]``) are recomputed from the new keys by the
    pyramid itself (eq. 5 iterated); every other row is kept as it was.
    """
    out = np.array(a_top, dtype=np.float64, copy=True)
    approx, _ = haar_pyramid(k_prompt_new, levels)
    for b in set(int(x) for x in blocks):
        out[b] = approx[levels][b]
    return out


def level_scores(q, coeff_rows, agg="max"):
    """Score of each region: the query rows' scaled dot products, aggregated.

    ``q`` is ``[n_q, d]``, ``coeff_rows`` is ``[m, d]`` (the approximation
    coefficients of the m candidate regions).  Returns ``[m]`` with
    ``s[c] = max_i (q_i . a_c) / sqrt(d)`` for ``agg="max"`` and the mean
    over i for ``agg="mean"``.  The dot product against the low-frequency
    keys is the "correlation" of Figure 2 (c); the 1/sqrt(d) factor is the
    one of eq. 3; how the query block is combined is not stated on the
    pages: the maximum is the main reading, the mean a variant.

    The variants "softmax_max" and "softmax_mean" score with attention
    probabilities instead of logits (section 1 speaks of the attention the
    queries pay to key regions): each row's logits are normalised by a
    softmax over the m candidates passed in (the level's candidate set),
    ``p_i[c] = exp(l_ic) / sum_c' exp(l_ic')``, and ``s[c]`` is the maximum
    or the mean over i of ``p_i[c]``.
    """
    if agg not in AGGREGATIONS:
        raise ValueError("unknown aggregation")
    q = np.asarray(q, dtype=np.float64)
    coeff_rows = np.asarray(coeff_rows, dtype=np.float64)
    d = q.shape[1]
    logits = q @ coeff_rows.T / math.sqrt(d)
    if agg == "max":
        return logits.max(axis=0)
    if agg == "mean":
        return logits.mean(axis=0)
    # softmax of every row over the candidates (max-subtracted for range safety)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return p.max(axis=0) if agg == "softmax_max" else p.mean(axis=0)


def top_k(candidates, scores, k):
    """Top-K choice (Figure 2 (c)/(d)): keep the k best candidates.

    Order is higher score first, and on equal scores the lower candidate
    index first.  Returns ``(chosen_ascending, gap)`` where ``gap`` is the
    relative distance between the k-th best and the (k+1)-th best score,
    ``(s_k - s_k1) / max(|s_k|, |s_k1|)``, or +inf when every candidate is
    kept.
    """
    candidates = np.asarray(candidates, dtype=np.int64)
    scores = np.asarray(scores, dtype=np.float64)
    if not 0 <= k <= len(candidates):
        raise ValueError("k out of range")
    order = sorted(range(len(candidates)), key=lambda i: (-scores[i], candidates[i]))
    chosen = np.sort(candidates[order[:k]])
    if k == len(candidates) or k == 0:
        gap = math.inf
    else:
        s_in = scores[order[k - 1]]
        s_out = scores[order[k]]
        den = max(abs(s_in), abs(s_out))
        gap = 0.0 if den == 0.0 else (s_in - s_out) / den
    return chosen, gap


@dataclass
class SelectResult:
    """Outcome of the coarse-to-fine selection for one head.

    ``sel[j]`` are the chosen level-j region indices (ascending), ``cand[j]``
    the level-j candidates and ``scores[j]`` their scores (aligned with
    ``cand[j]``), ``gap[j]`` the relative boundary gap, for j = 0..L.
    ``sel[0]`` are prompt token indices.
    """

    levels: int
    sel: dict = field(default_factory=dict)
    cand: dict = field(default_factory=dict)
    scores: dict = field(default_factory=dict)
    gap: dict = field(default_factory=dict)
    approx: list = None
    detail: list = None


def select(q, k_prompt, budgets, levels, agg="max", wavelet="haar"):
    """Coarse-to-fine token selection for one head.

    Steps (WaveFilter section 3.1 and Figure 2 (b)-(d)):

    1. Haar pyramid of the prompt keys along the token axis (eq. 5).
    2. Level L: every coefficient of A_L is a candidate; score it against the
       query block and keep the top ``budgets[0]`` (the coarse Top-K).
    3. For j = L-1 down to 0: the candidates are the two children of every
       region kept at level j+1; score them with A_j and keep the top
       ``budgets[L-j]``.

    ``budgets`` lists k_L, k_{L-1}, ..., k_0; ``agg`` is the aggregation of
    ``level_scores``; ``wavelet`` the basis of ``dwt_pyramid``.  With a
    longer basis a coefficient's support reaches past its block of 2^j
    tokens, but the refinement tree is the same: the children of level-(j+1)
    coefficient n are level-j coefficients 2n and 2n+1.  Returns a
    ``SelectResult``.
    """
    q = np.asarray(q, dtype=np.float64)
    if len(budgets) != levels + 1:
        raise ValueError("need one budget per level L..0")
    approx, detail = dwt_pyramid(k_prompt, levels, wavelet)
    res = SelectResult(levels=levels, approx=approx, detail=detail)
    n_top = approx[levels].shape[0]
    cand = np.arange(n_top)
    for j in range(levels, -1, -1):
        if j < levels:
            parents = res.sel[j + 1]
            cand = np.sort(np.concatenate([2 * parents, 2 * parents + 1]))
        s = level_scores(q, approx[j][cand], agg)
        chosen, gap = top_k(cand, s, budgets[levels - j])
        res.cand[j] = cand
        res.scores[j] = s
        res.sel[j] = chosen
        res.gap[j] = gap
    return res


def attend(q, keys, values):
    """Softmax attention of eq. 3 over the given key/value rows (no mask).

    ``O_i = sum_t softmax_t(q_i . k_t / sqrt(d)) v_t`` with the softmax taken
    over exactly the rows passed in.  Max-subtracted for range safety.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    d = q.shape[1]
    z = q @ keys.T / math.sqrt(d)
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    w /= w.sum(axis=1, keepdims=True)
    return w @ values


def select_attend(q, k_all, v_all, n_prompt, gen_idx, budgets, levels, agg="max", wavelet="haar"):
    """One per-step call for one head: select prompt tokens, then attend.

    ``k_all``/``v_all`` are the cached rows ``[N_tot, d]`` with the prompt at
    rows ``[0, n_prompt)``; ``gen_idx`` are the generated positions, which
    are attended in full and never scored.  The attended set is the chosen
    prompt tokens (ascending) followed by ``gen_idx`` (eq. 3 restricted to
    that set).  Returns ``(O, SelectResult)``.
    """
    k_all = np.asarray(k_all, dtype=np.float64)
    v_all = np.asarray(v_all, dtype=np.float64)
    res = select(q, k_all[:n_prompt], budgets, levels, agg, wavelet)
    rows = np.concatenate([res.sel[0], np.asarray(gen_idx, dtype=np.int64)])
    out = attend(q, k_all[rows], v_all[rows])
    return out, res


def attend_selected(q, k_all, v_all, sel, gen_idx):
    """Attention of a later step over a selection made earlier (one head).

    The pages say the DWT is taken at the initial time step to locate the
    key tokens (section 1, section 3.1); one reading is that the selection
    itself is then kept for the following denoising steps, so a later step
    only attends.  This is eq. 3 restricted to the given prompt tokens
    ``sel`` followed by the generated positions ``gen_idx``, with the
    current queries ``q``: exactly the attention stage of ``select_attend``
    with the selection handed in.
    """
    k_all = np.asarray(k_all, dtype=np.float64)
    v_all = np.asarray(v_all, dtype=np.float64)
    rows = np.concatenate([np.asarray(sel, dtype=np.int64), np.asarray(gen_idx, dtype=np.int64)])
    return attend(q, k_all[rows], v_all[rows])
