"""Pins of the oracle's Haar pyramid (WaveFilter section 2.2, eq. 5).

Each pin is independent of the oracle's own code: a direct-loop closed form,
the textbook orthonormal Haar matrix built by its Kronecker recursion, a
hand-worked example, and the invariants of an orthonormal transform.
"""

import math
import os

import numpy as np
import pytest

from oracle import HAAR_G as HAAR_G_, HAAR_H as HAAR_H_, haar_pyramid, haar_reconstruct, analysis_step, synthesis_step

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "haar_worked_example.txt")


def closed_form(x, j):
    """A_j[n] = 2^{-j/2} sum_{t in [n 2^j, (n+1) 2^j)} x[t] and
    D_j[n] = 2^{-j/2} (sum of the first half of that range - sum of the second half),
    by explicit loops."""
    n_out = x.shape[0] >> j
    a = np.zeros((n_out,) + x.shape[1:])
    dd = np.zeros_like(a)
    w = 1 << j
    for n in range(n_out):
        for t in range(n * w, (n + 1) * w):
            a[n] += x[t]
            if j >= 1:
                dd[n] += x[t] if t < n * w + w // 2 else -x[t]
    return a / 2 ** (j / 2), dd / 2 ** (j / 2)


def haar_matrix(n):
    """Orthonormal Haar matrix by H_{2m} = [H_m (x) (1, 1); I_m (x) (1, -1)] / sqrt2."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        m = h.shape[0]
        top = np.kron(h, np.array([[1.0, 1.0]]))
        bot = np.kron(np.eye(m), np.array([[1.0, -1.0]]))
        h = np.vstack([top, bot]) / math.sqrt(2.0)
    return h


@pytest.mark.parametrize("levels", [0, 1, 2, 3, 5, 6])
def test_closed_form(levels):
    rng = np.random.default_rng(1 + levels)
    x = rng.standard_normal((64, 3))
    approx, detail = haar_pyramid(x, levels)
    for j in range(levels + 1):
        a, dd = closed_form(x, j)
        np.testing.assert_allclose(approx[j], a, rtol=0, atol=1e-13)
        if j >= 1:
            np.testing.assert_allclose(detail[j], dd, rtol=0, atol=1e-13)


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64])
def test_textbook_haar_matrix(n):
    h = haar_matrix(n)
    np.testing.assert_allclose(h @ h.T, np.eye(n), atol=1e-13)
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n)
    levels = int(math.log2(n))
    approx, detail = haar_pyramid(x, levels)
    stacked = np.concatenate([approx[levels]] + [detail[j] for j in range(levels, 0, -1)])
    np.testing.assert_allclose(stacked, h @ x, atol=1e-13)


def _parse_golden():
    vals = {}
    r2 = math.sqrt(2.0)
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rhs = (s.strip() for s in line.split("=", 1))
            vals[key] = np.array([eval(e, {"r2": r2}) for e in rhs.split(",")], dtype=float)
    return vals


def test_hand_worked_example():
    g = _parse_golden()
    approx, detail = haar_pyramid(g["x"], 3)
    for j in (1, 2, 3):
        np.testing.assert_allclose(approx[j], g[f"A{j}"], atol=1e-14)
        np.testing.assert_allclose(detail[j], g[f"D{j}"], atol=1e-14)
    energy = (approx[3] ** 2).sum() + sum((detail[j] ** 2).sum() for j in (1, 2, 3))
    assert abs(energy - g["energy"][0]) < 1e-12


@pytest.mark.parametrize("levels", [1, 3, 6, 10])
def test_perfect_reconstruction(levels):
    rng = np.random.default_rng(10 + levels)
    x = rng.standard_normal((1024, 8)) * 3.0
    approx, detail = haar_pyramid(x, levels)
    y = haar_reconstruct(approx[levels], detail)
    assert np.max(np.abs(y - x)) <= 1e-12 * np.max(np.abs(x))


@pytest.mark.parametrize("levels", [1, 4, 7])
def test_parseval(levels):
    rng = np.random.default_rng(20 + levels)
    x = rng.standard_t(4, size=(512, 5))
    approx, detail = haar_pyramid(x, levels)
    e_in = (x ** 2).sum(axis=0)
    e_out = (approx[levels] ** 2).sum(axis=0) + sum((detail[j] ** 2).sum(axis=0) for j in range(1, levels + 1))
    np.testing.assert_allclose(e_out, e_in, rtol=1e-12)


def test_special_signals():
    c = 1.75
    approx, detail = haar_pyramid(np.full(64, c), 6)
    for j in range(1, 7):
        np.testing.assert_allclose(detail[j], 0.0, atol=1e-14)
        np.testing.assert_allclose(approx[j], c * 2 ** (j / 2), rtol=1e-14)
    alt = np.array([1.0, -1.0] * 32)
    approx, detail = haar_pyramid(alt, 1)
    np.testing.assert_allclose(approx[1], 0.0, atol=1e-15)
    np.testing.assert_allclose(detail[1], math.sqrt(2.0), rtol=1e-15)
    imp = np.zeros(64)
    imp[13] = 1.0
    approx, detail = haar_pyramid(imp, 6)
    for j in range(1, 7):
        nz = np.flatnonzero(approx[j])
        assert list(nz) == [13 >> j]
        assert abs(approx[j][13 >> j] - 2 ** (-j / 2)) < 1e-15


def test_single_step_roundtrip_and_shape_errors():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 2))
    a, dd = analysis_step(x)
    np.testing.assert_allclose(synthesis_step(a, dd), x, atol=1e-15)
    with pytest.raises(ValueError):
        analysis_step(np.zeros(5))
    with pytest.raises(ValueError):
        haar_pyramid(np.zeros((12, 2)), 3)


def test_refresh_recomputes_only_the_listed_blocks():
    """Incremental refresh: listed level-L blocks equal the block-sum closed
    form on the new keys (a direct loop), unlisted blocks keep their old
    rows even when their keys changed; an empty list and repeated entries
    change nothing more."""
    from oracle import refresh_top
    rng = np.random.default_rng(31)
    levels, n_p, d = 3, 64, 5
    k_old = rng.standard_normal((n_p, d))
    a_old, _ = haar_pyramid(k_old, levels)
    k_new = k_old.copy()
    k_new[8:10] += 1.0      # block 1
    k_new[40] -= 2.0        # block 5
    k_new[60:64] *= 3.0     # block 7, left out of the list below
    got = refresh_top(a_old[levels], k_new, [1, 5, 5], levels)
    for b in range(n_p >> levels):
        if b in (1, 5):
            want = [sum(k_new[t, c] for t in range(b * 8, b * 8 + 8)) * 2.0 ** (-levels / 2) for c in range(d)]
            assert np.allclose(got[b], want, atol=1e-12)
        else:
            assert np.array_equal(got[b], a_old[levels][b])
    assert np.array_equal(refresh_top(a_old[levels], k_new, [], levels), a_old[levels])
    full = refresh_top(a_old[levels], k_new, range(n_p >> levels), levels)
    assert np.allclose(full, haar_pyramid(k_new, levels)[0][levels], atol=1e-12)


# -- Daubechies' four-tap basis (the longer-wavelet variant) -----------------

def test_db2_filter_identities():
    """The defining identities of an orthonormal four-tap pair with two
    vanishing moments: sum g = sqrt2, unit energy, orthogonal to its even
    shifts, h a quadrature mirror with zero sum and zero first moment."""
    from oracle import DB2_G as g, DB2_H as h
    assert abs(g.sum() - math.sqrt(2.0)) < 1e-14
    assert abs((g * g).sum() - 1.0) < 1e-14
    assert abs(g[0] * g[2] + g[1] * g[3]) < 1e-14
    assert abs(h.sum()) < 1e-14 and abs((np.arange(4) * h).sum()) < 1e-14
    assert abs((g * h).sum()) < 1e-14 and abs(g[0] * h[2] + g[1] * h[3]) < 1e-14


def test_db2_periodic_level_is_orthogonal():
    """The periodic analysis level as a matrix (applied to unit vectors) is
    orthogonal: Parseval holds and its transpose reconstructs."""
    from oracle import DB2_G, DB2_H, analysis_step_periodic
    n = 16
    w = np.zeros((n, n))
    for i in range(n):
        e = np.zeros(n)
        e[i] = 1.0
        a, dd = analysis_step_periodic(e, DB2_G, DB2_H)
        w[:, i] = np.concatenate([a, dd])
    assert np.allclose(w @ w.T, np.eye(n), atol=1e-13)
    x = np.random.default_rng(41).standard_normal(n)
    a, dd = analysis_step_periodic(x, DB2_G, DB2_H)
    assert abs((a * a).sum() + (dd * dd).sum() - (x * x).sum()) < 1e-12


def test_db2_annihilates_lines_away_from_the_wrap():
    """Two vanishing moments: a linear signal has zero detail wherever the
    filter does not wrap around the end; a constant gives sqrt2 x c."""
    from oracle import DB2_G, DB2_H, analysis_step_periodic
    x = 0.3 + 0.7 * np.arange(32.0)
    _, dd = analysis_step_periodic(x, DB2_G, DB2_H)
    assert np.abs(dd[:15]).max() < 1e-12 and abs(dd[15]) > 1.0
    a, dd = analysis_step_periodic(np.full(8, 2.5), DB2_G, DB2_H)
    assert np.allclose(a, 2.5 * math.sqrt(2.0)) and np.abs(dd).max() < 1e-12


def test_periodic_step_with_haar_is_the_plain_step():
    from oracle import analysis_step_periodic, dwt_pyramid
    x = np.random.default_rng(42).standard_normal((16, 3))
    a1, d1 = analysis_step_periodic(x, HAAR_G_, HAAR_H_)
    a2, d2 = analysis_step(x)
    assert np.allclose(a1, a2, atol=1e-15) and np.allclose(d1, d2, atol=1e-15)
    ap, _ = dwt_pyramid(x, 3, "haar")
    hp, _ = haar_pyramid(x, 3)
    assert all(np.array_equal(ap[j], hp[j]) for j in range(4))


def test_db2_selection_tree_and_scores():
    """With the db2 basis the selection still refines children 2n, 2n+1, and
    each level's candidate scores are the query block's dot products with
    the level's db2 coefficients (checked against a direct cascade loop)."""
    from oracle import DB2_G, select
    rng = np.random.default_rng(43)
    q = rng.standard_normal((3, 4))
    kp = rng.standard_normal((32, 4))
    res = select(q, kp, [2, 3, 5, 9], 3, wavelet="db2")
    for j in range(2, -1, -1):
        assert set(res.cand[j]) == set(2 * c for c in res.sel[j + 1]) | set(2 * c + 1 for c in res.sel[j + 1])
    # level-2 coefficients by an explicit two-step loop with wrap-around
    lv1 = np.array([[sum(DB2_G[m] * kp[(2 * n + m) % 32, c] for m in range(4)) for c in range(4)] for n in range(16)])
    lv2 = np.array([[sum(DB2_G[m] * lv1[(2 * n + m) % 16, c] for m in range(4)) for c in range(4)] for n in range(8)])
    s_want = (q @ lv2[res.cand[2]].T / 2.0).max(axis=0)
    assert np.allclose(res.scores[2], s_want, atol=1e-12)
