"""Pins of the oracle's attention (WaveFilter section 2.1, eq. 3).

With no pyramid (L = 0) and a budget covering every prompt token, the
per-step call must be plain dense attention over all cached positions: it is
checked against torch's CPU float64 ``scaled_dot_product_attention``.  Closed
forms (identical keys, constant values) and permutation invariance cover the
restricted case.
"""

import numpy as np
import pytest
import torch

from oracle import attend, attend_selected, select_attend


@pytest.mark.parametrize("n_p,n_g,d", [(64, 8, 16), (256, 0, 32), (128, 32, 64)])
def test_dense_limit_matches_library_attention(n_p, n_g, d):
    rng = np.random.default_rng(n_p + d)
    q = rng.standard_normal((12, d))
    k = rng.standard_normal((n_p + n_g, d)) * 2.0
    v = rng.standard_normal((n_p + n_g, d))
    out, res = select_attend(q, k, v, n_p, np.arange(n_p, n_p + n_g), [n_p], 0)
    assert list(res.sel[0]) == list(range(n_p))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0].numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_identical_keys_average_values():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((5, 8))
    k = np.tile(rng.standard_normal((1, 8)), (20, 1))
    v = rng.standard_normal((20, 8))
    np.testing.assert_allclose(attend(q, k, v), np.tile(v.mean(axis=0), (5, 1)), atol=1e-14)


def test_constant_values():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((5, 8)) * 4
    k = rng.standard_normal((30, 8)) * 4
    v = np.full((30, 8), -0.625)
    np.testing.assert_allclose(attend(q, k, v), -0.625, atol=1e-14)


def test_permutation_invariance():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((5, 8))
    k = rng.standard_normal((40, 8))
    v = rng.standard_normal((40, 8))
    p = rng.permutation(40)
    np.testing.assert_allclose(attend(q, k[p], v[p]), attend(q, k, v), atol=1e-14)


def test_restricted_set_is_selected_plus_generated():
    rng = np.random.default_rng(3)
    n_p, n_g, d = 64, 6, 8
    q = rng.standard_normal((4, d))
    k = rng.standard_normal((n_p + n_g, d))
    v = rng.standard_normal((n_p + n_g, d))
    gen = np.array([n_p + 5, n_p + 1, n_p + 3])
    out, res = select_attend(q, k, v, n_p, gen, [4, 6, 12], 2)
    rows = list(res.sel[0]) + list(gen)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k[rows])[None], torch.from_numpy(v[rows])[None])[0].numpy()
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_reused_selection_matches_select_attend_and_library():
    """A selection made at one step, attended with the same queries, gives
    select_attend's output; with the next step's queries it is eq. 3 over the
    same rows (checked against torch's float64 attention)."""
    rng = np.random.default_rng(9)
    n_p, n_g, d = 256, 12, 16
    q0 = rng.standard_normal((8, d))
    q1 = rng.standard_normal((8, d))
    k = rng.standard_normal((n_p + n_g, d))
    v = rng.standard_normal((n_p + n_g, d))
    gen = np.arange(n_p, n_p + n_g)
    out0, res = select_attend(q0, k, v, n_p, gen, [6, 12, 24, 40], 3)
    np.testing.assert_array_equal(attend_selected(q0, k, v, res.sel[0], gen), out0)
    rows = list(res.sel[0]) + list(gen)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q1)[None], torch.from_numpy(k[rows])[None], torch.from_numpy(v[rows])[None])[0].numpy()
    np.testing.assert_allclose(attend_selected(q1, k, v, res.sel[0], gen), ref, atol=1e-12)
    # only generated positions, and only prompt tokens
    ref_g = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q1)[None], torch.from_numpy(k[gen])[None], torch.from_numpy(v[gen])[None])[0].numpy()
    np.testing.assert_allclose(attend_selected(q1, k, v, np.zeros(0, dtype=np.int64), gen), ref_g, atol=1e-12)
    np.testing.assert_allclose(attend_selected(q1, k, v, np.arange(n_p), np.zeros(0, dtype=np.int64)),
                               attend(q1, k[:n_p], v[:n_p]), atol=1e-14)

