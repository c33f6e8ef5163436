"""The GPU tests' checking machinery, pinned on the CPU: the process-pool
planting equals the serial one, and the Top-K validity check used for heads
whose margins are not planted accepts the oracle's own selection and rejects
a selection with a planted mistake."""

import dataclasses

import numpy as np
import torch

import _pool
from _parity import bits, plant, plant_many, split_levels_np
from oracle import select_attend
from workloads.configs import CONFIGS
from workloads.gen import make_layer, to_f64


def small(cid=40, heads=2):
    return dataclasses.replace(CONFIGS[2], cid=cid, heads=heads, n_prompt=1024, n_gen=16, levels=4)


def test_pool_planting_equals_serial_planting():
    cfg = small()
    a, b = make_layer(cfg, 0), make_layer(cfg, 0)
    heads = [(0, h) for h in range(cfg.heads)]
    assert all(plant(a, heads).values())
    assert all(plant_many(b, heads))
    assert torch.equal(a.k, b.k)


def _job(inp, h, levels_sel, band=1e-3):
    cfg = inp.cfg
    return (0, cfg.dtype, bits(inp.q[0, h]), bits(inp.k[0, h]), bits(inp.v[0, h]), cfg.n_prompt,
            inp.gen_idx.numpy().astype(np.int64), list(cfg.budgets), cfg.levels, "max", "haar", levels_sel, band)


def test_decode_is_exact():
    x = torch.randn(1000).bfloat16()
    assert np.array_equal(_pool.decode(bits(x), "bf16"), to_f64(x))
    y = torch.randn(1000)
    assert np.array_equal(_pool.decode(bits(y), "f32"), to_f64(y))


def test_validity_accepts_the_oracles_own_selection():
    cfg = small(41)
    inp = make_layer(cfg, 0)
    out, res = select_attend(to_f64(inp.q[0, 0]), to_f64(inp.k[0, 0]), to_f64(inp.v[0, 0]), cfg.n_prompt,
                             inp.gen_idx.numpy(), cfg.budgets, cfg.levels)
    _, err, (o, margin) = _pool.validity_job(_job(inp, 0, {j: res.sel[j] for j in res.sel}))
    assert err is None and margin >= 0
    assert np.abs(o - out).max() < 1e-12


def test_validity_rejects_a_swapped_token():
    """Level 0 keeps its worst candidate's place for the best dropped one's
    sibling with the lowest score: a clear Top-K violation."""
    cfg = small(42)
    inp = make_layer(cfg, 0)
    _, res = select_attend(to_f64(inp.q[0, 0]), to_f64(inp.k[0, 0]), to_f64(inp.v[0, 0]), cfg.n_prompt,
                           inp.gen_idx.numpy(), cfg.budgets, cfg.levels)
    cand, s, sel = res.cand[0], res.scores[0], res.sel[0]
    dropped = cand[~np.isin(cand, sel)]
    worst_dropped = dropped[np.argmin(s[np.searchsorted(cand, dropped)])]
    best_kept = sel[np.argmax(s[np.searchsorted(cand, sel)])]
    bad = np.sort(np.concatenate([sel[sel != best_kept], [worst_dropped]]))
    lv = {j: res.sel[j] for j in res.sel}
    lv[0] = bad
    _, err, _ = _pool.validity_job(_job(inp, 0, lv))
    assert err is not None and "level 0" in err


def test_validity_rejects_a_token_outside_the_candidates():
    cfg = small(43)
    inp = make_layer(cfg, 0)
    _, res = select_attend(to_f64(inp.q[0, 0]), to_f64(inp.k[0, 0]), to_f64(inp.v[0, 0]), cfg.n_prompt,
                           inp.gen_idx.numpy(), cfg.budgets, cfg.levels)
    lv = {j: res.sel[j].copy() for j in res.sel}
    outside = np.setdiff1d(np.arange(cfg.n_prompt), res.cand[0])[0]
    lv[0][0] = outside
    lv[0] = np.sort(lv[0])
    _, err, _ = _pool.validity_job(_job(inp, 0, lv))
    assert err is not None


def test_split_levels_np_order():
    flat = np.arange(1 + 2 + 3)
    out = split_levels_np(flat, [1, 2, 3])
    assert list(out[2]) == [0] and list(out[1]) == [1, 2] and list(out[0]) == [3, 4, 5]
