"""Workload recipe, budget schedules and margin planting (CPU)."""

import numpy as np
import pytest
import torch

from oracle import select
from oracle.planting import plant_margins
from workloads.configs import CONFIGS, resolve_budgets, check_budgets
from workloads.gen import make_layer, span_layout, to_f64

# Resolved schedules k_L..k_0 (rule in workloads.configs.resolve_budgets).
EXPECTED_BUDGETS = {
    1: [8, 16, 32, 64],
    2: [64, 112, 192, 320, 512],
    3: [16, 32, 64, 128, 256, 512],
    4: [64, 118, 214, 384, 683, 1195, 2048],
    5: [64, 119, 220, 403, 732, 1317, 2341, 4096],
}


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_budgets(cid):
    cfg = CONFIGS[cid]
    assert cfg.budgets == EXPECTED_BUDGETS[cid]
    assert check_budgets(cfg.n_prompt, cfg.levels, cfg.budgets)


def test_the_16k_workload_has_two_budget_readings():
    from workloads.configs import C3_READINGS, budget_reading
    capped, full = C3_READINGS["capped"], C3_READINGS["full"]
    assert capped is CONFIGS[3] and capped.budgets == EXPECTED_BUDGETS[3]
    # coarse top-16 dropped: k_L = min(512, 2 ceil(1024 / 32)) = 64, and k_0 reaches B = 1 024
    assert full.budgets == [64, 116, 205, 359, 615, 1024]
    assert check_budgets(full.n_prompt, full.levels, full.budgets)
    assert budget_reading(capped) == "capped" and budget_reading(full) == "full"
    assert budget_reading(CONFIGS[4]) is None
    # same inputs under both readings
    a, b = make_layer(capped, 0), make_layer(full, 0)
    assert torch.equal(a.k, b.k) and torch.equal(a.q, b.q)


def test_budget_rule_edges():
    assert resolve_budgets(64, 0, 16) == [16]
    assert resolve_budgets(64, 6, 64) == [1, 2, 4, 8, 16, 32, 64]
    assert not check_budgets(64, 2, [4, 9, 12])      # k_1 > 2 k_2
    assert not check_budgets(64, 2, [17, 20, 30])    # k_2 > n_2
    with pytest.raises(ValueError):
        resolve_budgets(100, 3, 10)


def test_generator_is_deterministic_and_layered():
    a = make_layer(1, 0)
    b = make_layer(1, 0)
    c = make_layer(1, 1)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert torch.equal(x, y)
    assert not torch.equal(a.k, c.k)
    assert a.k.dtype == torch.float32 and a.k.shape == (1, 2, 1056, 64)
    assert list(a.gen_idx) == list(range(1024, 1056))


def test_spans_are_planted_needles():
    inp = make_layer(2, 0)
    cfg = inp.cfg
    assert inp.k.dtype == torch.bfloat16
    for (b, h), lay in inp.spans.items():
        assert len(lay) == cfg.n_spans
        ends = [o + n for o, n in lay]
        assert all(o >= 0 for o, _ in lay) and max(ends) <= cfg.n_prompt
        assert all(ends[i] <= lay[i + 1][0] for i in range(len(lay) - 1))
        qbar = to_f64(inp.q[b, h]).mean(axis=0)
        for o, n in lay:
            rows = to_f64(inp.k[b, h, o:o + n])
            resid = rows - cfg.alpha * qbar
            assert np.abs(resid).max() < 0.8 and np.abs(resid).std() < 0.15
    assert span_layout(cfg, 0, 0, 3) == inp.spans[(0, 3)]


def test_student_t_keys_are_heavy_tailed():
    from workloads.gen import _randn
    gen = torch.Generator().manual_seed(0)
    z = _randn((5, 200000), gen, "cpu")
    t = z[0] / torch.sqrt((z[1:] ** 2).sum(0) / 4.0)
    # Student-t(4): variance nu/(nu-2) = 2, excess kurtosis infinite; check the variance and tails
    assert abs(float(t.var()) - 2.0) < 0.15
    assert float((t.abs() > 4.6).float().mean()) > 5e-3  # P(|t4| > 4.6) ~ 0.01


@pytest.mark.parametrize("cid,heads", [(1, [0, 1]), (2, [0, 5])])
def test_margin_planting_converges(cid, heads):
    inp = make_layer(cid, 0)
    cfg = inp.cfg
    for h in heads:
        q = to_f64(inp.q[0, h])
        kp = to_f64(inp.k[0, h, :cfg.n_prompt])
        k_new, ops, ok = plant_margins(q, kp, cfg.budgets, cfg.levels)
        assert ok
        res = select(q, k_new, cfg.budgets, cfg.levels)
        assert min(res.gap.values()) > 2e-3
        # replaying the edits on the rounded tensor reproduces the same bytes
        kt = inp.k[0, h, :cfg.n_prompt].clone()
        for r0, r1, f in ops:
            kt[r0:r1] *= f
        assert np.array_equal(to_f64(kt), k_new)
