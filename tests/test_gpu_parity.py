"""GPU parity of the HIP path against the float64 oracle (through the C ABI).

Selected index sets must match the oracle exactly at every level whose
boundary gap exceeds 1e-3 (margins are planted so that all do); attention
outputs must match within 2e-3 (bfloat16 inputs) or 1e-5 (float32).
"""

import dataclasses

import numpy as np
import pytest
import torch

import long_context_kv_haar_amd as wf
from oracle import haar_pyramid
from workloads.configs import C3_READINGS, CONFIGS, Config, budget_reading
from workloads.gen import make_layer, to_f64

from _parity import (TOL, check_head, check_structure, check_validity_many, oracle_many, plant, plant_many,
                     say, torch_attend_all)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(inp):
    inp.q, inp.k, inp.v, inp.gen_idx = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.gen_idx))
    return inp


def run(inp, budgets=None, levels=None, flags=0):
    cfg = inp.cfg
    budgets = cfg.budgets if budgets is None else budgets
    levels = cfg.levels if levels is None else levels
    pyr = wf.build_pyramid(inp.k, cfg.n_prompt, levels, flags)
    res = wf.select_attend(inp.q, pyr, inp.k, inp.v, inp.gen_idx, budgets, levels_out=True)
    torch.cuda.synchronize()
    return pyr, res


@pytest.mark.parametrize("cid", [1, 2, 3])
def test_pyramid_matches_oracle(cid):
    say(f"[pyramid c{cid}]")
    inp = to_dev(make_layer(cid, 0))
    cfg = inp.cfg
    for flags in (0, wf.WF_PYR_ALL_LEVELS):
        pyr = wf.build_pyramid(inp.k, cfg.n_prompt, cfg.levels, flags)
        torch.cuda.synchronize()
        for h in range(cfg.heads):
            approx, detail = haar_pyramid(to_f64(inp.k[0, h, :cfg.n_prompt]), cfg.levels)
            top = pyr.top[0, h].cpu().numpy()
            assert np.abs(top - approx[cfg.levels]).max() <= 1e-5 * (1 + np.abs(approx[cfg.levels]).max())
            if flags:
                for j in range(1, cfg.levels + 1):
                    for band, ref in ((0, approx[j]), (1, detail[j])):
                        got = pyr.band(band, j)[0, h].cpu().numpy()
                        assert np.abs(got - ref).max() <= 1e-5 * (1 + np.abs(ref).max()), (band, j)


@pytest.mark.parametrize("cid", [1, 2])
def test_select_attend_matches_oracle(cid):
    say(f"[select_attend c{cid}]")
    _select_attend_case(make_layer(cid, 0))


def test_select_attend_16k_budget_readings(c3_reading):
    """The 16K workload under the reading of its budgets chosen with
    --c3-reading (both by default); the result names the reading."""
    cfg = C3_READINGS[c3_reading]
    say(f"[select_attend 16K, budget reading {budget_reading(cfg)}: {cfg.budgets}]")
    _select_attend_case(make_layer(cfg, 0))


def _select_attend_case(inp):
    cfg = inp.cfg
    heads = [(0, h) for h in range(cfg.heads)]
    ok = plant(inp, heads)
    assert all(ok.values())
    to_dev(inp)
    _, res = run(inp)
    check_structure(res, cfg.budgets, cfg.levels, cfg.n_prompt)
    unpinned = sum(check_head(inp, res, b, h) for b, h in heads)
    assert unpinned == 0


@pytest.mark.timeout(900)
def test_full_size_64k():
    """The 64K-token workload at its full size, in the launch shape the
    benchmark times: every one of the 32 heads is planted and compared with
    the oracle (exact kept indices at every level, O within 2e-3)."""
    say("[full size c4] generate")
    inp = make_layer(4, 0, device=DEV)
    cfg = inp.cfg
    heads = [(0, h) for h in range(cfg.heads)]
    say(f"[full size c4] plant {len(heads)} heads")
    assert all(plant_many(inp, heads))
    pyr, res = run(inp)
    say("[full size c4] oracle")
    ora = oracle_many(inp, heads)
    check_structure(res, cfg.budgets, cfg.levels, cfg.n_prompt)
    for (b, h), o in zip(heads, ora):
        assert check_head(inp, res, b, h, ora=o) == 0
        approx, _ = haar_pyramid(to_f64(inp.k[b, h, :cfg.n_prompt]), cfg.levels)
        top = pyr.top[b, h].cpu().numpy()
        assert np.abs(top - approx[cfg.levels]).max() <= 1e-5 * (1 + np.abs(approx[cfg.levels]).max())
    say(f"[full size c4] {len(heads)} heads exact")
    assert torch_attend_all(inp, res) <= TOL["bf16"]


def c5_sample(layer, cfg):
    """The planted head of one layer of the 128K sweep: the sequences
    alternate over the layers and the head index steps by 13 (mod 32), so the
    32 layers visit every head index once and both sequences 16 times."""
    return (layer % cfg.batch, (13 * layer + 5) % cfg.heads)


@pytest.mark.timeout(1200)
def test_full_size_128k_32_layers():
    """32 layers x 2 sequences x 32 heads of a 128K-token prompt resident at
    once (about 128 GiB of KV), every layer built and stepped.  One head per
    layer is planted and compared with the oracle exactly (a stratified
    sample: every layer, both sequences, every head index); in four layers
    four more heads each, not planted, are checked as valid Top-K selections
    under the oracle's scores, with O against the oracle over the device's
    own set."""
    cfg = CONFIGS[5]
    layers = []
    planted = [(layer, c5_sample(layer, cfg)) for layer in range(cfg.layers)]
    try:
        for layer in range(cfg.layers):
            say(f"[full size c5] generate layer {layer}")
            layers.append(make_layer(5, layer, device=DEV))
        say(f"[full size c5] plant {len(planted)} heads")
        assert all(plant_many([(layers[layer], bh) for layer, bh in planted], max_iter=256))
        pyrs = [wf.build_pyramid(inp.k, cfg.n_prompt, cfg.levels) for inp in layers]
        results = [wf.select_attend(inp.q, pyrs[i], inp.k, inp.v, inp.gen_idx, cfg.budgets, levels_out=True)
                   for i, inp in enumerate(layers)]
        torch.cuda.synchronize()
        say("[full size c5] structure")
        for layer in range(cfg.layers):
            check_structure(results[layer], cfg.budgets, cfg.levels, cfg.n_prompt)
        say("[full size c5] oracle on the planted heads")
        ora = oracle_many([(layers[layer], bh) for layer, bh in planted])
        for (layer, (b, h)), o in zip(planted, ora):
            assert check_head(layers[layer], results[layer], b, h, ora=o) == 0, (layer, b, h)
        say("[full size c5] validity of unplanted heads")
        extra = [(layers[layer], results[layer], ((layer + 1 + i) % cfg.batch, (7 * i + layer) % cfg.heads))
                 for layer in (1, 10, 21, 31) for i in range(4)]
        extra = [e for e in extra if (e[0].layer, e[2]) not in set(planted)]
        worst = check_validity_many(extra)
        say(f"[full size c5] {len(planted)} planted heads exact, {len(extra)} unplanted heads valid "
            f"(least relative margin {worst:.3g})")
        assert torch_attend_all(layers[cfg.layers - 1], results[cfg.layers - 1]) <= TOL["bf16"]
        say("[full size c5] all 32 layers in one batched call")
        batched = wf.select_attend_layers([(inp.q, pyrs[i], inp.k, inp.v) for i, inp in enumerate(layers)],
                                          layers[0].gen_idx, cfg.budgets)
        torch.cuda.synchronize()
        for layer in range(cfg.layers):
            # the same kept tokens for every head; O to float32 rounding (other split sums)
            assert torch.equal(batched[layer]["sel"], results[layer]["sel"]), layer
            assert (batched[layer]["out"] - results[layer]["out"]).abs().max().item() <= 1e-5, layer
        for (layer, (b, h)), o in zip(planted, ora):
            err = np.abs(batched[layer]["out"][b, h].double().cpu().numpy() - o.out).max()
            assert err <= TOL["bf16"], (layer, b, h, err)
        say(f"[full size c5] batched call: every head's kept tokens equal, O within 1e-5 of the per-layer calls")
    finally:
        del layers
        torch.cuda.empty_cache()


@pytest.mark.parametrize("agg", ["max", "mean"])
def test_batched_layers_match_per_layer_calls(agg):
    """Three 4K-token layers (own seeds) in one batched call: every head's
    kept tokens equal the per-layer call's, O agrees to float32 rounding, and
    one planted head per layer matches the oracle.  A batch of one layer is
    the per-layer call bit for bit."""
    cfg = CONFIGS[2]
    say(f"[batched layers {agg}]")
    layers = [make_layer(cfg, layer) for layer in range(3)]
    planted = [(layer, (0, (11 * layer + 3) % cfg.heads)) for layer in range(3)]
    assert all(plant_many([(layers[layer], bh) for layer, bh in planted], agg=agg))
    for inp in layers:
        to_dev(inp)
    pyrs = [wf.build_pyramid(inp.k, cfg.n_prompt, cfg.levels) for inp in layers]
    single = [wf.select_attend(inp.q, pyrs[i], inp.k, inp.v, inp.gen_idx, cfg.budgets, agg=agg)
              for i, inp in enumerate(layers)]
    batched = wf.select_attend_layers([(inp.q, pyrs[i], inp.k, inp.v) for i, inp in enumerate(layers)],
                                      layers[0].gen_idx, cfg.budgets, agg=agg)
    one = wf.select_attend_layers([(layers[1].q, pyrs[1], layers[1].k, layers[1].v)], layers[1].gen_idx,
                                  cfg.budgets, agg=agg)
    torch.cuda.synchronize()
    for layer in range(3):
        assert torch.equal(batched[layer]["sel"], single[layer]["sel"])
        assert (batched[layer]["out"] - single[layer]["out"]).abs().max().item() <= 1e-5
    assert torch.equal(one[0]["sel"], single[1]["sel"])
    assert torch.equal(one[0]["out"].view(torch.int32), single[1]["out"].view(torch.int32))
    ora = oracle_many([(layers[layer], bh) for layer, bh in planted], agg=agg)
    for (layer, (b, h)), o in zip(planted, ora):
        np.testing.assert_array_equal(batched[layer]["sel"][b, h].cpu().numpy(), o.sel[0])
        assert np.abs(batched[layer]["out"][b, h].double().cpu().numpy() - o.out).max() <= TOL["bf16"]


def test_batched_layers_reject_mismatched_layers():
    cfg = CONFIGS[1]
    say("[batched layers reject]")
    a, b = to_dev(make_layer(cfg, 0)), to_dev(make_layer(cfg, 1))
    pa = wf.build_pyramid(a.k, cfg.n_prompt, cfg.levels)
    pb = wf.build_pyramid(b.k, cfg.n_prompt, cfg.levels - 1)  # other level count
    with pytest.raises((ValueError, wf.WfError)):  # the binding's checks see it first
        wf.select_attend_layers([(a.q, pa, a.k, a.v), (b.q, pb, b.k, b.v)], a.gen_idx, cfg.budgets)
    pf = wf.build_pyramid(b.k.bfloat16().contiguous(), cfg.n_prompt, cfg.levels)  # other element type
    with pytest.raises((ValueError, wf.WfError)):
        wf.select_attend_layers([(a.q, pa, a.k, a.v), (b.q, pf, b.k, b.v)], a.gen_idx, cfg.budgets)


def custom(base, **kw):
    return dataclasses.replace(CONFIGS[base], **kw)


EDGE = [
    # name, config, budgets, levels
    ("dense-L0-f32", custom(1, cid=90, n_prompt=512, n_gen=16, levels=0, n_spans=0), [512], 0),
    ("dense-L0-bf16", custom(2, cid=91, heads=2, n_prompt=256, n_gen=0, levels=0, n_spans=0), [256], 0),
    ("ragged-nq20-b2", custom(2, cid=92, batch=2, heads=3, n_q=20, n_prompt=2048, n_gen=7, levels=4), [5, 9, 17, 30, 50], 4),
    ("nq1-full-budget", custom(2, cid=93, heads=2, n_q=1, n_prompt=512, n_gen=3, levels=3),
     [64, 128, 256, 512], 3),
    ("nq64-L7", custom(5, cid=94, layers=1, batch=1, heads=2, n_q=64, n_prompt=8192, n_gen=40, levels=7, n_spans=4),
     [9, 17, 33, 60, 110, 200, 350, 600], 7),
    ("f32-d128", custom(2, cid=95, dtype="f32", heads=2, n_q=48, n_prompt=2048, levels=5), [6, 11, 20, 36, 64, 100], 5),
    ("bf16-d64", custom(2, cid=96, head_dim=64, heads=4, n_q=33, n_prompt=4096, n_gen=100, levels=6),
     [3, 6, 12, 23, 40, 70, 120], 6),
    ("L1", custom(1, cid=97, dtype="bf16", n_prompt=256, levels=1), [70, 101], 1),
    # selections too large for the register-resident Top-K take the general path
    ("coarse-8192-keys", custom(2, cid=86, heads=2, n_prompt=16384, n_gen=16, levels=1, n_spans=4),
     [300, 500], 1),
    ("coarse-20480-keys-global", custom(2, cid=87, head_dim=64, heads=1, n_prompt=20480, n_gen=8, levels=0,
                                        n_spans=2), [1000], 0),
    # more than 1 024 cover workgroups (64 heads x 17): the coarse Top-K runs in a launch of its own
    ("topk-apart-b2", custom(2, cid=89, batch=2, n_prompt=8192, n_gen=16, levels=3, n_spans=2),
     [520, 1000, 1900, 3000], 3),
    ("refine-6000-candidates", custom(4, cid=88, heads=2, n_prompt=32768, n_gen=32, levels=2, n_spans=4,
                                      key_law="normal"), [2000, 3000, 5600], 2),
]


@pytest.mark.parametrize("name,cfg,budgets,levels", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(name, cfg, budgets, levels):
    say(f"[edge {name}]")
    inp = make_layer(cfg, 0)
    heads = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    assert all(plant(inp, heads, budgets, levels).values())
    to_dev(inp)
    if cfg.n_gen == 0:
        inp.gen_idx = torch.zeros(0, dtype=torch.int32, device=DEV)
    elif name.startswith("ragged"):
        # generated positions in a scrambled order
        inp.gen_idx = inp.gen_idx[torch.randperm(cfg.n_gen, generator=torch.Generator().manual_seed(1)).to(DEV)]
    _, res = run(inp, budgets, levels)
    check_structure(res, budgets, levels, cfg.n_prompt)
    for b, h in heads:
        assert check_head(inp, res, b, h, budgets, levels) == 0


def test_exact_ties_take_the_lower_index():
    say("[ties]")
    cfg = custom(2, cid=98, heads=1, n_prompt=1024, n_gen=8, levels=4, n_spans=0)
    inp = make_layer(cfg, 0)
    # two identical 16-token regions far above the rest: regions 5 and 40
    inp.k[0, 0, 40 * 16:41 * 16] = inp.k[0, 0, 5 * 16:6 * 16] = (2.5 * inp.q[0, 0].float().mean(0)).to(inp.k.dtype)
    to_dev(inp)
    budgets = [1, 2, 4, 8, 16]
    _, res = run(inp, budgets, 4)
    lv = res["sel_levels"][0, 0].cpu().numpy()
    assert lv[0] == 5
    assert list(res["sel"][0, 0].cpu().numpy()) == list(range(80, 96))


def test_repeat_calls_are_bitwise_identical():
    say("[determinism]")
    inp = to_dev(make_layer(2, 0))
    cfg = inp.cfg
    pyr = wf.build_pyramid(inp.k, cfg.n_prompt, cfg.levels)
    outs = [wf.select_attend(inp.q, pyr, inp.k, inp.v, inp.gen_idx, cfg.budgets, levels_out=True) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        for key in ("out", "sel", "sel_levels", "score_levels"):
            assert torch.equal(o[key], outs[0][key]), key


def test_one_workspace_serves_different_shapes():
    """Calls of different head counts share one workspace (the counters keep
    one fixed place, so a 1-head call cannot leave data where a 32-head call
    keeps its counters)."""
    say("[workspace reuse]")
    ws = wf.Workspace(DEV)
    one = to_dev(make_layer(dataclasses.replace(CONFIGS[2], cid=99, heads=1, n_prompt=1024, n_gen=8), 0))
    p1 = wf.build_pyramid(one.k, 1024, 4)
    r1 = wf.select_attend(one.q, p1, one.k, one.v, one.gen_idx, [4, 8, 16, 32, 64], workspace=ws)
    a = to_dev(make_layer(1, 0))
    b = to_dev(make_layer(2, 0))
    pa = wf.build_pyramid(a.k, a.cfg.n_prompt, a.cfg.levels)
    pb = wf.build_pyramid(b.k, b.cfg.n_prompt, b.cfg.levels)
    ra1 = wf.select_attend(a.q, pa, a.k, a.v, a.gen_idx, a.cfg.budgets, workspace=ws)
    rb = wf.select_attend(b.q, pb, b.k, b.v, b.gen_idx, b.cfg.budgets, workspace=ws)
    ra2 = wf.select_attend(a.q, pa, a.k, a.v, a.gen_idx, a.cfg.budgets, workspace=ws)
    rb2 = wf.select_attend(b.q, pb, b.k, b.v, b.gen_idx, b.cfg.budgets)
    r1b = wf.select_attend(one.q, p1, one.k, one.v, one.gen_idx, [4, 8, 16, 32, 64], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(r1["out"], r1b["out"])
    assert torch.equal(ra1["out"], ra2["out"]) and torch.equal(ra1["sel"], ra2["sel"])
    assert torch.equal(rb["out"], rb2["out"])


def oracle_attend_selected_head(q, inp, sel_bh, gen, b, h):
    from oracle import attend_selected
    return attend_selected(to_f64(q[b, h]), to_f64(inp.k[b, h]), to_f64(inp.v[b, h]), sel_bh, gen)


@pytest.mark.parametrize("cid", [1, 2])
def test_attend_selected_reuses_a_selection(cid):
    """Attention over a selection made by an earlier call: with the same
    queries it reproduces that call's output up to float32 rounding (the
    selecting call may split the attention differently, its generated
    positions' splits running beside the refinement); with the queries of a
    later step it matches the oracle's attention over the same rows."""
    say(f"[attend_selected c{cid}]")
    inp = to_dev(make_layer(cid, 0))
    cfg = inp.cfg
    _, res = run(inp)
    again = wf.attend_selected(inp.q, inp.k, inp.v, res["sel"], inp.gen_idx)
    torch.cuda.synchronize()
    assert torch.allclose(again, res["out"], rtol=1e-5, atol=1e-6), (again - res["out"]).abs().max().item()
    q2 = make_layer(cid, 1).q.to(DEV)          # the queries of another step, same shape
    out2 = wf.attend_selected(q2, inp.k, inp.v, res["sel"], inp.gen_idx)
    torch.cuda.synchronize()
    gen = inp.gen_idx.cpu().numpy().astype(np.int64)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            ref = oracle_attend_selected_head(q2, inp, res["sel"][b, h].cpu().numpy(), gen, b, h)
            err = np.abs(out2[b, h].cpu().numpy() - ref).max()
            assert err <= TOL[cfg.dtype], (b, h, err)


ATTEND_EDGE = [
    # name, config, k0 (kept prompt rows per head), generated rows
    ("gen-only", custom(2, cid=80, heads=2, n_prompt=1024, n_gen=40), 0, 40),
    ("prompt-only", custom(2, cid=81, heads=3, n_prompt=2048, n_gen=8), 300, 0),
    ("ragged-b2-nq20", custom(2, cid=82, batch=2, heads=3, n_q=20, n_prompt=4096, n_gen=7), 777, 7),
    ("f32-d64-nq64", custom(1, cid=83, head_dim=64, heads=2, n_q=64, n_prompt=2048, n_gen=16), 513, 16),
    ("one-row", custom(2, cid=84, heads=1, n_q=1, n_prompt=256, n_gen=0), 1, 0),
    ("many-splits", custom(2, cid=85, heads=1, n_q=16, n_prompt=32768, n_gen=64), 9000, 64),
]


@pytest.mark.parametrize("name,cfg,k0,n_gen", ATTEND_EDGE, ids=[e[0] for e in ATTEND_EDGE])
def test_attend_selected_edge_cases(name, cfg, k0, n_gen):
    say(f"[attend_selected edge {name}]")
    inp = make_layer(cfg, 0)
    gsel = torch.Generator().manual_seed(cfg.cid)
    # any rows, in any order, repeats allowed: a random draw over the prompt
    sel = torch.randint(0, cfg.n_prompt, (cfg.batch, cfg.heads, k0), generator=gsel, dtype=torch.int32)
    gen = inp.gen_idx[:n_gen]
    to_dev(inp)
    sel_d = sel.to(DEV) if k0 else None
    gen_d = gen.to(DEV) if n_gen else None
    out = wf.attend_selected(inp.q, inp.k, inp.v, sel_d, gen_d)
    torch.cuda.synchronize()
    g = gen.numpy().astype(np.int64)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            ref = oracle_attend_selected_head(inp.q, inp, sel[b, h].numpy(), g, b, h)
            err = np.abs(out[b, h].cpu().numpy() - ref).max()
            assert err <= TOL[cfg.dtype], (b, h, err)


@pytest.mark.parametrize("spike", [False, True], ids=["flat", "crowded"])
def test_tied_levels_match_the_oracle_exactly(spike):
    """Prompt keys that are all one row give every candidate of a level the
    same score (no score range to bin); with a block of rows three times
    larger on top, most candidates of a level tie inside one bin, more than
    the in-bin ranking takes at level 0.  Both take the general path where
    needed; ties go to the lower index, at every level."""
    say(f"[tied levels {'crowded' if spike else 'flat'}]")
    from _parity import oracle_head, split_levels_np
    cfg = custom(2, cid=79, heads=2, n_prompt=4096, n_gen=8, levels=4, n_spans=0)
    budgets = [32, 60, 110, 200, 350]
    inp = make_layer(cfg, 0)
    for h in range(cfg.heads):
        row = (0.5 * inp.q[0, h].float().mean(0)).to(inp.k.dtype)
        inp.k[0, h, :cfg.n_prompt] = row
        if spike:
            inp.k[0, h, 1000:1100] = (3.0 * row.float()).to(inp.k.dtype)
    to_dev(inp)
    _, res = run(inp, budgets, 4)
    check_structure(res, budgets, 4, cfg.n_prompt)
    for h in range(cfg.heads):
        out_ora, ora = oracle_head(inp, 0, h, budgets, 4)
        lv = split_levels_np(res["sel_levels"][0, h].cpu().numpy(), budgets)
        for j in range(4, -1, -1):
            np.testing.assert_array_equal(lv[j], ora.sel[j], err_msg=f"level {j} head {h}")
        np.testing.assert_array_equal(res["sel"][0, h].cpu().numpy(), ora.sel[0])
        assert np.abs(res["out"][0, h].cpu().numpy() - out_ora).max() <= TOL["bf16"]


MEAN_CASES = [
    ("1k-f32", CONFIGS[1], None, None),
    ("4k-bf16", CONFIGS[2], None, None),
    ("ragged-nq20-b2", custom(2, cid=78, batch=2, heads=2, n_q=20, n_prompt=2048, n_gen=7, levels=4),
     [5, 9, 17, 30, 50], 4),
    ("bf16-d64-nq48", custom(2, cid=77, head_dim=64, heads=3, n_q=48, n_prompt=4096, n_gen=40, levels=5),
     [6, 11, 20, 36, 64, 100], 5),
]


@pytest.mark.parametrize("name,cfg,budgets,levels", MEAN_CASES, ids=[c[0] for c in MEAN_CASES])
def test_mean_aggregation_matches_oracle(name, cfg, budgets, levels):
    """The region scores average the query rows (WF_AGG_MEAN); rows past
    n_q in the last query tile must count as absent, not as zero scores."""
    say(f"[mean {name}]")
    inp = make_layer(cfg, 0)
    budgets = cfg.budgets if budgets is None else budgets
    levels = cfg.levels if levels is None else levels
    heads = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    assert all(plant(inp, heads, budgets, levels, agg="mean").values())
    to_dev(inp)
    pyr = wf.build_pyramid(inp.k, cfg.n_prompt, levels)
    res = wf.select_attend(inp.q, pyr, inp.k, inp.v, inp.gen_idx, budgets, levels_out=True, agg="mean")
    torch.cuda.synchronize()
    check_structure(res, budgets, levels, cfg.n_prompt)
    for b, h in heads:
        assert check_head(inp, res, b, h, budgets, levels, agg="mean") == 0


SOFT_CASES = [
    ("4k-bf16", CONFIGS[2], None, None),
    ("ragged-nq20-b2", custom(2, cid=78, batch=2, heads=2, n_q=20, n_prompt=2048, n_gen=7, levels=4),
     [5, 9, 17, 30, 50], 4),
    ("1k-f32", CONFIGS[1], None, None),
    ("dense-L0", custom(2, cid=75, heads=2, n_prompt=512, n_gen=8, levels=0, n_spans=0), [100], 0),
]


@pytest.mark.parametrize("agg", ["softmax_max", "softmax_mean"])
@pytest.mark.parametrize("name,cfg,budgets,levels", SOFT_CASES, ids=[c[0] for c in SOFT_CASES])
def test_softmax_aggregations_match_oracle(agg, name, cfg, budgets, levels):
    """Region scores from attention probabilities: every query row's logits
    normalised by a softmax over the level's candidates, then the maximum or
    the mean over the rows.  Planted heads match the oracle exactly at every
    level, with the kept regions' probabilities to float32 accuracy."""
    say(f"[{agg} {name}]")
    inp = make_layer(cfg, 0)
    budgets = cfg.budgets if budgets is None else budgets
    levels = cfg.levels if levels is None else levels
    heads = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    assert all(plant_many(inp, heads, budgets, levels, agg=agg))
    to_dev(inp)
    pyr = wf.build_pyramid(inp.k, cfg.n_prompt, levels)
    res = wf.select_attend(inp.q, pyr, inp.k, inp.v, inp.gen_idx, budgets, levels_out=True, agg=agg)
    torch.cuda.synchronize()
    check_structure(res, budgets, levels, cfg.n_prompt)
    ora = oracle_many(inp, heads, budgets, levels, agg=agg)
    for (b, h), o in zip(heads, ora):
        assert check_head(inp, res, b, h, budgets, levels, agg=agg, ora=o) == 0, (b, h)


def test_one_query_row_softmax_max_selects_what_max_selects():
    """With one query row a level's softmax is monotone in the row's logits,
    so the softmax maximum keeps exactly the regions the logit maximum keeps
    (margins planted for the logits)."""
    say("[softmax n_q=1]")
    cfg = custom(2, cid=74, heads=4, n_q=1, n_prompt=2048, n_gen=8, levels=4)
    inp = make_layer(cfg, 0)
    budgets = [8, 15, 28, 50, 90]
    heads = [(0, h) for h in range(cfg.heads)]
    assert all(plant_many(inp, heads, budgets, 4, agg="max"))
    to_dev(inp)
    pyr = wf.build_pyramid(inp.k, cfg.n_prompt, 4)
    hard = wf.select_attend(inp.q, pyr, inp.k, inp.v, inp.gen_idx, budgets, levels_out=True, agg="max")
    soft = wf.select_attend(inp.q, pyr, inp.k, inp.v, inp.gen_idx, budgets, levels_out=True, agg="softmax_max")
    torch.cuda.synchronize()
    assert torch.equal(hard["sel_levels"], soft["sel_levels"])
    assert torch.equal(hard["out"].view(torch.int32), soft["out"].view(torch.int32))


def test_one_query_row_mean_equals_max():
    say("[mean n_q=1]")
    cfg = custom(2, cid=76, heads=2, n_q=1, n_prompt=2048, n_gen=8, levels=4)
    inp = to_dev(make_layer(cfg, 0))
    budgets = [8, 15, 28, 50, 90]
    pyr = wf.build_pyramid(inp.k, cfg.n_prompt, 4)
    a = wf.select_attend(inp.q, pyr, inp.k, inp.v, inp.gen_idx, budgets, levels_out=True, agg="max")
    m = wf.select_attend(inp.q, pyr, inp.k, inp.v, inp.gen_idx, budgets, levels_out=True, agg="mean")
    torch.cuda.synchronize()
    assert torch.equal(a["sel_levels"], m["sel_levels"])
    assert torch.equal(a["out"], m["out"])


def _modify_blocks(k, n_prompt, L, blocks, gen):
    """Change the prompt keys of the given level-L blocks (some rows of each)."""
    rows = 1 << L
    for b in blocks:
        r0 = b * rows + int(torch.randint(0, rows, (1,), generator=gen))
        r1 = min((b + 1) * rows, r0 + max(1, rows // 2))
        k[:, :, r0:r1] = (k[:, :, r0:r1].float() * 1.5 + 0.25).to(k.dtype)


REFRESH_CASES = [
    ("1k-f32-L3", custom(1, cid=70), 3),
    ("4k-bf16-L4", custom(2, cid=71, heads=4), 4),
    ("bf16-d64-L6", custom(2, cid=72, head_dim=64, heads=3, n_prompt=8192, levels=6), 6),
    ("bf16-L0", custom(2, cid=73, heads=2, n_prompt=512, levels=0), 0),
    ("bf16-L1", custom(2, cid=74, heads=2, n_prompt=1024, levels=1), 1),
    # blocks of more than 16 passes of one wave-wide load (summed in groups of 16 loads)
    ("bf16-L7", custom(2, cid=75, heads=2, n_prompt=16384, levels=7), 7),
    ("f32-d128-L7", custom(2, cid=76, dtype="f32", heads=2, n_prompt=8192, levels=7), 7),
]


@pytest.mark.parametrize("name,cfg,L", REFRESH_CASES, ids=[c[0] for c in REFRESH_CASES])
def test_refresh_equals_a_rebuild(name, cfg, L):
    """Listed blocks after a refresh are bit for bit what a full rebuild on the
    changed keys writes (and match the oracle); unlisted blocks keep their old
    rows, even those whose keys changed."""
    say(f"[refresh {name}]")
    inp = to_dev(make_layer(cfg, 0))
    n_top = cfg.n_prompt >> L
    old = wf.build_pyramid(inp.k, cfg.n_prompt, L)
    torch.cuda.synchronize()
    a_old = old.top.clone()
    gen = torch.Generator().manual_seed(cfg.cid)
    perm = torch.randperm(n_top, generator=gen)
    listed = sorted(perm[: max(1, n_top // 8)].tolist())
    stale = sorted(perm[n_top // 8: n_top // 8 + max(1, n_top // 16)].tolist())  # changed but not listed
    _modify_blocks(inp.k, cfg.n_prompt, L, listed + stale, gen)
    blocks = torch.tensor(listed + [listed[0]], dtype=torch.int32, device=DEV)  # a repeat is harmless
    wf.refresh_pyramids([(inp.k, old, blocks)])
    full = wf.build_pyramid(inp.k, cfg.n_prompt, L)
    torch.cuda.synchronize()
    got, ref = old.top, full.top
    lst = torch.tensor(listed, device=DEV)
    keep = torch.ones(n_top, dtype=torch.bool, device=DEV)
    keep[lst] = False
    assert torch.equal(got[:, :, lst], ref[:, :, lst])
    assert torch.equal(got[:, :, keep], a_old[:, :, keep])
    from oracle import refresh_top
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            want = refresh_top(a_old[b, h].cpu().numpy(), to_f64(inp.k[b, h, :cfg.n_prompt]), listed, L)
            err = np.abs(got[b, h].cpu().numpy() - want)[listed].max()
            assert err <= 1e-5 * (1 + np.abs(want).max()), (b, h, err)


def test_refresh_batched_over_layers():
    """One call refreshes three pyramids of different shapes; an entry past
    the last block is skipped."""
    say("[refresh batch]")
    cfgs = [custom(2, cid=60, heads=2, n_prompt=2048, levels=4), custom(2, cid=61, heads=3, n_prompt=4096, levels=5),
            custom(2, cid=62, heads=1, n_prompt=1024, levels=2)]
    layers, items, olds = [], [], []
    gen = torch.Generator().manual_seed(5)
    for cfg in cfgs:
        inp = to_dev(make_layer(cfg, 0))
        pyr = wf.build_pyramid(inp.k, cfg.n_prompt, cfg.levels)
        torch.cuda.synchronize()
        olds.append(pyr.top.clone())
        n_top = cfg.n_prompt >> cfg.levels
        listed = sorted(torch.randperm(n_top, generator=gen)[: n_top // 4].tolist())
        _modify_blocks(inp.k, cfg.n_prompt, cfg.levels, listed, gen)
        blocks = torch.tensor(listed + [n_top + 3], dtype=torch.int32, device=DEV)
        layers.append((inp, cfg, listed))
        items.append((inp.k, pyr, blocks))
    wf.refresh_pyramids(items)
    torch.cuda.synchronize()
    for (inp, cfg, listed), (_, pyr, _), a_old in zip(layers, items, olds):
        full = wf.build_pyramid(inp.k, cfg.n_prompt, cfg.levels)
        torch.cuda.synchronize()
        lst = torch.tensor(listed, device=DEV)
        keep = torch.ones(cfg.n_prompt >> cfg.levels, dtype=torch.bool, device=DEV)
        keep[lst] = False
        assert torch.equal(pyr.top[:, :, lst], full.top[:, :, lst])
        assert torch.equal(pyr.top[:, :, keep], a_old[:, :, keep])


def test_db2_pyramid_matches_oracle():
    """Every band of the Daubechies four-tap pyramid (periodic extension)."""
    say("[db2 pyramid]")
    from oracle import dwt_pyramid
    for cfg in (custom(1, cid=50), custom(2, cid=51, heads=3, n_prompt=2048, levels=5)):
        inp = to_dev(make_layer(cfg, 0))
        pyr = wf.build_pyramid(inp.k, cfg.n_prompt, cfg.levels, wf.WF_PYR_DB2)
        torch.cuda.synchronize()
        for h in range(cfg.heads):
            approx, detail = dwt_pyramid(to_f64(inp.k[0, h, :cfg.n_prompt]), cfg.levels, "db2")
            for j in range(1, cfg.levels + 1):
                for band, ref in ((0, approx[j]), (1, detail[j])):
                    got = pyr.band(band, j)[0, h].cpu().numpy()
                    assert np.abs(got - ref).max() <= 1e-5 * (1 + np.abs(ref).max()), (band, j)


DB2_CASES = [
    ("1k-f32", custom(1, cid=52), "max"),
    ("4k-bf16-4h", custom(2, cid=53, heads=4), "max"),
    ("bf16-d64-nq20-mean", custom(2, cid=54, head_dim=64, heads=3, n_q=20, n_prompt=2048, n_gen=12, levels=4), "mean"),
]


@pytest.mark.parametrize("name,cfg,agg", DB2_CASES, ids=[c[0] for c in DB2_CASES])
def test_db2_select_attend_matches_oracle(name, cfg, agg):
    """Selection on the Daubechies pyramid: the finer levels are scored from
    the stored bands, the refinement tree is the dyadic one."""
    say(f"[db2 select {name}]")
    inp = make_layer(cfg, 0)
    heads = [(0, h) for h in range(cfg.heads)]
    assert all(plant(inp, heads, agg=agg, wavelet="db2").values())
    to_dev(inp)
    pyr = wf.build_pyramid(inp.k, cfg.n_prompt, cfg.levels, wf.WF_PYR_DB2)
    res = wf.select_attend(inp.q, pyr, inp.k, inp.v, inp.gen_idx, cfg.budgets, levels_out=True, agg=agg)
    torch.cuda.synchronize()
    check_structure(res, cfg.budgets, cfg.levels, cfg.n_prompt)
    for b, h in heads:
        assert check_head(inp, res, b, h, agg=agg, wavelet="db2") == 0
