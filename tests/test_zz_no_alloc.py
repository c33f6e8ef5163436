"""wf_select_attend_noalloc against wf_select_attend: the same kernels with
the workspace taken from the library's static per-device scratch array.
Outputs must agree bit for bit, also on a call that follows a larger one in
the same scratch (its stale contents must not matter)."""

import pytest
import torch

import long_context_kv_haar_amd as wf
from workloads.configs import CONFIGS
from workloads.gen import make_layer

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _pair(cfg, agg, layer=0):
    """One select-attend case through both entry points, compared bitwise."""
    print(f"[no-alloc {cfg.name} agg={agg}]", flush=True)
    inp = make_layer(cfg, layer, device=DEV)
    pyr = wf.build_pyramid(inp.k, cfg.n_prompt, cfg.levels)
    B, H, n_q, d = inp.q.shape
    nk = sum(cfg.budgets)
    want = wf.select_attend(inp.q, pyr, inp.k, inp.v, inp.gen_idx, cfg.budgets, levels_out=True, agg=agg)
    # outputs pre-filled with garbage: every element must be written
    out = torch.full((B, H, n_q, d), float("nan"), device=DEV)
    sel = torch.full((B, H, cfg.budgets[-1]), -7, dtype=torch.int32, device=DEV)
    sel_lv = torch.full((B, H, nk), -7, dtype=torch.int32, device=DEV)
    score_lv = torch.full((B, H, nk), float("nan"), device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(DEV)
    wf.select_attend_noalloc(inp.q, pyr, inp.k, inp.v, inp.gen_idx, cfg.budgets, out, sel, sel_lv, score_lv, agg=agg)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated(DEV) == before
    assert torch.equal(sel, want["sel"])
    assert torch.equal(sel_lv, want["sel_levels"])
    assert torch.equal(score_lv.view(torch.int32), want["score_levels"].view(torch.int32))
    assert torch.equal(out.view(torch.int32), want["out"].view(torch.int32))
    return out


def test_noalloc_matches_the_workspace_call_on_consecutive_calls():
    # the largest workspace first (a 128K layer, two sequences: 13.8 MiB), then smaller calls
    _pair(CONFIGS[5], "max")
    _pair(CONFIGS[2], "mean")
    _pair(CONFIGS[1], "max")


def test_noalloc_rejects_a_call_beyond_its_scratch():
    cfg = CONFIGS[1]
    print("[no-alloc oversize]", flush=True)
    # 2 048 heads of a 1K prompt: the split partials alone need more than 16 MiB
    k = torch.zeros((1, 2048, 1056, 64), dtype=torch.float32, device=DEV)
    q = torch.zeros((1, 2048, 32, 64), dtype=torch.float32, device=DEV)
    gen = torch.arange(1024, 1056, dtype=torch.int32, device=DEV)
    pyr = wf.build_pyramid(k, 1024, 3)
    budgets = [8, 16, 32, 64]
    assert wf.workspace_bytes(pyr, 32, 32, budgets) > 16 << 20
    out = torch.full((1, 2048, 32, 64), 5.0, device=DEV)
    with pytest.raises(wf.WfError) as err:
        wf.select_attend_noalloc(q, pyr, k, k, gen, budgets, out)
    assert err.value.status == -6  # WF_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())
