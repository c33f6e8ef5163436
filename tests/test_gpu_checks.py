"""Debug checks (WF_OPT_CHECK) on the GPU: bad indices and non-finite inputs
come back in the workspace's status word, the calls complete (indices are
clamped into their buffers), and clean inputs report nothing and compute
the same bits as an unchecked call."""

import pytest
import torch

import long_context_kv_haar_amd as wf
from workloads.configs import CONFIGS
from workloads.gen import make_layer

from _parity import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def layer(cid=2, seed=0):
    inp = make_layer(cid, seed, device=DEV)
    pyr = wf.build_pyramid(inp.k, inp.cfg.n_prompt, inp.cfg.levels)
    return inp, pyr


def run(inp, pyr, ws, check=True, **kw):
    cfg = inp.cfg
    res = wf.select_attend(inp.q, pyr, inp.k, inp.v, inp.gen_idx, cfg.budgets, workspace=ws, check=check, **kw)
    torch.cuda.synchronize()
    return res


def test_clean_inputs_report_nothing_and_match_the_unchecked_call():
    say("[checks clean]")
    inp, pyr = layer()
    ws = wf.Workspace(torch.device(DEV))
    plain = run(inp, pyr, ws, check=False)
    checked = run(inp, pyr, ws)
    assert wf.check_status(ws) == set()
    assert torch.equal(plain["sel"], checked["sel"])
    assert torch.equal(plain["out"].view(torch.int32), checked["out"].view(torch.int32))


def test_out_of_range_generated_index_is_reported_and_clamped():
    say("[checks gen index]")
    inp, pyr = layer()
    ws = wf.Workspace(torch.device(DEV))
    n_tot = inp.k.shape[2]
    inp.gen_idx[3] = n_tot + 5
    res = run(inp, pyr, ws)
    assert wf.check_status(ws) == {"gen_index"}
    assert bool(torch.isfinite(res["out"]).all())  # the row was clamped into the buffer
    inp.gen_idx[3] = -1
    run(inp, pyr, ws)
    assert wf.check_status(ws) == {"gen_index"}
    # the next call with clean inputs clears the word
    inp.gen_idx[3] = inp.cfg.n_prompt + 3
    run(inp, pyr, ws)
    assert wf.check_status(ws) == set()


def test_non_finite_values_are_reported_per_tensor():
    say("[checks non-finite]")
    inp, pyr = layer()
    ws = wf.Workspace(torch.device(DEV))
    cfg = inp.cfg
    inp.v[0, 5, 17, 3] = float("inf")
    run(inp, pyr, ws)
    assert wf.check_status(ws) == {"nonfinite_v"}
    inp.v[0, 5, 17, 3] = 0.0
    inp.k[0, 2, cfg.n_prompt + 1, 0] = float("nan")  # a generated row: attended, never scored
    run(inp, pyr, ws)
    assert wf.check_status(ws) == {"nonfinite_k"}
    inp.k[0, 2, cfg.n_prompt + 1, 0] = 0.0
    # a prompt key: the pyramid built from it carries the NaN too
    inp.k[0, 9, 100, 7] = float("nan")
    pyr_nan = wf.build_pyramid(inp.k, cfg.n_prompt, cfg.levels)
    run(inp, pyr_nan, ws)
    assert wf.check_status(ws) == {"nonfinite_k", "nonfinite_pyramid"}


def test_attend_selected_reports_bad_selection_and_query():
    say("[checks attend_selected]")
    inp, pyr = layer()
    cfg = inp.cfg
    ws = wf.Workspace(torch.device(DEV))
    sel = run(inp, pyr, ws, check=False)["sel"].clone()
    out_clean = wf.attend_selected(inp.q, inp.k, inp.v, sel, inp.gen_idx, workspace=ws, check=True)
    torch.cuda.synchronize()
    assert wf.check_status(ws) == set()
    sel[0, 4, 10] = inp.k.shape[2]
    out = wf.attend_selected(inp.q, inp.k, inp.v, sel, inp.gen_idx, workspace=ws, check=True)
    torch.cuda.synchronize()
    assert wf.check_status(ws) == {"sel_index"}
    assert bool(torch.isfinite(out).all())
    assert torch.equal(out[:, :4], out_clean[:, :4])  # other heads untouched
    sel[0, 4, 10] = 0
    q = inp.q.clone()
    q[0, 1, 2, 3] = float("nan")
    wf.attend_selected(q, inp.k, inp.v, sel, inp.gen_idx, workspace=ws, check=True)
    torch.cuda.synchronize()
    assert wf.check_status(ws) == {"nonfinite_q"}


def test_checks_in_the_no_alloc_and_batched_calls():
    say("[checks noalloc + layers]")
    inp, pyr = layer()
    cfg = inp.cfg
    inp.gen_idx[0] = -3
    out = torch.empty((cfg.batch, cfg.heads, cfg.n_q, cfg.head_dim), device=DEV)
    wf.select_attend_noalloc(inp.q, pyr, inp.k, inp.v, inp.gen_idx, cfg.budgets, out, check=True)
    torch.cuda.synchronize()
    assert wf.check_status("noalloc") == {"gen_index"}
    inp.gen_idx[0] = cfg.n_prompt
    other, pyr2 = layer(seed=1)
    other.v[0, 0, 0, 0] = float("nan")
    ws = wf.Workspace(torch.device(DEV))
    wf.select_attend_layers([(inp.q, pyr, inp.k, inp.v), (other.q, pyr2, other.k, other.v)], inp.gen_idx,
                            cfg.budgets, workspace=ws, check=True)
    torch.cuda.synchronize()
    assert wf.check_status(ws) == {"nonfinite_v"}
