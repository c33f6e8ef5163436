"""Helpers of the GPU parity tests: margin planting, oracle runs and checks."""

import math
import sys

import numpy as np
import torch

from oracle import attend, select_attend as oracle_select_attend
from oracle.planting import plant_margins
from workloads.gen import to_f64

PIN_GAP = 1e-3          # a level is compared bit for bit when the oracle's gap exceeds this
TOL = {"bf16": 2e-3, "f32": 1e-5}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def plant(inp, heads, budgets=None, levels=None, agg="max", wavelet="haar"):
    """Plant margins on the listed (b, h) heads, editing ``inp.k`` in place
    (scales by powers of two are exact in the stored dtype)."""
    cfg = inp.cfg
    budgets = cfg.budgets if budgets is None else budgets
    levels = cfg.levels if levels is None else levels
    ok = {}
    for b, h in heads:
        q = to_f64(inp.q[b, h])
        kp = to_f64(inp.k[b, h, :cfg.n_prompt])
        _, ops, conv = plant_margins(q, kp, budgets, levels, agg=agg, wavelet=wavelet)
        for r0, r1, f in ops:
            inp.k[b, h, r0:r1] *= f
        ok[(b, h)] = conv
    return ok


def oracle_head(inp, b, h, budgets=None, levels=None, agg="max", wavelet="haar"):
    cfg = inp.cfg
    budgets = cfg.budgets if budgets is None else budgets
    levels = cfg.levels if levels is None else levels
    q = to_f64(inp.q[b, h])
    k = to_f64(inp.k[b, h])
    v = to_f64(inp.v[b, h])
    gen = inp.gen_idx.cpu().numpy().astype(np.int64) if inp.gen_idx is not None else np.zeros(0, np.int64)
    return oracle_select_attend(q, k, v, cfg.n_prompt, gen, budgets, levels, agg, wavelet)


def split_levels_np(flat, budgets):
    L = len(budgets) - 1
    out, off = {}, 0
    for i, kb in enumerate(budgets):
        out[L - i] = flat[off:off + kb]
        off += kb
    return out


def check_head(inp, gpu, b, h, budgets=None, levels=None, tol=None, agg="max", wavelet="haar"):
    """Compare one head with the oracle under the margin rule.  Returns the
    number of unpinned levels (0 when every level was compared exactly)."""
    cfg = inp.cfg
    budgets = cfg.budgets if budgets is None else budgets
    levels = cfg.levels if levels is None else levels
    tol = TOL[cfg.dtype] if tol is None else tol
    out_ora, res = oracle_head(inp, b, h, budgets, levels, agg, wavelet)
    lv = split_levels_np(gpu["sel_levels"][b, h].cpu().numpy(), budgets)
    sc = split_levels_np(gpu["score_levels"][b, h].cpu().numpy(), budgets)
    pinned = True
    unpinned = 0
    for j in range(levels, -1, -1):
        if pinned and res.gap[j] > PIN_GAP:
            np.testing.assert_array_equal(lv[j], res.sel[j], err_msg=f"level {j} head {(b, h)}")
            # scores of the kept regions agree to float32 accuracy
            s_ora = res.scores[j][np.searchsorted(res.cand[j], res.sel[j])]
            err = np.abs(sc[j] - s_ora).max()
            assert err <= 1e-4 * (1 + np.abs(s_ora).max()), (j, err)
        else:
            pinned = False
            unpinned += 1
    o_gpu = gpu["out"][b, h].cpu().numpy().astype(np.float64)
    if unpinned == 0:
        err = np.abs(o_gpu - out_ora).max()
    else:
        # several selections are correct: attend over the device's own set
        rows = np.concatenate([lv[0].astype(np.int64), inp.gen_idx.cpu().numpy().astype(np.int64)])
        ref = attend(to_f64(inp.q[b, h]), to_f64(inp.k[b, h])[rows], to_f64(inp.v[b, h])[rows])
        err = np.abs(o_gpu - ref).max()
    assert err <= tol, f"head {(b, h)} max|dO| = {err:.3g} > {tol}"
    np.testing.assert_array_equal(gpu["sel"][b, h].cpu().numpy(), lv[0])
    return unpinned


def check_structure(gpu, budgets, levels, n_prompt):
    """Properties of a valid hierarchical selection, for every head."""
    sl = gpu["sel_levels"].cpu().numpy()
    B, H = sl.shape[:2]
    for b in range(B):
        for h in range(H):
            lv = split_levels_np(sl[b, h], budgets)
            for j in range(levels, -1, -1):
                s = lv[j]
                assert len(s) == budgets[levels - j]
                assert np.all(np.diff(s) > 0), (b, h, j)
                assert s[0] >= 0 and s[-1] < (n_prompt >> j)
                if j < levels:
                    assert np.all(np.isin(s >> 1, lv[j + 1])), (b, h, j)
            np.testing.assert_array_equal(gpu["sel"][b, h].cpu().numpy(), lv[0])


def torch_attend_all(inp, gpu):
    """Float32 torch attention over each head's device-selected set (a plain
    reference of the same op, for heads the float64 oracle does not visit)."""
    cfg = inp.cfg
    B, H, n_q, d = inp.q.shape
    sel = gpu["sel"].long()
    gen = inp.gen_idx.long()
    worst = 0.0
    for b in range(B):
        for h in range(H):
            rows = torch.cat([sel[b, h], gen])
            kk = inp.k[b, h].index_select(0, rows).float().contiguous()
            vv = inp.v[b, h].index_select(0, rows).float().contiguous()
            qq = inp.q[b, h].float()
            w = torch.softmax((qq @ kk.t().contiguous()) / math.sqrt(d), dim=-1)
            ref = w @ vv
            worst = max(worst, float((gpu["out"][b, h] - ref).abs().max()))
    return worst
