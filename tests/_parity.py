"""Helpers of the GPU parity tests: margin planting, oracle runs and checks."""

import math
import sys

import numpy as np
import torch

from oracle import attend, select_attend as oracle_select_attend
from oracle.planting import plant_margins
from workloads.gen import to_f64

import _pool

PIN_GAP = 1e-3          # a level is compared bit for bit when the oracle's gap exceeds this
TOL = {"bf16": 2e-3, "f32": 1e-5}


# pytest's capture manager (set by conftest): progress lines of the long GPU
# tests then reach the terminal or log as they happen, not when the test ends
_capman = None


def say(*a):
    if _capman is not None:
        with _capman.global_and_fixture_disabled():
            print(*a, flush=True)
    else:
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


def bits(t):
    """Raw stored values of a (device) tensor as numpy: bfloat16 as uint16 bits."""
    t = t.detach().contiguous().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _gen_np(inp):
    return inp.gen_idx.cpu().numpy().astype(np.int64) if inp.gen_idx is not None else np.zeros(0, np.int64)


def _items(inp, heads):
    """[(layer inputs, (b, h))] from one layer and its heads, or a list of such pairs."""
    return [(inp, bh) for bh in heads] if heads is not None else list(inp)


def plant_many(inp, heads=None, budgets=None, levels=None, agg="max", wavelet="haar", max_iter=64):
    """``plant`` for many heads at once (of one layer: ``inp, heads``; or of
    several: ``inp`` a list of ``(layer inputs, (b, h))``), the oracle work
    in a process pool; the edits (exact power-of-two scales) are applied to
    each layer's ``k`` wherever it lives.  ``max_iter`` bounds the planting
    passes per head (128K-token heads of eight levels can need about 90).
    Returns a list of converged flags."""
    items = _items(inp, heads)
    jobs = []
    for i, (x, (b, h)) in enumerate(items):
        cfg = x.cfg
        jobs.append((i, cfg.dtype, bits(x.q[b, h]), bits(x.k[b, h, :cfg.n_prompt]),
                     list(cfg.budgets if budgets is None else budgets), cfg.levels if levels is None else levels,
                     agg, wavelet, max_iter))
    ok = [False] * len(items)
    for i, ops, conv in _pool.run(_pool.plant_job, jobs):
        x, (b, h) = items[i]
        for r0, r1, f in ops:
            x.k[b, h, r0:r1] *= f
        ok[i] = conv
    return ok


class OracleHead:
    """The oracle's result for one head, without the stored bands."""

    def __init__(self, out, sel, cand, scores, gap):
        self.out, self.sel, self.cand, self.scores, self.gap = out, sel, cand, scores, gap


def oracle_many(inp, heads=None, budgets=None, levels=None, agg="max", wavelet="haar"):
    """The oracle on many heads in a process pool (arguments as for
    ``plant_many``): a list of ``OracleHead``, in item order."""
    items = _items(inp, heads)
    jobs = []
    for i, (x, (b, h)) in enumerate(items):
        cfg = x.cfg
        jobs.append((i, cfg.dtype, bits(x.q[b, h]), bits(x.k[b, h]), bits(x.v[b, h]), cfg.n_prompt, _gen_np(x),
                     list(cfg.budgets if budgets is None else budgets), cfg.levels if levels is None else levels,
                     agg, wavelet))
    res = [None] * len(items)
    for i, out, sel, cand, scores, gap in _pool.run(_pool.oracle_job, jobs):
        res[i] = OracleHead(out, sel, cand, scores, gap)
    return res


def check_validity_many(inp, heads=None, budgets=None, levels=None, tol=None, agg="max", wavelet="haar",
                        band=PIN_GAP):
    """For heads whose margins were not planted: every device level set must
    be a valid Top-K of the children of the device's own parent set under
    the oracle's float64 scores (a dropped candidate may beat a kept one by
    at most ``band``, relative), and O must match the oracle's attention over
    the device's own final set.  ``inp`` is a list of ``(layer inputs,
    device result, (b, h))`` (or one layer's inputs, with ``heads`` a pair
    (device result, heads)).  Returns the smallest relative margin seen."""
    if heads is not None:
        gpu, hs = heads
        items = [(inp, gpu, bh) for bh in hs]
    else:
        items = list(inp)
    jobs = []
    for i, (x, gpu, (b, h)) in enumerate(items):
        cfg = x.cfg
        bud = list(cfg.budgets if budgets is None else budgets)
        lv = split_levels_np(gpu["sel_levels"][b, h].cpu().numpy(), bud)
        jobs.append((i, cfg.dtype, bits(x.q[b, h]), bits(x.k[b, h]), bits(x.v[b, h]), cfg.n_prompt, _gen_np(x), bud,
                     cfg.levels if levels is None else levels, agg, wavelet, lv, band))
    worst = np.inf
    for i, err, res in _pool.run(_pool.validity_job, jobs):
        x, gpu, (b, h) = items[i]
        assert err is None, f"head {(b, h)} of layer {x.layer}: {err}"
        out_ref, margin = res
        worst = min(worst, margin)
        t = TOL[x.cfg.dtype] if tol is None else tol
        d = np.abs(gpu["out"][b, h].cpu().numpy().astype(np.float64) - out_ref).max()
        assert d <= t, f"head {(b, h)} of layer {x.layer}: max|dO| = {d:.3g} > {t}"
        bud = list(x.cfg.budgets if budgets is None else budgets)
        np.testing.assert_array_equal(gpu["sel"][b, h].cpu().numpy(),
                                      gpu["sel_levels"][b, h].cpu().numpy()[-bud[-1]:])
    return worst


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


def check_head(inp, gpu, b, h, budgets=None, levels=None, tol=None, agg="max", wavelet="haar", ora=None):
    """Compare one head with the oracle under the margin rule.  Returns the
    number of unpinned levels (0 when every level was compared exactly).
    ``ora`` is the head's precomputed ``OracleHead``, if any."""
    cfg = inp.cfg
    budgets = cfg.budgets if budgets is None else budgets
    levels = cfg.levels if levels is None else levels
    tol = TOL[cfg.dtype] if tol is None else tol
    if ora is None:
        out_ora, res = oracle_head(inp, b, h, budgets, levels, agg, wavelet)
    else:
        out_ora, res = ora.out, ora
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
