"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments on the host before touching the GPU (CPU only: no
call below reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

import long_context_kv_haar_amd as wf
from long_context_kv_haar_amd._lib import WfPyramid, lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "wavefilter.h")
FAKE = 0x10000   # a 16-byte-aligned address that is never dereferenced
MISALIGNED = 0x10004


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wf_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 14, names
    L = lib()
    for n in names:
        assert hasattr(L, n), n
    assert wf.version().startswith("wavefilter-gfx950")
    for st in range(-10, 1):
        assert wf.status_string(st) != "unknown status"


def test_pyramid_bytes():
    assert wf.pyramid_bytes(1, 32, 65536, 128, 6) == 32 * 1024 * 128 * 4
    # all levels: A_L + D_1..D_L + A_1..A_{L-1}, each rounded up to 256 bytes
    want = sum(-(-2 * (1024 >> j) * 64 * 4 // 256) * 256 for j in [3, 1, 2, 3, 1, 2])
    assert wf.pyramid_bytes(1, 2, 1024, 64, 3, wf.WF_PYR_ALL_LEVELS) == want
    assert wf.pyramid_bytes(1, 2, 1004, 64, 3) == 0     # N_p not a multiple of 2^L
    assert wf.pyramid_bytes(1, 2, 1024, 96, 3) == 0     # unsupported head dim
    assert wf.pyramid_bytes(1, 2, 1024, 64, 8) == 0     # too many levels
    assert wf.pyramid_bytes(1, 2, 1024, 64, 3, 4) == 0  # unknown flag
    # the Daubechies basis stores every band, like the inspection layout
    assert wf.pyramid_bytes(1, 2, 1024, 64, 3, wf.WF_PYR_DB2) == want


def build(k=FAKE, stride=1024 * 64, B=1, H=2, n=1024, d=64, dt=wf.WF_BF16, L=3, flags=0, mem=FAKE, nbytes=1 << 30,
          out=True):
    desc = WfPyramid()
    return lib().wf_build_pyramid(ctypes.c_void_p(k), stride, B, H, n, d, dt, L, flags, ctypes.c_void_p(mem), nbytes,
                                  ctypes.byref(desc) if out else None, None)


def test_build_pyramid_rejects_bad_arguments():
    assert build(k=0) == -1
    assert build(mem=0) == -1
    assert build(out=False) == -1
    assert build(dt=7) == -3
    assert build(L=8) == -4
    assert build(n=1004) == -4
    assert build(d=96) == -2
    assert build(flags=4) == -10
    assert build(stride=100) == -2
    assert build(k=MISALIGNED) == -7
    assert build(mem=MISALIGNED) == -7
    assert build(stride=1024 * 64 + 1) == -7
    assert build(nbytes=16) == -6


def fake_pyramid(levels=3, n=1024, d=64, H=2, dt=wf.WF_BF16, magic=0x57465059):
    """A descriptor shaped as wf_build_pyramid fills it (the tag is the library's)."""
    return WfPyramid(1, H, n, d, levels, dt, 0, magic, FAKE, 1 << 20)


def budgets_arr(b):
    return (ctypes.c_int32 * len(b))(*b)


def test_workspace_query_and_budget_checks():
    p = fake_pyramid()
    q = lambda *args: lib().wf_select_attend_workspace_bytes(*args, 0)  # noqa: E731
    assert q(ctypes.byref(p), 32, 32, budgets_arr([8, 16, 32, 64])) > 0
    assert q(ctypes.byref(p), 32, 32, budgets_arr([8, 17, 32, 64])) == 0   # k_2 > 2 k_3
    assert q(ctypes.byref(p), 32, 32, budgets_arr([0, 1, 1, 1])) == 0      # k_L < 1
    assert q(ctypes.byref(p), 32, 32, budgets_arr([129, 1, 1, 1])) == 0    # k_L > n_L
    assert q(ctypes.byref(p), 65, 32, budgets_arr([8, 16, 32, 64])) == 0   # n_q > 64
    assert q(ctypes.byref(fake_pyramid(magic=0)), 32, 32, budgets_arr([8, 16, 32, 64])) == 0
    # selection state beyond the on-chip capacity of the refinement
    big = fake_pyramid(levels=2, n=1 << 16)
    assert q(ctypes.byref(big), 32, 0, budgets_arr([16384, 16384, 16384])) == 0


def select(pyr=None, q=FAKE, k=FAKE, v=FAKE, n_tot=1056, gen=FAKE, n_gen=32, b=(8, 16, 32, 64), n_q=32, out=FAKE,
           ws=FAKE, ws_bytes=1 << 30, sel=None, agg=wf.WF_AGG_MAX):
    p = fake_pyramid() if pyr is None else pyr
    return lib().wf_select_attend(ctypes.c_void_p(q), ctypes.byref(p), ctypes.c_void_p(k), ctypes.c_void_p(v),
                                  n_tot, ctypes.c_void_p(gen), n_gen, budgets_arr(list(b)), n_q, agg,
                                  ctypes.c_void_p(out), ctypes.c_void_p(sel), None, None, ctypes.c_void_p(ws),
                                  ws_bytes, None)


def test_select_attend_rejects_bad_arguments():
    assert select(q=0) == -1
    assert select(out=0) == -1
    assert select(ws=0) == -1
    assert select(gen=0) == -1
    assert select(pyr=fake_pyramid(magic=1)) == -9
    assert select(b=(8, 16, 33, 64)) == -5
    assert select(b=(8, 16, 32, 65)) == -5
    assert select(n_q=0) == -2
    assert select(n_tot=1000) == -2
    assert select(q=MISALIGNED) == -7
    assert select(sel=FAKE + 2) == -7
    assert select(ws_bytes=64) == -6
    assert select(agg=4) == -10                                      # not an aggregation
    assert select(agg=-1) == -10
    assert select(agg=0x200) == -10                                  # an undefined option bit
    assert select(agg=wf.WF_AGG_MEAN | 0x200) == -10
    assert select(agg=wf.WF_AGG_MEAN | wf.WF_OPT_CHECK, ws_bytes=64) == -6   # the check bit is accepted


def test_check_bits_match_the_header():
    text = open(HEADER).read()
    assert int(re.search(r"#define WF_OPT_CHECK (0x[0-9a-fA-F]+)", text).group(1), 16) == wf.WF_OPT_CHECK
    for name, bit in wf.CHECK_BITS.items():
        m = re.search(rf"#define WF_CHECK_{name.upper()} (\d+)u", text)
        assert m and int(m.group(1)) == bit, name


def test_workspaces_start_with_the_status_word():
    # the status word takes the first 256 bytes of every workspace
    p = fake_pyramid()
    a = lib().wf_select_attend_workspace_bytes(ctypes.byref(p), 32, 32, budgets_arr([8, 16, 32, 64]), 0)
    b = lib().wf_attend_selected_workspace_bytes(1, 2, 64, wf.WF_BF16, 32, 64, 32)
    assert a > 256 and b > 256 and a % 256 == 0 and b % 256 == 0


def attend_sel(q=FAKE, k=FAKE, v=FAKE, B=1, H=2, n_tot=1100, d=64, dt=wf.WF_BF16, sel=FAKE, k0=64, gen=FAKE, n_gen=8,
               n_q=32, options=0, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib().wf_attend_selected(ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(v), B, H, n_tot, d, dt,
                                    ctypes.c_void_p(sel), k0, ctypes.c_void_p(gen), n_gen, n_q, options,
                                    ctypes.c_void_p(out), ctypes.c_void_p(ws), ws_bytes, None)


def test_attend_selected_rejects_bad_arguments():
    need = lib().wf_attend_selected_workspace_bytes(1, 2, 64, wf.WF_BF16, 32, 64, 8)
    assert need > 0
    assert lib().wf_attend_selected_workspace_bytes(1, 2, 96, wf.WF_BF16, 32, 64, 8) == 0   # head dim
    assert lib().wf_attend_selected_workspace_bytes(1, 2, 64, wf.WF_BF16, 65, 64, 8) == 0   # too many queries
    assert lib().wf_attend_selected_workspace_bytes(1, 2, 64, wf.WF_BF16, 32, 0, 0) == 0    # empty set
    assert attend_sel(q=0) == -1
    assert attend_sel(sel=0) == -1                 # a selection is needed when k0 > 0
    assert attend_sel(gen=0) == -1                 # generated rows are needed when n_gen > 0
    assert attend_sel(dt=5) == -3
    assert attend_sel(d=96) == -2
    assert attend_sel(k0=-1) == -2
    assert attend_sel(n_q=0) == -2
    assert attend_sel(n_tot=0) == -2
    assert attend_sel(q=MISALIGNED) == -7
    assert attend_sel(sel=FAKE + 2) == -7
    assert attend_sel(ws_bytes=need - 1) == -6
    assert attend_sel(options=1) == -10            # WF_ERR_OPTION: only WF_OPT_CHECK is defined
    assert attend_sel(options=wf.WF_OPT_CHECK, q=MISALIGNED) == -7   # the check bit itself is accepted


def refresh(items, n=None):
    arr = (wf._lib.WfRefreshItem * max(1, len(items)))()
    keep = []
    for slot, (k, pyr, blocks, n_blocks, stride) in zip(arr, items):
        slot.k_prompt = k
        slot.head_stride = stride
        slot.pyr = ctypes.pointer(pyr) if pyr is not None else None
        slot.blocks = blocks
        slot.n_blocks = n_blocks
        keep.append(pyr)
    return lib().wf_refresh_pyramids(arr, len(items) if n is None else n, None)


def test_refresh_rejects_bad_arguments():
    def one(k=FAKE, pyr=None, blocks=FAKE, n_blocks=8, stride=1024 * 64):
        return refresh([(k, fake_pyramid() if pyr is None else pyr, blocks, n_blocks, stride)])

    assert lib().wf_refresh_pyramids(None, 1, None) == -1
    assert refresh([(FAKE, fake_pyramid(), FAKE, 8, 1024 * 64)], n=0) == -2
    assert refresh([(FAKE, fake_pyramid(), FAKE, 8, 1024 * 64)], n=33) == -2
    assert one(k=0) == -1
    assert one(blocks=0) == -1
    assert one(blocks=0, n_blocks=0) != -1      # nothing to refresh needs no list
    assert one(n_blocks=-1) == -2
    assert one(pyr=fake_pyramid(magic=7)) == -9
    p_all = fake_pyramid()
    p_all.flags = wf.WF_PYR_ALL_LEVELS
    assert one(pyr=p_all) == -10
    assert one(stride=1000) == -2
    assert one(k=MISALIGNED) == -7
    assert one(blocks=FAKE + 2) == -7
    mixed = [(FAKE, fake_pyramid(), FAKE, 8, 1024 * 64), (FAKE, fake_pyramid(dt=wf.WF_F32), FAKE, 8, 1024 * 64)]
    assert refresh(mixed) == -3



def test_select_plan_rejects_an_attended_set_beyond_int_range():
    """The kept tokens plus the generated positions must stay within the
    attention's 2^24-entry bound, as for the attention-only call."""
    p = fake_pyramid()
    q = lambda *args: lib().wf_select_attend_workspace_bytes(*args, 0)  # noqa: E731
    assert q(ctypes.byref(p), 32, 5000, budgets_arr([8, 16, 32, 64])) > 0
    assert q(ctypes.byref(p), 32, (1 << 24) - 63, budgets_arr([8, 16, 32, 64])) == 0
    assert q(ctypes.byref(p), 32, 0x7FFFFFF0, budgets_arr([8, 16, 32, 64])) == 0
    assert select(n_gen=0x7FFFFFF0) == -2


class _FakePyr:
    """A Python-side pyramid over a fake descriptor (never passed to a kernel)."""

    def __init__(self, **kw):
        self.desc = fake_pyramid(**kw)


def _select_case(**over):
    """Consistent CPU tensors of a select-attend call on the fake pyramid
    (B=1, H=2, N_p=1024, d=64, bf16, L=3), with some replaced."""
    import torch
    bf = torch.bfloat16
    args = dict(q=torch.zeros(1, 2, 32, 64, dtype=bf), k=torch.zeros(1, 2, 1056, 64, dtype=bf),
                v=torch.zeros(1, 2, 1056, 64, dtype=bf), gen_idx=torch.arange(1024, 1056, dtype=torch.int32),
                budgets=[8, 16, 32, 64], out=torch.zeros(1, 2, 32, 64), sel_out=torch.zeros(1, 2, 64, dtype=torch.int32))
    args.update(over)
    return args


@pytest.mark.parametrize("bad", [
    dict(q=None),                                                    # q of fewer heads
    dict(v="short"),                                                 # v shorter than k
    dict(k="few_rows"),                                              # fewer rows than the prompt
    dict(k="d32"),                                                   # head dim differs from the pyramid's
    dict(gen_idx="int64"),
    dict(gen_idx="2d"),
    dict(out="bf16"),
    dict(out="shape"),
    dict(sel_out="shape"),
    dict(budgets=[8, 16, 64]),                                       # one budget per level
    dict(q="f32"),                                                   # dtype differs from the pyramid's
])
def test_select_args_are_checked_on_the_host(bad):
    """Mismatched tensors raise before any library call (so no kernel can
    read or write past a buffer)."""
    import torch
    from long_context_kv_haar_amd._lib import _check_select_args
    a = _select_case()
    key, val = next(iter(bad.items()))
    if key == "q" and val is None:
        a["q"] = torch.zeros(1, 1, 32, 64, dtype=torch.bfloat16)
    elif val == "short":
        a["v"] = a["v"][:, :, :1000].contiguous()
    elif val == "few_rows":
        a["k"] = a["k"][:, :, :1000].contiguous()
        a["v"] = a["v"][:, :, :1000].contiguous()
    elif val == "d32":
        a["k"] = torch.zeros(1, 2, 1056, 32, dtype=torch.bfloat16)
        a["v"] = torch.zeros(1, 2, 1056, 32, dtype=torch.bfloat16)
    elif val == "int64":
        a["gen_idx"] = a["gen_idx"].long()
    elif val == "2d":
        a["gen_idx"] = a["gen_idx"].view(2, 16)
    elif val == "bf16":
        a["out"] = a["out"].bfloat16()
    elif key == "out":
        a["out"] = torch.zeros(1, 2, 31, 64)
    elif key == "sel_out":
        a["sel_out"] = torch.zeros(1, 2, 63, dtype=torch.int32)
    elif key == "budgets":
        a["budgets"] = val
    elif val == "f32":
        a["q"], a["k"], a["v"] = (a[n].float() for n in ("q", "k", "v"))
    with pytest.raises((ValueError, TypeError)):
        _check_select_args(a["q"], _FakePyr(), a["k"], a["v"], a["gen_idx"], a["budgets"], a["out"], a["sel_out"])


def test_consistent_select_args_pass_the_host_checks():
    from long_context_kv_haar_amd._lib import _check_select_args
    a = _select_case()
    _check_select_args(a["q"], _FakePyr(), a["k"], a["v"], a["gen_idx"], a["budgets"], a["out"], a["sel_out"])


def test_attend_args_are_checked_on_the_host():
    import torch
    from long_context_kv_haar_amd._lib import _check_attend_args
    bf = torch.bfloat16
    q, k = torch.zeros(1, 2, 16, 64, dtype=bf), torch.zeros(1, 2, 300, 64, dtype=bf)
    v, out = torch.zeros(1, 2, 300, 64, dtype=bf), torch.zeros(1, 2, 16, 64)
    sel, gen = torch.zeros(1, 2, 10, dtype=torch.int32), torch.zeros(5, dtype=torch.int32)
    _check_attend_args(q, k, v, sel, gen, out)
    for bad in (dict(v=v[:, :, :10].contiguous()), dict(sel=sel.long()), dict(sel=torch.zeros(1, 3, 10, dtype=torch.int32)),
                dict(gen=gen.view(1, 5)), dict(out=out[:, :1].contiguous()), dict(k=k.float())):
        args = dict(q=q, k=k, v=v, sel=sel, gen=gen, out=out)
        args.update(bad)
        with pytest.raises((ValueError, TypeError)):
            _check_attend_args(args["q"], args["k"], args["v"], args["sel"], args["gen"], args["out"])


def test_public_calls_reject_host_tensors_before_the_library():
    import torch
    a = _select_case()
    with pytest.raises(ValueError):
        wf.select_attend(a["q"], _FakePyr(), a["k"], a["v"], a["gen_idx"], a["budgets"])
    with pytest.raises(ValueError):
        wf.attend_selected(a["q"], a["k"], a["v"], None, a["gen_idx"])


def noalloc_scratch_bytes():
    m = re.search(r"#define\s+WF_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", open(HEADER).read())
    return int(m.group(1)) << int(m.group(2))


def test_noalloc_scratch_holds_every_workload():
    from workloads.configs import CONFIGS
    cap = noalloc_scratch_bytes()
    assert cap == 16 << 20
    for c in CONFIGS.values():
        p = fake_pyramid(levels=c.levels, n=c.n_prompt, d=c.head_dim, H=c.batch * c.heads,
                         dt=wf.WF_BF16 if c.dtype == "bf16" else wf.WF_F32)
        need = lib().wf_select_attend_workspace_bytes(ctypes.byref(p), c.n_q, c.n_gen, budgets_arr(c.budgets), 0)
        assert 0 < need <= cap, (c.name, need)


def noalloc(p, budgets, n_q=32, n_gen=32, out=FAKE, q=FAKE, agg=wf.WF_AGG_MAX):
    return lib().wf_select_attend_noalloc(ctypes.c_void_p(q), ctypes.byref(p), ctypes.c_void_p(FAKE),
                                          ctypes.c_void_p(FAKE), 1 << 20, ctypes.c_void_p(FAKE), n_gen,
                                          budgets_arr(budgets), n_q, agg, ctypes.c_void_p(out), None, None, None, None)


def test_noalloc_rejects_a_workspace_beyond_its_scratch_before_any_device_call():
    # 2 048 heads of a 1K prompt: the split partials alone exceed the scratch array
    p = fake_pyramid(levels=3, n=1024, d=64, H=2048)
    need = lib().wf_select_attend_workspace_bytes(ctypes.byref(p), 32, 32, budgets_arr([8, 16, 32, 64]), 0)
    assert need > noalloc_scratch_bytes()
    assert noalloc(p, [8, 16, 32, 64]) == -6                  # WF_ERR_WORKSPACE


def test_noalloc_checks_its_arguments_like_the_workspace_call():
    p = fake_pyramid()
    assert noalloc(p, [8, 16, 32, 64], q=0) == -1              # WF_ERR_NULL
    assert noalloc(p, [8, 16, 32, 64], out=0) == -1
    assert noalloc(p, [8, 17, 32, 64]) == -5                   # k_2 > 2 k_3: WF_ERR_BUDGET
    assert noalloc(p, [8, 16, 32, 64], n_q=65) == -2           # WF_ERR_SHAPE
    assert noalloc(fake_pyramid(magic=0), [8, 16, 32, 64]) == -9  # WF_ERR_PYRAMID


def _layers(pyrs, q=FAKE):
    from long_context_kv_haar_amd._lib import WfLayerItem
    arr = (WfLayerItem * len(pyrs))()
    for i, p in enumerate(pyrs):
        arr[i] = WfLayerItem(q, ctypes.pointer(p), FAKE, FAKE, FAKE, None)
    return arr


def layers_call(pyrs, n_items=None, budgets=(8, 16, 32, 64), agg=wf.WF_AGG_MAX, q=FAKE, ws_bytes=1 << 30):
    arr = _layers(pyrs, q)
    n = len(pyrs) if n_items is None else n_items
    return lib().wf_select_attend_layers(arr, n, 1056, ctypes.c_void_p(FAKE), 32, budgets_arr(list(budgets)), 32, agg,
                                         ctypes.c_void_p(FAKE), ws_bytes, None)


def test_layers_workspace_grows_with_the_layers_and_caps_the_heads():
    q = lib().wf_select_attend_layers_workspace_bytes
    p = fake_pyramid()
    one = q(ctypes.byref(p), 1, 32, 32, budgets_arr([8, 16, 32, 64]))
    assert one == lib().wf_select_attend_workspace_bytes(ctypes.byref(p), 32, 32, budgets_arr([8, 16, 32, 64]), 0)
    assert q(ctypes.byref(p), 4, 32, 32, budgets_arr([8, 16, 32, 64])) > one
    assert q(ctypes.byref(p), 0, 32, 32, budgets_arr([8, 16, 32, 64])) == 0
    assert q(ctypes.byref(p), 33, 32, 32, budgets_arr([8, 16, 32, 64])) == 0
    # 32 layers of 2 048 heads exceed the head limit of a launch
    assert q(ctypes.byref(fake_pyramid(H=2048)), 32, 32, 32, budgets_arr([8, 16, 32, 64])) == 0
    # pyramids with stored finer bands are not batched
    db2 = WfPyramid(1, 2, 1024, 64, 3, wf.WF_BF16, wf.WF_PYR_DB2, 0x57465059, FAKE, 1 << 20)
    assert q(ctypes.byref(db2), 2, 32, 32, budgets_arr([8, 16, 32, 64])) == 0


def test_layers_call_checks_its_arguments_before_any_device_call():
    p = fake_pyramid()
    assert layers_call([p, fake_pyramid()], n_items=0) == -2            # WF_ERR_SHAPE
    assert layers_call([p] * 2, n_items=33) == -2
    assert layers_call([p, fake_pyramid(H=3)]) == -2                    # layers of different shapes
    assert layers_call([p, fake_pyramid(levels=2)]) == -2
    assert layers_call([p, fake_pyramid(dt=wf.WF_F32)]) == -3           # WF_ERR_DTYPE
    assert layers_call([p, fake_pyramid(magic=0)]) == -9                # WF_ERR_PYRAMID
    assert layers_call([p], q=0) == -1                                  # WF_ERR_NULL
    assert layers_call([p], q=MISALIGNED) == -7                         # WF_ERR_ALIGN
    assert layers_call([p], budgets=(8, 17, 32, 64)) == -5              # WF_ERR_BUDGET
    assert layers_call([p], agg=7) == -10                               # WF_ERR_OPTION
    assert layers_call([p], ws_bytes=16) == -6                          # WF_ERR_WORKSPACE
    db2 = WfPyramid(1, 2, 1024, 64, 3, wf.WF_BF16, wf.WF_PYR_DB2, 0x57465059, FAKE, 1 << 20)
    assert layers_call([p, db2]) == -10


def test_softmax_aggregations_plan_their_logits_and_limits():
    q = lib().wf_select_attend_workspace_bytes
    p = fake_pyramid()
    b = budgets_arr([8, 16, 32, 64])
    plain = q(ctypes.byref(p), 32, 32, b, wf.WF_AGG_MAX)
    assert q(ctypes.byref(p), 32, 32, b, wf.WF_AGG_MEAN) == plain
    # every row's logits: level L (128 regions) and the covered levels 0 .. 2 (64 + 32 + 16 positions)
    soft = q(ctypes.byref(p), 32, 32, b, wf.WF_AGG_SOFTMAX_MAX)
    assert soft >= plain + 2 * 32 * (128 + 64 + 32 + 16) * 4
    assert q(ctypes.byref(p), 32, 32, b, wf.WF_AGG_SOFTMAX_MEAN) == soft
    assert q(ctypes.byref(p), 32, 32, b, 4) == 0
    # covered sets beyond 8 192 positions have no softmax refinement
    big = fake_pyramid(levels=3, n=1 << 16, H=1)
    assert q(ctypes.byref(big), 32, 0, budgets_arr([1025, 2050, 4100, 8200]), wf.WF_AGG_MAX) > 0
    assert q(ctypes.byref(big), 32, 0, budgets_arr([1025, 2050, 4100, 8200]), wf.WF_AGG_SOFTMAX_MAX) == 0
    # not on a pyramid with stored bands, not batched over layers
    db2 = WfPyramid(1, 2, 1024, 64, 3, wf.WF_BF16, wf.WF_PYR_DB2, 0x57465059, FAKE, 1 << 20)
    assert q(ctypes.byref(db2), 32, 32, b, wf.WF_AGG_SOFTMAX_MAX) == 0
    assert select(pyr=db2, agg=wf.WF_AGG_SOFTMAX_MEAN) == -10
    assert layers_call([p, fake_pyramid()], agg=wf.WF_AGG_SOFTMAX_MAX) == -10
