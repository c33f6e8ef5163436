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
    assert len(names) == 10, names
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
    q = lib().wf_select_attend_workspace_bytes
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
    assert select(agg=2) == -10
    assert select(agg=-1) == -10


def attend_sel(q=FAKE, k=FAKE, v=FAKE, B=1, H=2, n_tot=1100, d=64, dt=wf.WF_BF16, sel=FAKE, k0=64, gen=FAKE, n_gen=8,
               n_q=32, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib().wf_attend_selected(ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(v), B, H, n_tot, d, dt,
                                    ctypes.c_void_p(sel), k0, ctypes.c_void_p(gen), n_gen, n_q, ctypes.c_void_p(out),
                                    ctypes.c_void_p(ws), ws_bytes, None)


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

