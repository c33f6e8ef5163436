"""ctypes binding of libwavefilter.so (argument marshalling only).

Every step of the path runs inside the HIP library.  PyTorch provides device
memory (tensors are passed by ``data_ptr``) and the stream
(``torch.cuda.current_stream().cuda_stream``).  There is no fallback: if the
library is missing or fails to load, every call raises.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwavefilter.so")

WF_OK = 0
WF_F32 = 0
WF_BF16 = 1
WF_AGG_MAX = 0
WF_AGG_MEAN = 1
WF_AGG_SOFTMAX_MAX = 2
WF_AGG_SOFTMAX_MEAN = 3
AGGREGATIONS = {"max": WF_AGG_MAX, "mean": WF_AGG_MEAN, "softmax_max": WF_AGG_SOFTMAX_MAX,
                "softmax_mean": WF_AGG_SOFTMAX_MEAN}
WF_PYR_ALL_LEVELS = 1
WF_PYR_DB2 = 2
WF_OPT_CHECK = 0x100
CHECK_BITS = {"gen_index": 1, "sel_index": 2, "nonfinite_q": 4, "nonfinite_k": 8, "nonfinite_v": 16,
              "nonfinite_pyramid": 32}
MAX_LEVELS = 7
MAX_QUERIES = 64
U64_MAX = (1 << 64) - 1

STATUS_NAMES = {
    0: "WF_OK", -1: "WF_ERR_NULL", -2: "WF_ERR_SHAPE", -3: "WF_ERR_DTYPE", -4: "WF_ERR_LEVELS",
    -5: "WF_ERR_BUDGET", -6: "WF_ERR_WORKSPACE", -7: "WF_ERR_ALIGN", -8: "WF_ERR_HIP", -9: "WF_ERR_PYRAMID",
    -10: "WF_ERR_OPTION",
}
MAX_REFRESH_ITEMS = 32


class WfPyramid(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("n_prompt", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("levels", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("magic", ctypes.c_uint32),
        ("base", ctypes.c_void_p),
        ("bytes", ctypes.c_uint64),
    ]


class WfRefreshItem(ctypes.Structure):
    _fields_ = [
        ("k_prompt", ctypes.c_void_p),
        ("head_stride", ctypes.c_int64),
        ("pyr", ctypes.POINTER(WfPyramid)),
        ("blocks", ctypes.c_void_p),
        ("n_blocks", ctypes.c_int32),
    ]


class WfLayerItem(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("pyr", ctypes.POINTER(WfPyramid)),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("sel_out", ctypes.c_void_p),
    ]


MAX_LAYER_ITEMS = 32


class WfError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


_LIB = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build it with long_context_kv_haar_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64
        pyr_p = ctypes.POINTER(WfPyramid)
        i32p = ctypes.POINTER(ctypes.c_int32)
        L.wf_version.restype = ctypes.c_char_p
        L.wf_version.argtypes = []
        L.wf_status_string.restype = ctypes.c_char_p
        L.wf_status_string.argtypes = [ctypes.c_int]
        L.wf_pyramid_bytes.restype = u64
        L.wf_pyramid_bytes.argtypes = [i32, i32, i32, i32, i32, u32]
        L.wf_pyramid_offset.restype = u64
        L.wf_pyramid_offset.argtypes = [pyr_p, i32, i32]
        L.wf_build_pyramid.restype = ctypes.c_int
        L.wf_build_pyramid.argtypes = [vp, i64, i32, i32, i32, i32, i32, i32, u32, vp, u64, pyr_p, vp]
        L.wf_select_attend_workspace_bytes.restype = u64
        L.wf_select_attend_workspace_bytes.argtypes = [pyr_p, i32, i32, i32p, i32]
        L.wf_select_attend.restype = ctypes.c_int
        L.wf_select_attend.argtypes = [vp, pyr_p, vp, vp, i32, vp, i32, i32p, i32, i32, vp, vp, vp, vp, vp, u64, vp]
        L.wf_select_attend_noalloc.restype = ctypes.c_int
        L.wf_select_attend_noalloc.argtypes = [vp, pyr_p, vp, vp, i32, vp, i32, i32p, i32, i32, vp, vp, vp, vp, vp]
        L.wf_select_attend_layers_workspace_bytes.restype = u64
        L.wf_select_attend_layers_workspace_bytes.argtypes = [pyr_p, i32, i32, i32, i32p]
        L.wf_select_attend_layers.restype = ctypes.c_int
        L.wf_select_attend_layers.argtypes = [ctypes.POINTER(WfLayerItem), i32, i32, vp, i32, i32p, i32, i32, vp, u64,
                                              vp]
        L.wf_refresh_pyramids.restype = ctypes.c_int
        L.wf_refresh_pyramids.argtypes = [ctypes.POINTER(WfRefreshItem), i32, vp]
        L.wf_attend_selected_workspace_bytes.restype = u64
        L.wf_attend_selected_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.wf_attend_selected.restype = ctypes.c_int
        L.wf_attend_selected.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, vp, i32, i32, i32, vp, vp, u64,
                                         vp]
        L.wf_check_status.restype = ctypes.c_int
        L.wf_check_status.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32)]
        _LIB = L
    return _LIB


def version():
    return lib().wf_version().decode()


def status_string(status):
    return lib().wf_status_string(int(status)).decode()


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return WF_BF16
    if t.dtype == torch.float32:
        return WF_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_handle(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _budget_array(budgets):
    arr = (ctypes.c_int32 * len(budgets))(*[int(b) for b in budgets])
    return arr


def pyramid_bytes(batch, heads, n_prompt, head_dim, levels, flags=0):
    return int(lib().wf_pyramid_bytes(batch, heads, n_prompt, head_dim, levels, flags))


class Pyramid:
    """Device pyramid buffer plus its C descriptor."""

    def __init__(self, buf, desc):
        self.buf = buf
        self.desc = desc

    @property
    def levels(self):
        return self.desc.levels

    def band(self, band, level):
        """Float32 view ``[B, H, N_p / 2^level, d]`` of a stored band (0 = A, 1 = D)."""
        off = int(lib().wf_pyramid_offset(ctypes.byref(self.desc), band, level))
        if off == U64_MAX:
            raise KeyError((band, level))
        d = self.desc
        n = (d.batch * d.heads * (d.n_prompt >> level) * d.head_dim)
        flat = self.buf[off:off + 4 * n].view(torch.float32)
        return flat.view(d.batch, d.heads, d.n_prompt >> level, d.head_dim)

    @property
    def top(self):
        return self.band(0, self.desc.levels)


def build_pyramid(k, n_prompt, levels, flags=0, buf=None):
    """Haar pyramid of the prompt rows ``k[:, :, :n_prompt]`` of a ``[B, H, N, d]`` cache."""
    if k.dim() != 4 or not k.is_cuda or not k.is_contiguous():
        raise ValueError("k must be a contiguous [B, H, N, d] device tensor")
    B, H, N, d = k.shape
    need = pyramid_bytes(B, H, n_prompt, d, levels, flags)
    if need == 0:
        raise WfError(-2, "wf_pyramid_bytes")
    if buf is None or buf.numel() < need:
        buf = torch.empty(need, dtype=torch.uint8, device=k.device)
    desc = WfPyramid()
    st = lib().wf_build_pyramid(ctypes.c_void_p(k.data_ptr()), N * d, B, H, n_prompt, d, _dtype_code(k), levels,
                                flags, ctypes.c_void_p(buf.data_ptr()), buf.numel(), ctypes.byref(desc),
                                _stream_handle(k.device))
    if st != WF_OK:
        raise WfError(st, "wf_build_pyramid")
    return Pyramid(buf, desc)


def _refresh_array(items):
    if not 1 <= len(items) <= MAX_REFRESH_ITEMS:
        raise ValueError(f"1 .. {MAX_REFRESH_ITEMS} items per call")
    arr = (WfRefreshItem * len(items))()
    keep = []
    for slot, (k, pyr, blocks) in zip(arr, items):
        if k.dim() != 4 or not k.is_cuda or not k.is_contiguous():
            raise ValueError("k must be a contiguous [B, H, N, d] device tensor")
        d = pyr.desc
        _need(tuple(k.shape[:2]) == (d.batch, d.heads) and k.shape[3] == d.head_dim and k.shape[2] >= d.n_prompt,
              "k must be [B, H, N >= N_p, d] of the pyramid's shape")
        _need(_dtype_code(k) == d.dtype, "k must have the dtype the pyramid was built from")
        if blocks is not None:
            _check_tensor(blocks, "blocks", k.device, dtype=torch.int32)
            _need(blocks.dim() == 1, "blocks must be 1-d")
        slot.k_prompt = k.data_ptr()
        slot.head_stride = k.shape[2] * k.shape[3]
        slot.pyr = ctypes.pointer(pyr.desc)
        slot.blocks = 0 if blocks is None else blocks.data_ptr()
        slot.n_blocks = 0 if blocks is None else blocks.numel()
        keep.append((k, pyr, blocks))
    return arr, keep


def refresh_pyramids(items):
    """Recompute the listed level-L blocks of several pyramids in one launch.

    ``items`` is a list of ``(k, pyr, blocks)``: the layer's current
    ``[B, H, N, d]`` cache (prompt rows first, as built), its ``Pyramid`` and
    an int32 device tensor of level-L block indices shared by all heads.
    """
    arr, _ = _refresh_array(items)
    st = lib().wf_refresh_pyramids(arr, len(items), _stream_handle(items[0][0].device))
    if st != WF_OK:
        raise WfError(st, "wf_refresh_pyramids")


class PreparedRefresh:
    """A refresh call with its item array marshalled once."""

    def __init__(self, items):
        self._arr, self._keep = _refresh_array(items)
        self._n = len(items)
        self._stream = _stream_handle(items[0][0].device)
        self._fn = lib().wf_refresh_pyramids

    def __call__(self):
        st = self._fn(self._arr, self._n, self._stream)
        if st != WF_OK:
            raise WfError(st, "wf_refresh_pyramids")


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_tensor(t, name, device, dtype=None, shape=None):
    """``t`` lives on ``device``, is contiguous, and has the given dtype and shape."""
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.device == device, f"{name} must be on {device} (got {t.device})")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _check_qkv(q, k, v, batch, heads, head_dim):
    """q ``[B, H, n_q, d]`` and k, v ``[B, H, N_tot, d]`` of one dtype on q's device."""
    dev = q.device
    _need(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be 4-d [B, H, rows, d] tensors")
    _need(q.dtype == k.dtype == v.dtype, "q, k, v must share one dtype")
    _dtype_code(q)
    _check_tensor(q, "q", dev, shape=(batch, heads, q.shape[2], head_dim))
    _check_tensor(k, "k", dev, shape=(batch, heads, k.shape[2], head_dim))
    _check_tensor(v, "v", dev, shape=tuple(k.shape))
    _need(1 <= q.shape[2] <= MAX_QUERIES, f"n_q must be 1 .. {MAX_QUERIES}")


def _check_select_args(q, pyr, k, v, gen_idx, budgets, out, sel_out, sel_levels=None, score_levels=None):
    """Host-side checks of a select-attend call: the tensors must match the
    pyramid descriptor and each other, so no kernel reads or writes past a
    buffer.  Raises ValueError (or WfError for a dtype mismatch with the
    pyramid); launches nothing."""
    d = pyr.desc
    _check_qkv(q, k, v, d.batch, d.heads, d.head_dim)
    _need(_dtype_code(q) == d.dtype, "q, k, v must have the dtype the pyramid was built from")
    _need(k.shape[2] >= d.n_prompt, f"k, v must hold at least the {d.n_prompt} prompt rows")
    _need(len(budgets) == d.levels + 1, f"need {d.levels + 1} budgets (k_L .. k_0)")
    dev = q.device
    if gen_idx is not None:
        _check_tensor(gen_idx, "gen_idx", dev, dtype=torch.int32)
        _need(gen_idx.dim() == 1, "gen_idx must be 1-d")
    B, H, n_q, hd = q.shape
    _check_tensor(out, "out", dev, dtype=torch.float32, shape=(B, H, n_q, hd))
    if sel_out is not None:
        _check_tensor(sel_out, "sel_out", dev, dtype=torch.int32, shape=(B, H, int(budgets[-1])))
    total = sum(int(b) for b in budgets)
    if sel_levels is not None:
        _check_tensor(sel_levels, "sel_levels", dev, dtype=torch.int32, shape=(B, H, total))
    if score_levels is not None:
        _check_tensor(score_levels, "score_levels", dev, dtype=torch.float32, shape=(B, H, total))


def _check_attend_args(q, k, v, sel, gen_idx, out):
    """Host-side checks of an attend-selected call (see _check_select_args)."""
    _need(q.dim() == 4, "q must be a 4-d [B, H, n_q, d] tensor")
    B, H, n_q, hd = q.shape
    _check_qkv(q, k, v, B, H, hd)
    dev = q.device
    if sel is not None:
        _check_tensor(sel, "sel", dev, dtype=torch.int32)
        _need(sel.dim() == 3 and tuple(sel.shape[:2]) == (B, H), "sel must be int32 [B, H, k0]")
    if gen_idx is not None:
        _check_tensor(gen_idx, "gen_idx", dev, dtype=torch.int32)
        _need(gen_idx.dim() == 1, "gen_idx must be 1-d")
    _check_tensor(out, "out", dev, dtype=torch.float32, shape=(B, H, n_q, hd))


def _check_workspace(ws, dev, need):
    _check_tensor(ws, "workspace", dev, dtype=torch.uint8)
    _need(ws.numel() >= need, f"workspace holds {ws.numel()} bytes, the call needs {need}")


def workspace_bytes(pyr, n_q, n_gen, budgets, agg="max"):
    return int(lib().wf_select_attend_workspace_bytes(ctypes.byref(pyr.desc), n_q, n_gen, _budget_array(budgets),
                                                      _agg_code(agg)))


class Workspace:
    """Zero-filled device workspace, grown on demand and reused across calls."""

    def __init__(self, device):
        self.device = device
        self.buf = torch.zeros(0, dtype=torch.uint8, device=device)

    def get(self, nbytes):
        if self.buf.numel() < nbytes:
            self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf


_WORKSPACES = {}


def default_workspace(device):
    """The workspace calls without an explicit one use: one per (device,
    current stream), so calls on different streams never share scratch
    memory (concurrent calls on one workspace would race)."""
    device = torch.device(device)
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    ws = _WORKSPACES.get(key)
    if ws is None:
        ws = _WORKSPACES[key] = Workspace(device)
    return ws


def _agg_code(agg, check=False):
    if agg not in AGGREGATIONS:
        raise ValueError(f"agg must be one of {sorted(AGGREGATIONS)}")
    return AGGREGATIONS[agg] | (WF_OPT_CHECK if check else 0)


def check_status(workspace=None, device=None):
    """The status word the last call made with ``check=True`` left in its
    workspace: a ``Workspace``, a uint8 device tensor, None for the default
    workspace of ``device`` (current device) on the current stream, or the
    string "noalloc" for the static scratch of ``select_attend_noalloc``.
    Returns the set of names of ``CHECK_BITS`` that are set (empty: the
    inputs met every checked precondition).  Synchronises the stream."""
    if isinstance(workspace, str):
        _need(workspace == "noalloc", "workspace must be a tensor, a Workspace, None or 'noalloc'")
        dev = torch.device(device if device is not None else torch.cuda.current_device())
        ptr = None
    else:
        if workspace is None:
            dev = torch.device(device if device is not None else torch.cuda.current_device())
            if dev.index is None:
                dev = torch.device("cuda", torch.cuda.current_device())
            workspace = default_workspace(dev)
        buf = workspace.buf if isinstance(workspace, Workspace) else workspace
        _need(isinstance(buf, torch.Tensor) and buf.is_cuda and buf.numel() >= 4, "no workspace to read")
        dev = buf.device
        ptr = buf.data_ptr()
    word = ctypes.c_uint32(0)
    st = lib().wf_check_status(ctypes.c_void_p(ptr), _stream_handle(dev), ctypes.byref(word))
    if st != WF_OK:
        raise WfError(st, "wf_check_status")
    return {name for name, bit in CHECK_BITS.items() if word.value & bit}


def select_attend(q, pyr, k, v, gen_idx, budgets, out=None, sel_out=None, levels_out=False, workspace=None,
                  agg="max", check=False):
    """One step for every (sequence, head).

    ``agg`` combines the query rows into region scores: "max" or "mean".
    ``check`` runs the debug input checks (read with ``check_status``).
    Returns a dict with ``out`` (float32 ``[B, H, n_q, d]``), ``sel``
    (int32 ``[B, H, k_0]``) and, with ``levels_out``, ``sel_levels`` /
    ``score_levels`` (``[B, H, sum k_j]``, level L first).
    """
    agg_code = _agg_code(agg, check)
    _need(isinstance(q, torch.Tensor) and q.is_cuda, "q must be a device tensor")
    _need(q.dim() == 4, "q must be a 4-d [B, H, n_q, d] tensor")
    B, H, n_q, d = q.shape
    n_tot = k.shape[2]
    dev = q.device
    n_gen = 0 if gen_idx is None else gen_idx.numel()
    budgets = [int(b) for b in budgets]
    if out is None:
        out = torch.empty((B, H, n_q, d), dtype=torch.float32, device=dev)
    k0 = budgets[-1]
    if sel_out is None:
        sel_out = torch.empty((B, H, k0), dtype=torch.int32, device=dev)
    sel_levels = score_levels = None
    if levels_out:
        sel_levels = torch.empty((B, H, sum(budgets)), dtype=torch.int32, device=dev)
        score_levels = torch.empty((B, H, sum(budgets)), dtype=torch.float32, device=dev)
    _check_select_args(q, pyr, k, v, gen_idx, budgets, out, sel_out, sel_levels, score_levels)
    barr = _budget_array(budgets)
    ws_need = int(lib().wf_select_attend_workspace_bytes(ctypes.byref(pyr.desc), n_q, n_gen, barr, agg_code))
    if ws_need == 0:
        raise WfError(-5, "wf_select_attend_workspace_bytes")
    if workspace is None:
        workspace = default_workspace(dev)
    ws = workspace.get(ws_need)

    def ptr(t):
        return ctypes.c_void_p(0 if t is None else t.data_ptr())

    st = lib().wf_select_attend(ptr(q), ctypes.byref(pyr.desc), ptr(k), ptr(v), n_tot, ptr(gen_idx), n_gen, barr,
                                n_q, agg_code, ptr(out), ptr(sel_out), ptr(sel_levels), ptr(score_levels), ptr(ws),
                                ws.numel(), _stream_handle(dev))
    if st != WF_OK:
        raise WfError(st, "wf_select_attend")
    res = {"out": out, "sel": sel_out}
    if levels_out:
        res["sel_levels"] = sel_levels
        res["score_levels"] = score_levels
    return res


def select_attend_noalloc(q, pyr, k, v, gen_idx, budgets, out, sel_out=None, sel_levels=None, score_levels=None,
                          agg="max", check=False):
    """``select_attend`` through ``wf_select_attend_noalloc``: the workspace is
    the library's static per-device scratch array, and the caller passes
    every output (``out`` float32 ``[B, H, n_q, d]``; optional ``sel_out``
    int32 ``[B, H, k_0]``, ``sel_levels`` int32 / ``score_levels`` float32
    ``[B, H, sum k_j]``), so nothing is allocated by this call.  Calls that
    overlap on one device race on the scratch array.  ``check``: read the
    status with ``check_status("noalloc")``."""
    agg_code = _agg_code(agg, check)
    _need(isinstance(q, torch.Tensor) and q.is_cuda, "q must be a device tensor")
    _need(q.dim() == 4, "q must be a 4-d [B, H, n_q, d] tensor")
    _need(out is not None, "out must be passed (this call allocates nothing)")
    budgets = [int(b) for b in budgets]
    _check_select_args(q, pyr, k, v, gen_idx, budgets, out, sel_out, sel_levels, score_levels)
    n_q, n_tot = q.shape[2], k.shape[2]
    n_gen = 0 if gen_idx is None else gen_idx.numel()

    def ptr(t):
        return ctypes.c_void_p(0 if t is None else t.data_ptr())

    st = lib().wf_select_attend_noalloc(ptr(q), ctypes.byref(pyr.desc), ptr(k), ptr(v), n_tot, ptr(gen_idx), n_gen,
                                        _budget_array(budgets), n_q, agg_code, ptr(out), ptr(sel_out),
                                        ptr(sel_levels), ptr(score_levels), _stream_handle(q.device))
    if st != WF_OK:
        raise WfError(st, "wf_select_attend_noalloc")
    return {"out": out, "sel": sel_out, "sel_levels": sel_levels, "score_levels": score_levels}


def attend_selected_workspace_bytes(batch, heads, head_dim, dtype_code, n_q, k0, n_gen):
    return int(lib().wf_attend_selected_workspace_bytes(batch, heads, head_dim, dtype_code, n_q, k0, n_gen))


def _attend_selected_args(q, k, v, sel, gen_idx, out, ws, check=False):
    B, H, n_q, d = q.shape
    k0 = 0 if sel is None else sel.shape[-1]
    n_gen = 0 if gen_idx is None else gen_idx.numel()

    def ptr(t):
        return ctypes.c_void_p(0 if t is None else t.data_ptr())

    return (ptr(q), ptr(k), ptr(v), B, H, k.shape[2], d, _dtype_code(q), ptr(sel), k0, ptr(gen_idx), n_gen, n_q,
            WF_OPT_CHECK if check else 0, ptr(out), ptr(ws), ws.numel(), _stream_handle(q.device))


def attend_selected(q, k, v, sel, gen_idx, out=None, workspace=None, check=False):
    """Attention only over a selection made earlier (``sel``: int32
    ``[B, H, k0]`` prompt rows, e.g. ``select_attend(...)["sel"]``) plus the
    generated rows ``gen_idx``.  Returns float32 ``[B, H, n_q, d]``.
    ``check`` runs the debug input checks (read with ``check_status``)."""
    _need(isinstance(q, torch.Tensor) and q.is_cuda, "q must be a device tensor")
    _need(q.dim() == 4, "q must be a 4-d [B, H, n_q, d] tensor")
    B, H, n_q, d = q.shape
    if out is None:
        out = torch.empty((B, H, n_q, d), dtype=torch.float32, device=q.device)
    _check_attend_args(q, k, v, sel, gen_idx, out)
    k0 = 0 if sel is None else sel.shape[-1]
    n_gen = 0 if gen_idx is None else gen_idx.numel()
    need = attend_selected_workspace_bytes(B, H, d, _dtype_code(q), n_q, k0, n_gen)
    if need == 0:
        raise WfError(-2, "wf_attend_selected_workspace_bytes")
    if workspace is None:
        workspace = default_workspace(q.device)
    ws = workspace.get(need)
    st = lib().wf_attend_selected(*_attend_selected_args(q, k, v, sel, gen_idx, out, ws, check))
    if st != WF_OK:
        raise WfError(st, "wf_attend_selected")
    return out


class PreparedAttend:
    """An attend_selected call with its arguments marshalled once."""

    def __init__(self, q, k, v, sel, gen_idx, out, workspace, check=False):
        _need(isinstance(q, torch.Tensor) and q.is_cuda and q.dim() == 4, "q must be a 4-d device tensor")
        _check_attend_args(q, k, v, sel, gen_idx, out)
        B, H, n_q, d = q.shape
        need = attend_selected_workspace_bytes(B, H, d, _dtype_code(q), n_q, 0 if sel is None else sel.shape[-1],
                                               0 if gen_idx is None else gen_idx.numel())
        if need == 0:
            raise WfError(-2, "PreparedAttend")
        _check_workspace(workspace, q.device, need)
        self._keep = (q, k, v, sel, gen_idx, out, workspace)
        self._args = _attend_selected_args(q, k, v, sel, gen_idx, out, workspace, check)
        self._fn = lib().wf_attend_selected

    def __call__(self):
        st = self._fn(*self._args)
        if st != WF_OK:
            raise WfError(st, "wf_attend_selected")


def split_levels(flat, budgets):
    """Split a ``[..., sum k_j]`` per-level tensor into {level j: [..., k_j]}."""
    L = len(budgets) - 1
    out, off = {}, 0
    for i, kb in enumerate(budgets):
        out[L - i] = flat[..., off:off + kb]
        off += kb
    return out


class PreparedStep:
    """A select-attend call with every argument marshalled once, for tight
    loops (benchmarks, serving): calling it only crosses into the library."""

    def __init__(self, q, pyr, k, v, gen_idx, budgets, out, sel_out, workspace, sel_levels=None, score_levels=None,
                 agg="max", check=False):
        n_gen = 0 if gen_idx is None else gen_idx.numel()
        _need(isinstance(q, torch.Tensor) and q.is_cuda and q.dim() == 4, "q must be a 4-d device tensor")
        budgets = [int(b) for b in budgets]
        _check_select_args(q, pyr, k, v, gen_idx, budgets, out, sel_out, sel_levels, score_levels)
        self._keep = (q, pyr, k, v, gen_idx, out, sel_out, workspace, sel_levels, score_levels)
        self._barr = _budget_array(budgets)
        need = int(lib().wf_select_attend_workspace_bytes(ctypes.byref(pyr.desc), q.shape[2], n_gen, self._barr,
                                                          _agg_code(agg)))
        if need == 0:
            raise WfError(-5, "PreparedStep")
        _check_workspace(workspace, q.device, need)

        def ptr(t):
            return ctypes.c_void_p(0 if t is None else t.data_ptr())

        self._args = (ptr(q), ctypes.byref(pyr.desc), ptr(k), ptr(v), k.shape[2], ptr(gen_idx), n_gen, self._barr,
                      q.shape[2], _agg_code(agg, check), ptr(out), ptr(sel_out), ptr(sel_levels), ptr(score_levels),
                      ptr(workspace), workspace.numel(), _stream_handle(q.device))
        self._fn = lib().wf_select_attend

    def __call__(self):
        st = self._fn(*self._args)
        if st != WF_OK:
            raise WfError(st, "wf_select_attend")


def _layer_array(layers, gen_idx, budgets):
    """Check the layers of a batched call against one another and marshal
    them: ``layers`` is a list of (q, pyr, k, v, out, sel_out) with sel_out
    optionally None."""
    _need(1 <= len(layers) <= MAX_LAYER_ITEMS, f"1 to {MAX_LAYER_ITEMS} layers")
    q0, p0, k0_, v0 = layers[0][:4]
    for q, pyr, k, v, out, sel_out in layers:
        _check_select_args(q, pyr, k, v, gen_idx, budgets, out, sel_out)
        _need(q.shape == q0.shape and k.shape == k0_.shape and v.shape == v0.shape and q.dtype == q0.dtype,
              "every layer must have the same shapes and element type")
        _need(q.device == q0.device, "every layer must be on one device")
    arr = (WfLayerItem * len(layers))()
    for i, (q, pyr, k, v, out, sel_out) in enumerate(layers):
        arr[i] = WfLayerItem(q.data_ptr(), ctypes.pointer(pyr.desc), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             None if sel_out is None else sel_out.data_ptr())
    return arr


def layers_workspace_bytes(pyr, n_items, n_q, n_gen, budgets):
    return int(lib().wf_select_attend_layers_workspace_bytes(ctypes.byref(pyr.desc), n_items, n_q, n_gen,
                                                             _budget_array(budgets)))


def select_attend_layers(layers, gen_idx, budgets, agg="max", workspace=None, check=False):
    """``select_attend`` for several layers of one shape in one call.

    ``layers`` is a list of (q, pyr, k, v) or (q, pyr, k, v, out, sel_out);
    missing outputs are allocated.  Returns a list of dicts with ``out`` and
    ``sel`` per layer."""
    budgets = [int(b) for b in budgets]
    full = []
    for lay in layers:
        q, pyr, k, v = lay[:4]
        _need(isinstance(q, torch.Tensor) and q.is_cuda and q.dim() == 4, "q must be a 4-d device tensor")
        out = lay[4] if len(lay) > 4 and lay[4] is not None else torch.empty(q.shape, dtype=torch.float32,
                                                                             device=q.device)
        sel = lay[5] if len(lay) > 5 and lay[5] is not None else torch.empty(
            (q.shape[0], q.shape[1], budgets[-1]), dtype=torch.int32, device=q.device)
        full.append((q, pyr, k, v, out, sel))
    arr = _layer_array(full, gen_idx, budgets)
    q0, p0, k0_ = full[0][:3]
    n_gen = 0 if gen_idx is None else gen_idx.numel()
    barr = _budget_array(budgets)
    need = int(lib().wf_select_attend_layers_workspace_bytes(ctypes.byref(p0.desc), len(full), q0.shape[2], n_gen,
                                                             barr))
    if need == 0:
        raise WfError(-5, "wf_select_attend_layers_workspace_bytes")
    if workspace is None:
        workspace = default_workspace(q0.device)
    ws = workspace.get(need)
    st = lib().wf_select_attend_layers(arr, len(full), k0_.shape[2],
                                       ctypes.c_void_p(0 if gen_idx is None else gen_idx.data_ptr()), n_gen, barr,
                                       q0.shape[2], _agg_code(agg, check), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                       _stream_handle(q0.device))
    if st != WF_OK:
        raise WfError(st, "wf_select_attend_layers")
    return [{"out": f[4], "sel": f[5]} for f in full]


class PreparedLayers:
    """A batched select-attend call over several layers, marshalled once."""

    def __init__(self, layers, gen_idx, budgets, workspace, agg="max", check=False):
        budgets = [int(b) for b in budgets]
        self._arr = _layer_array(layers, gen_idx, budgets)
        q0, p0, k0_ = layers[0][:3]
        n_gen = 0 if gen_idx is None else gen_idx.numel()
        self._barr = _budget_array(budgets)
        need = int(lib().wf_select_attend_layers_workspace_bytes(ctypes.byref(p0.desc), len(layers), q0.shape[2],
                                                                 n_gen, self._barr))
        if need == 0:
            raise WfError(-5, "PreparedLayers")
        _check_workspace(workspace, q0.device, need)
        self._keep = (layers, gen_idx, workspace)
        self._args = (self._arr, len(layers), k0_.shape[2], ctypes.c_void_p(0 if gen_idx is None else gen_idx.data_ptr()),
                      n_gen, self._barr, q0.shape[2], _agg_code(agg, check), ctypes.c_void_p(workspace.data_ptr()),
                      workspace.numel(), _stream_handle(q0.device))
        self._fn = lib().wf_select_attend_layers

    def __call__(self):
        st = self._fn(*self._args)
        if st != WF_OK:
            raise WfError(st, "wf_select_attend_layers")


class PreparedBuild:
    """A pyramid build with its arguments marshalled once."""

    def __init__(self, k, n_prompt, levels, buf, flags=0):
        B, H, N, d = k.shape
        self.desc = WfPyramid()
        self._keep = (k, buf)
        self._args = (ctypes.c_void_p(k.data_ptr()), N * d, B, H, n_prompt, d, _dtype_code(k), levels, flags,
                      ctypes.c_void_p(buf.data_ptr()), buf.numel(), ctypes.byref(self.desc), _stream_handle(k.device))
        self._fn = lib().wf_build_pyramid
        self.pyramid = Pyramid(buf, self.desc)

    def __call__(self):
        st = self._fn(*self._args)
        if st != WF_OK:
            raise WfError(st, "wf_build_pyramid")
        return self.pyramid
