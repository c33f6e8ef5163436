"""WaveFilter per-step sparse attention for AMD Instinct MI355X (gfx950).

The work runs in ``libwavefilter.so`` (hand-written HIP, C ABI declared in
``include/wavefilter.h``); this package only marshals arguments to it.
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    MAX_LEVELS,
    MAX_LAYER_ITEMS,
    MAX_QUERIES,
    WF_AGG_MAX,
    WF_AGG_MEAN,
    WF_BF16,
    WF_F32,
    WF_PYR_ALL_LEVELS,
    WF_PYR_DB2,
    WF_OPT_CHECK,
    CHECK_BITS,
    Pyramid,
    PreparedAttend,
    PreparedBuild,
    PreparedLayers,
    PreparedRefresh,
    PreparedStep,
    WfError,
    Workspace,
    attend_selected,
    attend_selected_workspace_bytes,
    build_pyramid,
    check_status,
    lib,
    pyramid_bytes,
    refresh_pyramids,
    select_attend,
    select_attend_layers,
    layers_workspace_bytes,
    select_attend_noalloc,
    split_levels,
    status_string,
    version,
    workspace_bytes,
)
