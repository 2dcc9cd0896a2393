"""GDN token mixer for AMD Instinct MI355X: HIP kernels behind a C ABI (include/gdn.h).

The Python side is the ctypes binding in ``gdn`` (argument marshalling only).
"""
from .gdn import (  # noqa: F401
    GDN_BF16, GDN_F32, GDN_CONV, GDN_L2QK, GDN_NORM, GDN_GATE, GDN_ALL, EXPORTS, GdnError, gdn_cfg,
    load_library, gdn_cfg_default, gdn_abi_version, gdn_prefill_workspace, gdn_prefill,
    gdn_decode_step, gdn_set_stage_events, cfg_for, LIB_PATH, N_STAGES, STAGE_NAMES,
)
