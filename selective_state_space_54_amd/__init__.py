"""mssm: the Mamba selective scan as hand-written HIP kernels for MI355X (gfx950).

The compute path is libmssm.so (C ABI, declared in include/mssm.h); this
package holds its sources (csrc/), the build step (build.py) and a thin ctypes
binding (mssm.py) whose functions carry the C entry points' names.
"""
from .mssm import (  # noqa: F401
    MssmError,
    exported_symbols,
    load,
    mssm_abi_version,
    mssm_fused_supports,
    mssm_selective_ssm_fused_fwd,
    mssm_selective_ssm_fused_workspace_size,
    mssm_selective_scan_fwd,
    mssm_selective_scan_fwd_ex,
    mssm_selective_scan_fwd_ws,
    mssm_selective_scan_step,
    mssm_selective_scan_workspace_size,
    mssm_supports_state_size,
    selective_scan,
    selective_scan_ex,
    selective_scan_step,
    selective_ssm_fused,
)
