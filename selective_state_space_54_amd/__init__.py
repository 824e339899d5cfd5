"""mssm: the Mamba selective scan as hand-written HIP kernels for MI355X (gfx950).

The compute path is libmssm.so (C ABI, declared in include/mssm.h); this
package holds its sources (csrc/), the build step (build.py) and a thin ctypes
binding (mssm.py) whose functions carry the C entry points' names.
"""
from .mssm import (  # noqa: F401
    MssmError,
    causal_conv1d_silu,
    exported_symbols,
    load,
    mamba_block,
    mssm_abi_version,
    mssm_causal_conv1d_silu,
    mssm_fused_supports,
    mssm_mamba_block_fwd,
    mssm_mamba_block_supports,
    mssm_mamba_block_workspace_size,
    mssm_selective_ssm_fused_fwd,
    mssm_selective_ssm_fused_workspace_size,
    mssm_selective_scan_bwd,
    mssm_selective_scan_bwd_workspace_size,
    mssm_selective_scan_fwd,
    mssm_selective_scan_fwd_ex,
    mssm_selective_scan_fwd_ws,
    mssm_selective_scan_step,
    mssm_selective_scan_workspace_size,
    mssm_supports_state_size,
    selective_scan,
    selective_scan_bwd,
    selective_scan_ex,
    selective_scan_step,
    selective_ssm_fused,
)
