"""Batched Muon optimizer step for AMD Instinct MI355X (gfx950).

The work runs in libdmuon.so (HIP kernels + a C ABI, see include/dmuon.h);
this package is its thin Python binding.  Build the library with
``python -m newton_schulz_08_amd.build``.
"""
from .api import (  # noqa: F401
    AdamWStep,
    MuonStep,
    adamw_step_,
    adamw_step_workspace_bytes,
    alloc_workspace,
    backend_info,
    plan_summary,
    clip_grad_norm_,
    clip_grad_norm_workspace_bytes,
    dtype_code,
    muon_step,
    muon_step_workspace_bytes,
    muon_step_clip_workspace_bytes,
    ns_batched,
    ns_config,
    ns_workspace_bytes,
    profile_enable,
    profile_read,
)
from ._lib import DmuonError, load  # noqa: F401
