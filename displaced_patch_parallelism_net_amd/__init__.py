"""MI355X (gfx950) kernels for one device's share of a displaced-patch-parallel
diffusion denoising step.

The compute lives in libdpp.so (C ABI, include/dpp.h); `_lib` is its ctypes
binding (same names as the C entry points) and `step` sequences the calls of
one patch-layer step.  Importing the package fails if libdpp.so is missing.
"""
from ._lib import (  # noqa: F401
    DPP_BF16,
    DPP_F32,
    DppError,
    LIB_PATH,
    dpp_cfg_combine_relmae,
    dpp_cfg_combine_workspace_bytes,
    dpp_conv3x3_halo,
    dpp_conv3x3_halo_gn,
    dpp_conv3x3_halo_gn_chunks,
    dpp_conv3x3_halo_workspace_bytes,
    dpp_groupnorm_silu_stale,
    dpp_groupnorm_stale,
    dpp_groupnorm_stale_noalloc,
    dpp_groupnorm_stale_presummed,
    dpp_groupnorm_stale_workspace_bytes,
    dpp_hybrid_schedule,
    dpp_linear,
    dpp_linear_gn,
    dpp_linear_gn_chunks,
    dpp_self_attn_displaced,
    dpp_self_attn_workspace_bytes,
    dpp_splice_patch,
    dpp_strerror,
    dpp_version,
)
