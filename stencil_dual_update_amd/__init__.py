"""MI355X (gfx950) FGP step on the 3D total-variation dual.

The computation runs in hand-written HIP kernels in ``libtvfgp.so`` behind a
C ABI (``include/tv_fgp.h``); this package is its Python binding.  torch
tensors provide device memory and streams.  See ``_lib`` for the entry
points: ``tv_fgp_step``, ``tv_fgp_run``, ``tv_primal``, ``tv_fgp_duality_gap``,
``tv_fgp_solve``.
"""
from ._lib import (  # noqa: F401
    EXPORTS, CUBE, FUSED, LDS_MARCH, PAIR, POINT, REG_MARCH, TB2, TB3, TWO_KERNEL, VARIANTS,
    LIB_PATH,
    TV_ERR_ALIAS, TV_ERR_ALIGN, TV_ERR_DIMS, TV_ERR_LAUNCH, TV_ERR_NULL,
    TV_ERR_PARAM, TV_ERR_VARIANT, TV_ERR_WORKSPACE, TV_OK, TvFgpError, lib,
    gap_workspace_bytes, momentum, status_string, tv_fgp_duality_gap,
    tv_fgp_duality_gap_noalloc, tv_fgp_run, tv_fgp_run_pp,
    tv_fgp_run_h, tv_fgp_run2_h, tv_fgp_solve, tv_fgp_step, tv_fgp_step2, tv_fgp_step2_h,
    tv_fgp_step3, tv_fgp_step_h, tv_fgp_step_march, tv_fgp_stream_probe,
    tv_fgp_stream_probe_ex, STREAM_SHAPES, tv_primal,
    tv_primal_h, MARCH_SHAPES,
    variant_name, workspace_bytes)
