"""Deterministic FP32 per-step d_u update for MI355X (gfx950): Python binding of libsdm_gx_gemm.

The operation (page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_gemm_cuda.py", module docstring): for
every chunk n = ti*P + p of step ti, row i < C and column c < hd, d_u[n, i, c] += acc with
acc = fmaf(x[n, j, i], d_dv[n, j, c], acc) over j = 0..C-1 from +0 and one separately rounded add. Phase A, the
consumer of the updated d_u (page "... gx_pa2_cuda.py", gx_pa2_kernel), is in the same library. The C ABI is in
include/sdm_gx_gemm.h and include/sdm_gx_pa2.h; the functions below carry the same names and only marshal arguments.
"""

from ._binding import (  # noqa: F401
    EXPORTS,
    SDM_GX_ENGINE_MFMA,
    SDM_GX_ENGINE_VALU,
    SDM_GX_ERR_ALIGN,
    SDM_GX_ERR_ARG,
    SDM_GX_ERR_DEVICE,
    SDM_GX_ERR_HIP,
    SDM_GX_ERR_LIMIT,
    SDM_GX_ERR_NULL,
    SDM_GX_ERR_OVERLAP,
    SDM_GX_ERR_PLAN,
    SDM_GX_ERR_SHAPE,
    SDM_GX_ERR_STEP,
    SDM_GX_ERR_STRIDE,
    SDM_GX_OK,
    SDM_GX_STEPS_FORWARD,
    SDM_GX_STEPS_FUSED,
    SDM_GX_STEPS_REVERSE,
    Graph,
    load,
    make_mfma_plan,
    make_plan,
    sdm_gx_abi_version,
    sdm_gx_check,
    sdm_gx_gemm,
    sdm_gx_gemm_ex,
    sdm_gx_gemm_steps,
    sdm_gx_graph_create,
    sdm_gx_graph_destroy,
    sdm_gx_graph_launch,
    sdm_gx_graph_nodes,
    sdm_gx_kernel_attrs,
    sdm_gx_last_hip_error,
    sdm_gx_launch,
    sdm_gx_launch_fused,
    sdm_gx_launch_t,
    sdm_gx_plan,
    sdm_gx_plan_complete,
    sdm_gx_plan_for,
    sdm_gx_plan_t,
    sdm_gx_prepare,
    sdm_gx_strerror,
    make_pa2_plan,
    pa2_args,
    sdm_pa2_args_t,
    sdm_pa2_check,
    sdm_pa2_plan_for,
    sdm_pa2_plan_t,
    sdm_pa2_step,
    sdm_pa2_steps,
)
from .step import make_step, tensor_layout  # noqa: F401
