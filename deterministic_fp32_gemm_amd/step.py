"""Per-backward step factory over the prepared-launch entry points (the page's make_step: validate once, then one
launch per step with only ti changed), and the device-memory helper used to place operands at a chosen alignment."""

from __future__ import annotations

from . import _binding as B


def tensor_layout(d_u, x, d_dv):
    """(N, C, hd, ld_u, ld_dv) from torch tensors: x [N, C, C] contiguous; d_u [N, C, hd] with unit column stride and
    row stride ld_u (chunk stride C*ld_u); d_dv the same as d_u, or a 2-D [N*C, hd] view."""
    if x.dim() != 3 or x.shape[1] != x.shape[2] or not x.is_contiguous():
        raise ValueError("x must be a contiguous [N, C, C] tensor")
    N, C = int(x.shape[0]), int(x.shape[1])
    if d_u.dim() != 3 or tuple(d_u.shape[:2]) != (N, C) or d_u.stride(2) != 1 or d_u.stride(0) != C * d_u.stride(1):
        raise ValueError("d_u must be [N, C, hd] with unit column stride and rows of a fixed stride")
    hd, ld_u = int(d_u.shape[2]), int(d_u.stride(1))
    if d_dv.dim() == 2:
        if tuple(d_dv.shape) != (N * C, hd) or d_dv.stride(1) != 1:
            raise ValueError("d_dv must be [N*C, hd] (or [N, C, hd]) like d_u")
        ld_dv = int(d_dv.stride(0))
    elif d_dv.dim() == 3:
        if tuple(d_dv.shape) != (N, C, hd) or d_dv.stride(2) != 1 or d_dv.stride(0) != C * d_dv.stride(1):
            raise ValueError("d_dv must be [N, C, hd] like d_u")
        ld_dv = int(d_dv.stride(1))
    else:
        raise ValueError("d_dv must be 2-D or 3-D")
    return N, C, hd, ld_u, ld_dv


def make_step(d_u, x, d_dv, P: int, plan=None):
    """step(ti, stream=None) for 0 <= ti < N // P, plus step.fused(ti_begin, ti_end) (one launch for a range of
    steps), step.graph(ti_begin, ti_end, mode) (a replayable HIP graph of that range), step.prepared (the
    sdm_gx_launch_t) and step.geom (the plans). Everything is validated here, once."""
    N, C, hd, ld_u, ld_dv = tensor_layout(d_u, x, d_dv)
    P = int(P)
    if not 1 <= P <= N:
        raise ValueError(f"need 1 <= P <= N chunks; got P {P}, N {N}")
    lim = N // P
    prepared = B.sdm_gx_prepare(d_u, ld_u, x, d_dv, ld_dv, N, P, C, hd, lim - 1, plan)
    keep = (d_u, x, d_dv)            # the prepared launch holds their addresses

    def step(ti: int, stream=None) -> None:
        if not 0 <= int(ti) < lim:
            raise ValueError(f"step {ti} outside [0, {lim})")
        B.sdm_gx_launch(prepared, int(ti), stream)

    def fused(ti_begin: int, ti_end: int, stream=None) -> None:
        B.sdm_gx_launch_fused(prepared, int(ti_begin), int(ti_end), stream)

    def graph(ti_begin: int = 0, ti_end: int = lim, mode=B.SDM_GX_STEPS_FUSED) -> B.Graph:
        """A HIP graph of steps ti_begin .. ti_end - 1 (per-step nodes or the fused launch), replayed with .launch()."""
        return B.Graph(prepared, ti_begin, ti_end, mode)

    step.fused = fused
    step.graph = graph
    step.prepared = prepared
    step.steps = lim
    step.geom = dict(step=prepared.plan_step.as_dict(), fused=prepared.plan_fused.as_dict())
    step._keep = keep
    return step


def aligned_empty(nfloats: int, residue_bytes: int = 0, device="cuda"):
    """A float32 device tensor of nfloats elements whose address is residue_bytes past a 256-byte boundary
    (residue_bytes a multiple of 4). The returned view keeps its backing allocation alive."""
    import torch
    if residue_bytes % 4 or not 0 <= residue_bytes < 256:
        raise ValueError("residue_bytes: a multiple of 4 in [0, 256)")
    buf = torch.empty(int(nfloats) + 128, dtype=torch.float32, device=device)
    off = ((residue_bytes - buf.data_ptr()) % 256) // 4
    return buf[off:off + int(nfloats)]
