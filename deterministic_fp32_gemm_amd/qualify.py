"""Vendor-BLAS qualification probe (diagnostic): does a vendor strided-batched SGEMM with beta = 1 give the fixed
chain's bits for this update?

The page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_gemm_cuda.py" (its cuBLAS qualification:
matches_cublas and the probe patterns) routes shapes to the vendor BLAS only after checking, pattern by pattern and
alignment class by alignment class, that the library reproduces the chain bit for bit. This module runs the same
question on MI355X against two vendor paths:

  * "rocblas": rocblas_sgemm_strided_batched called directly (column-major: d_u^T = d_dv^T * x, beta = 1);
  * "torch":   torch.baddbmm(d_u, x^T, d_dv) in FP32 (whatever BLAS torch dispatches to on ROCm).

The reference is this library's own update (sdm_gx_gemm_steps), which runs the chain exactly. The report says
"equal" or "differ" per case, with the number of differing outputs and the largest difference in units in the last
place among finite outputs. Differences are expected wherever the BLAS sums in another order (MFMA K > 1 tiles,
split-K): that is why the update keeps its own kernels. Nothing here feeds the update; it is a diagnostic.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from . import _binding as B
from . import inputs

_ROCBLAS_OPERATION_NONE = 111
_ROCBLAS_OPERATION_TRANSPOSE = 112

_rocblas = None


def _rocblas_lib():
    global _rocblas
    if _rocblas is None:
        path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "librocblas.so")
        lib = ctypes.CDLL(path)
        lib.rocblas_create_handle.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        lib.rocblas_destroy_handle.argtypes = [ctypes.c_void_p]
        lib.rocblas_set_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        lib.rocblas_sgemm_strided_batched.argtypes = [vp, ctypes.c_int, ctypes.c_int, i32, i32, i32,
                                                      ctypes.POINTER(ctypes.c_float), vp, i32, i64, vp, i32, i64,
                                                      ctypes.POINTER(ctypes.c_float), vp, i32, i64, i32]
        lib.rocblas_get_version_string.argtypes = [ctypes.c_char_p, ctypes.c_size_t]
        _rocblas = lib
    return _rocblas


def rocblas_version() -> str:
    buf = ctypes.create_string_buffer(256)
    _rocblas_lib().rocblas_get_version_string(buf, 256)
    return buf.value.decode()


def rocblas_update(d_u, ld_u, x, d_dv, ld_dv, n_begin, nchunks, C, hd, stream=None) -> None:
    """d_u[n] += x[n]^T d_dv[n] for chunks n_begin .. n_begin + nchunks - 1 with rocblas_sgemm_strided_batched.

    Row-major d_u[n] (C x hd, stride ld_u) is column-major (hd x C, ld ld_u); so is d_dv[n]; row-major x[n] (C x C)
    read column-major is x[n]^T. Hence d_u^T (hd x C) = d_dv^T (hd x C) * (x^T)^T with op(B) = transpose."""
    lib = _rocblas_lib()
    handle = ctypes.c_void_p()
    if lib.rocblas_create_handle(ctypes.byref(handle)) != 0:
        raise RuntimeError("rocblas_create_handle failed")
    try:
        if lib.rocblas_set_stream(handle, B._stream(stream)) != 0:
            raise RuntimeError("rocblas_set_stream failed")
        one = ctypes.c_float(1.0)
        du0 = B._ptr(d_u, "d_u") + 4 * n_begin * C * ld_u
        dv0 = B._ptr(d_dv, "d_dv") + 4 * n_begin * C * ld_dv
        x0 = B._ptr(x, "x") + 4 * n_begin * C * C
        st = lib.rocblas_sgemm_strided_batched(handle, _ROCBLAS_OPERATION_NONE, _ROCBLAS_OPERATION_TRANSPOSE,
                                               int(hd), int(C), int(C), ctypes.byref(one),
                                               dv0, int(ld_dv), int(C * ld_dv), x0, int(C), int(C * C),
                                               ctypes.byref(one), du0, int(ld_u), int(C * ld_u), int(nchunks))
        if st != 0:
            raise RuntimeError(f"rocblas_sgemm_strided_batched failed with status {st}")
    finally:
        lib.rocblas_destroy_handle(handle)


def _ulp_gap(a: np.ndarray, b: np.ndarray) -> int:
    """Largest distance in units in the last place between finite entries (0 if none differ)."""
    fin = np.isfinite(a) & np.isfinite(b)
    if not fin.any():
        return 0
    ia = a[fin].view(np.int32).astype(np.int64)
    ib = b[fin].view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)       # monotone integer line through +-0
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return int(np.abs(ia - ib).max())


def compare(got: np.ndarray, ref: np.ndarray) -> dict:
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    return {"outputs": int(same.size), "differ": int((~same).sum()), "max_ulp": _ulp_gap(got, ref),
            "verdict": "equal" if same.all() else "differ"}


DEFAULT_CASES = (  # (C, hd, ld, residue bytes of d_u / d_dv)
    (64, 64, 64, 0), (64, 128, 128, 0), (128, 128, 128, 0), (64, 256, 260, 4), (37, 150, 157, 12), (16, 16, 16, 8),
)


def qualify(cases=DEFAULT_CASES, patterns=None, backends=("rocblas", "torch"), N=8, P=8, seed=7) -> list:
    """Run every backend and this library's chain on the same inputs; one report row per (case, pattern, backend).
    Needs a GPU; inputs are seeded and synthetic (the generators of `inputs`)."""
    import torch

    from .step import aligned_empty

    patterns = patterns or (inputs.PATTERNS + inputs.HAZARD_PATTERNS)
    rows = []
    for C, hd, ld, res in cases:
        for pattern in patterns:
            x_h, dv_h, du_h = inputs.shape_inputs(N, C, hd, ld, pattern, seed=seed + C + hd + res)
            outs = {}
            for who in ("chain",) + tuple(backends):
                x = aligned_empty(x_h.size, 0)
                dv = aligned_empty(dv_h.size, res)
                du = aligned_empty(du_h.size, res)
                x.copy_(torch.from_numpy(x_h.reshape(-1)))
                dv.copy_(torch.from_numpy(dv_h.reshape(-1)))
                du.copy_(torch.from_numpy(du_h.reshape(-1)))
                if who == "chain":
                    B.sdm_gx_gemm_steps(du, ld, x, dv, ld, N, P, C, hd, 0, N // P, B.SDM_GX_STEPS_FUSED)
                elif who == "rocblas":
                    rocblas_update(du, ld, x, dv, ld, 0, (N // P) * P, C, hd)
                elif who == "torch":
                    x3 = x.view(N, C, C).transpose(1, 2).contiguous()
                    du3 = du.view(N, C, ld)[:, :, :hd]
                    dv3 = dv.view(N, C, ld)[:, :, :hd]
                    du3.copy_(torch.baddbmm(du3, x3, dv3))
                else:
                    raise ValueError(f"unknown backend {who}")
                torch.cuda.synchronize()
                outs[who] = du.cpu().numpy().reshape(N, C, ld)[:, :, :hd].copy()
            for who in backends:
                rows.append(dict(C=C, hd=hd, ld=ld, residue=res, pattern=pattern, backend=who,
                                 **compare(outs[who], outs["chain"])))
    return rows


if __name__ == "__main__":
    import json
    for row in qualify():
        print(json.dumps(row), flush=True)
