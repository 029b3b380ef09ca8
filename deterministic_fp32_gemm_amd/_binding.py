"""ctypes binding of libsdm_gx_gemm (include/sdm_gx_gemm.h): the same names, argument marshalling only.

Tensor arguments may be torch tensors (their data_ptr() is passed; they must be float32 CUDA/HIP tensors with
materialised values) or plain integers (device addresses). ``stream=None`` means torch's current stream on the
current device. A non-zero status raises: ValueError for argument errors, RuntimeError for device / HIP errors.
Every step of the update runs in the library's HIP kernels; nothing here computes.
"""

from __future__ import annotations

import ctypes
import os
import threading

from ._build import LIB_PATH

SDM_GX_OK = 0
SDM_GX_ERR_NULL = -1
SDM_GX_ERR_SHAPE = -2
SDM_GX_ERR_STEP = -3
SDM_GX_ERR_ALIGN = -4
SDM_GX_ERR_OVERLAP = -5
SDM_GX_ERR_STRIDE = -6
SDM_GX_ERR_LIMIT = -7
SDM_GX_ERR_HIP = -8
SDM_GX_ERR_PLAN = -9
SDM_GX_ERR_DEVICE = -10
SDM_GX_ERR_ARG = -11

SDM_GX_ENGINE_VALU = 0
SDM_GX_ENGINE_MFMA = 1

SDM_GX_STEPS_FORWARD = 0
SDM_GX_STEPS_REVERSE = 1
SDM_GX_STEPS_FUSED = 2

_ARG_ERRORS = {SDM_GX_ERR_NULL, SDM_GX_ERR_SHAPE, SDM_GX_ERR_STEP, SDM_GX_ERR_ALIGN, SDM_GX_ERR_OVERLAP,
               SDM_GX_ERR_STRIDE, SDM_GX_ERR_PLAN, SDM_GX_ERR_ARG}


class sdm_gx_plan_t(ctypes.Structure):
    _fields_ = [("engine", ctypes.c_int32),
                ("rows_per_wave", ctypes.c_int32), ("cols_per_lane", ctypes.c_int32),
                ("waves_per_wg", ctypes.c_int32), ("staging", ctypes.c_int32), ("xcd_remap", ctypes.c_int32),
                ("slab_rows", ctypes.c_int32),
                ("mf_row_waves", ctypes.c_int32), ("mf_col_waves", ctypes.c_int32), ("mf_stages", ctypes.c_int32),
                ("mf_reg_slabs", ctypes.c_int32), ("mf_loader_waves", ctypes.c_int32),
                ("mf_workgroups", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("wgs_per_cu", ctypes.c_int32), ("mf_du_at_end", ctypes.c_int32),
                ("mf_block", ctypes.c_int32), ("mf_stream_du", ctypes.c_int32), ("mf_aln", ctypes.c_int32),
                ("grid", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}

    def __repr__(self):
        return "sdm_gx_plan_t(" + ", ".join(f"{k}={v}" for k, v in self.as_dict().items()) + ")"


class sdm_gx_launch_t(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint64), ("device", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("d_u", ctypes.c_void_p), ("x", ctypes.c_void_p), ("d_dv", ctypes.c_void_p),
                ("ld_u", ctypes.c_int64), ("ld_dv", ctypes.c_int64), ("N", ctypes.c_int64), ("P", ctypes.c_int64),
                ("C", ctypes.c_int64), ("hd", ctypes.c_int64), ("ti_max", ctypes.c_int64),
                ("plan_step", sdm_gx_plan_t), ("plan_fused", sdm_gx_plan_t)]


class sdm_pa2_args_t(ctypes.Structure):
    _fields_ = [("grad", ctypes.c_void_p), ("bank", ctypes.c_void_p), ("slots", ctypes.c_int64),
                ("snap", ctypes.c_void_p), ("snap_rows", ctypes.c_int64), ("ssr", ctypes.c_int64),
                ("d_u", ctypes.c_void_p), ("ld_u", ctypes.c_int64), ("beta", ctypes.c_void_p),
                ("kpay", ctypes.c_void_p), ("rec", ctypes.c_void_p), ("bpre", ctypes.c_void_p),
                ("out_eff", ctypes.c_void_p), ("out_g", ctypes.c_void_p), ("plane", ctypes.c_int64),
                ("planes", ctypes.c_int64), ("N", ctypes.c_int64), ("P", ctypes.c_int64), ("C", ctypes.c_int64),
                ("W", ctypes.c_int64), ("hd", ctypes.c_int64)]


class sdm_pa2_plan_t(ctypes.Structure):
    _fields_ = [("slices_per_wave", ctypes.c_int32), ("waves_per_wg", ctypes.c_int32), ("tile_len", ctypes.c_int32),
                ("ctas", ctypes.c_int32), ("npair", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("stage_out", ctypes.c_int32), ("grid", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


EXPORTS = ("sdm_gx_gemm", "sdm_gx_gemm_ex", "sdm_gx_gemm_steps", "sdm_gx_check", "sdm_gx_plan", "sdm_gx_plan_for",
           "sdm_gx_plan_complete", "sdm_gx_prepare", "sdm_gx_launch", "sdm_gx_launch_fused", "sdm_gx_graph_create",
           "sdm_gx_graph_launch", "sdm_gx_graph_nodes", "sdm_gx_graph_destroy", "sdm_gx_kernel_attrs",
           "sdm_gx_strerror", "sdm_gx_last_hip_error", "sdm_gx_abi_version",
           "sdm_pa2_check", "sdm_pa2_plan_for", "sdm_pa2_step", "sdm_pa2_steps")

_lib = None
_lock = threading.Lock()
_i64, _i32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
_PP = ctypes.POINTER(sdm_gx_plan_t)
_LP = ctypes.POINTER(sdm_gx_launch_t)
_AP = ctypes.POINTER(sdm_pa2_args_t)
_QP = ctypes.POINTER(sdm_pa2_plan_t)


def lib_path() -> str:
    return os.environ.get("SDM_GX_LIB", LIB_PATH)


def load() -> ctypes.CDLL:
    """Load the HIP library (once). Fails loudly if it has not been built: there is no fallback path."""
    global _lib
    if _lib is not None:                # loaded: no lock on the launch path
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(path)
        sig = {
            "sdm_gx_gemm": [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp],
            "sdm_gx_gemm_ex": [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _PP, _vp],
            "sdm_gx_gemm_steps": [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i32, _PP, _vp],
            "sdm_gx_check": [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64],
            "sdm_gx_plan": [_i64, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _PP],
            "sdm_gx_plan_for": [_i64, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _i32, _PP],
            "sdm_gx_plan_complete": [_PP, _i64, _i64, _i64, _i64, _i64, _i32, _i32, _i32],
            "sdm_gx_prepare": [_LP, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _PP],
            "sdm_gx_launch": [_LP, _i64, _vp],
            "sdm_gx_launch_fused": [_LP, _i64, _i64, _vp],
            "sdm_gx_kernel_attrs": [_PP, ctypes.POINTER(ctypes.c_int64)],
            "sdm_gx_strerror": [ctypes.c_int],
            "sdm_gx_last_hip_error": [],
            "sdm_gx_abi_version": [],
            "sdm_gx_graph_create": [ctypes.POINTER(_vp), _LP, _i64, _i64, _i32],
            "sdm_gx_graph_launch": [_vp, _vp],
            "sdm_gx_graph_nodes": [_vp],
            "sdm_gx_graph_destroy": [_vp],
            "sdm_pa2_check": [_AP, _i64],
            "sdm_pa2_plan_for": [_AP, _i32, _i32, _QP],
            "sdm_pa2_step": [_AP, _i64, _QP, _vp],
            "sdm_pa2_steps": [_AP, _i64, _i64, _i32, _QP, _vp],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = {"sdm_gx_strerror": ctypes.c_char_p, "sdm_gx_graph_nodes": ctypes.c_int64}.get(name, ctypes.c_int)
        _lib = lib
        return lib


# ---- marshalling helpers --------------------------------------------------------------------------------------------
def _ptr(t, name: str) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: a torch tensor or a device address")
    if t.dtype != torch.float32:
        raise TypeError(f"{name}: float32 required, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if t.is_neg() or t.is_conj():
        raise ValueError(f"{name}: lazy negative / conjugate views are not supported (materialise them first)")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream           # a torch.cuda.Stream


def _raise(code: int, what: str):
    if code == SDM_GX_OK:
        return
    msg = load().sdm_gx_strerror(code).decode()
    if code == SDM_GX_ERR_HIP:
        msg += f" (hipError {load().sdm_gx_last_hip_error()})"
    exc = ValueError if code in _ARG_ERRORS else RuntimeError
    raise exc(f"{what}: {msg} [status {code}]")


def _plan_ptr(plan):
    if plan is None:
        return None
    if not isinstance(plan, sdm_gx_plan_t):
        raise TypeError("plan: an sdm_gx_plan_t")
    return ctypes.byref(plan)


def strerror(code: int) -> str:
    return load().sdm_gx_strerror(int(code)).decode()


# ---- entry points (same names as the C ABI) ---------------------------------------------------------------------------
def sdm_gx_gemm(d_u, x, d_dv, ti, P, C, hd, stream=None) -> None:
    _raise(load().sdm_gx_gemm(_ptr(d_u, "d_u"), _ptr(x, "x"), _ptr(d_dv, "d_dv"), int(ti), int(P), int(C), int(hd),
                              _stream(stream)), "sdm_gx_gemm")


def sdm_gx_gemm_ex(d_u, ld_u, x, d_dv, ld_dv, N, ti, P, C, hd, plan=None, stream=None) -> None:
    _raise(load().sdm_gx_gemm_ex(_ptr(d_u, "d_u"), int(ld_u), _ptr(x, "x"), _ptr(d_dv, "d_dv"), int(ld_dv), int(N),
                                 int(ti), int(P), int(C), int(hd), _plan_ptr(plan), _stream(stream)), "sdm_gx_gemm_ex")


def sdm_gx_gemm_steps(d_u, ld_u, x, d_dv, ld_dv, N, P, C, hd, ti_begin, ti_end, mode=SDM_GX_STEPS_FORWARD,
                      plan=None, stream=None) -> None:
    _raise(load().sdm_gx_gemm_steps(_ptr(d_u, "d_u"), int(ld_u), _ptr(x, "x"), _ptr(d_dv, "d_dv"), int(ld_dv),
                                    int(N), int(P), int(C), int(hd), int(ti_begin), int(ti_end), int(mode),
                                    _plan_ptr(plan), _stream(stream)), "sdm_gx_gemm_steps")


def sdm_gx_check(d_u, ld_u, x, d_dv, ld_dv, N, ti, P, C, hd) -> int:
    """The status code (no exception): argument checks only, no device access. Pointers may be plain integers."""
    return load().sdm_gx_check(_ptr(d_u, "d_u"), int(ld_u), _ptr(x, "x"), _ptr(d_dv, "d_dv"), int(ld_dv), int(N),
                               int(ti), int(P), int(C), int(hd))


def sdm_gx_plan(nchunks, C, hd, ld_u=None, ld_dv=None, x_mod16=0, dv_mod16=0, engine=-1, device=-1) -> sdm_gx_plan_t:
    """The plan a launch with these strides (default: hd) and placements (address mod 16 of x and d_dv) runs."""
    p = sdm_gx_plan_t()
    _raise(load().sdm_gx_plan(int(nchunks), int(C), int(hd), int(hd if ld_u is None else ld_u),
                              int(hd if ld_dv is None else ld_dv), int(x_mod16), int(dv_mod16), int(engine),
                              int(device), ctypes.byref(p)), "sdm_gx_plan")
    return p


def sdm_gx_plan_for(nchunks, C, hd, num_cus=256, lds_per_cu=160 * 1024, ld_u=None, ld_dv=None, x_mod16=0,
                    dv_mod16=0, engine=-1) -> sdm_gx_plan_t:
    p = sdm_gx_plan_t()
    _raise(load().sdm_gx_plan_for(int(nchunks), int(C), int(hd), int(hd if ld_u is None else ld_u),
                                  int(hd if ld_dv is None else ld_dv), int(x_mod16), int(dv_mod16), int(engine),
                                  int(num_cus), int(lds_per_cu), ctypes.byref(p)), "sdm_gx_plan_for")
    return p


def make_plan(rows_per_wave, cols_per_lane, waves_per_wg, staging=0, xcd_remap=0, slab_rows=0) -> sdm_gx_plan_t:
    """A caller-made plan for the vector-ALU engine (validated by the entry point that receives it)."""
    p = sdm_gx_plan_t()
    p.engine = SDM_GX_ENGINE_VALU
    p.rows_per_wave, p.cols_per_lane, p.waves_per_wg = rows_per_wave, cols_per_lane, waves_per_wg
    p.staging, p.xcd_remap, p.slab_rows = staging, xcd_remap, slab_rows
    return p


def make_mfma_plan(row_waves, col_waves, stages=4, reg_slabs=4, loader_waves=4, workgroups=0,
                   du_at_end=0, block=32, slab_rows=0, stream_du=0) -> sdm_gx_plan_t:
    """A caller-made plan for the matrix-core engine (validated by the entry point that receives it)."""
    p = sdm_gx_plan_t()
    p.engine = SDM_GX_ENGINE_MFMA
    p.mf_row_waves, p.mf_col_waves, p.mf_stages = row_waves, col_waves, stages
    p.mf_reg_slabs, p.mf_loader_waves, p.mf_workgroups = reg_slabs, loader_waves, workgroups
    p.mf_du_at_end, p.mf_block, p.slab_rows, p.mf_stream_du = du_at_end, block, slab_rows, stream_du
    return p


def sdm_gx_plan_complete(plan: sdm_gx_plan_t, nchunks, C, hd, lds_per_cu=160 * 1024, ld_u=None, ld_dv=None,
                         x_mod16=0, dv_mod16=0) -> sdm_gx_plan_t:
    _raise(load().sdm_gx_plan_complete(ctypes.byref(plan), int(nchunks), int(C), int(hd),
                                       int(hd if ld_u is None else ld_u), int(hd if ld_dv is None else ld_dv),
                                       int(x_mod16), int(dv_mod16), int(lds_per_cu)), "sdm_gx_plan_complete")
    return plan


def sdm_gx_prepare(d_u, ld_u, x, d_dv, ld_dv, N, P, C, hd, ti_max, plan=None) -> sdm_gx_launch_t:
    out = sdm_gx_launch_t()
    _raise(load().sdm_gx_prepare(ctypes.byref(out), _ptr(d_u, "d_u"), int(ld_u), _ptr(x, "x"), _ptr(d_dv, "d_dv"),
                                 int(ld_dv), int(N), int(P), int(C), int(hd), int(ti_max), _plan_ptr(plan)),
           "sdm_gx_prepare")
    return out


def sdm_gx_launch(prepared: sdm_gx_launch_t, ti, stream=None) -> None:
    _raise(load().sdm_gx_launch(ctypes.byref(prepared), int(ti), _stream(stream)), "sdm_gx_launch")


def sdm_gx_launch_fused(prepared: sdm_gx_launch_t, ti_begin, ti_end, stream=None) -> None:
    _raise(load().sdm_gx_launch_fused(ctypes.byref(prepared), int(ti_begin), int(ti_end), _stream(stream)),
           "sdm_gx_launch_fused")


class Graph:
    """A HIP graph of a prepared step range (sdm_gx_graph_create). launch(stream) replays it; close() (or garbage
    collection) releases it. Keeps the prepared launch it was built from alive."""

    def __init__(self, prepared: sdm_gx_launch_t, ti_begin, ti_end, mode=SDM_GX_STEPS_FUSED):
        self._h = ctypes.c_void_p()
        self._prepared = prepared
        _raise(load().sdm_gx_graph_create(ctypes.byref(self._h), ctypes.byref(prepared), int(ti_begin), int(ti_end),
                                          int(mode)), "sdm_gx_graph_create")

    @property
    def nodes(self) -> int:
        return int(load().sdm_gx_graph_nodes(self._h)) if self._h else -1

    def launch(self, stream=None) -> None:
        if not self._h:
            raise ValueError("graph already closed")
        _raise(load().sdm_gx_graph_launch(self._h, _stream(stream)), "sdm_gx_graph_launch")

    def close(self) -> None:
        if self._h:
            h, self._h = self._h, ctypes.c_void_p()
            _raise(load().sdm_gx_graph_destroy(h), "sdm_gx_graph_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def sdm_gx_graph_create(prepared: sdm_gx_launch_t, ti_begin, ti_end, mode=SDM_GX_STEPS_FUSED) -> Graph:
    return Graph(prepared, ti_begin, ti_end, mode)


def sdm_gx_graph_launch(graph: Graph, stream=None) -> None:
    graph.launch(stream)


def sdm_gx_graph_nodes(graph: Graph) -> int:
    return graph.nodes


def sdm_gx_graph_destroy(graph: Graph) -> None:
    graph.close()


def sdm_gx_kernel_attrs(plan: sdm_gx_plan_t) -> dict:
    out = (ctypes.c_int64 * 5)()
    _raise(load().sdm_gx_kernel_attrs(ctypes.byref(plan), out), "sdm_gx_kernel_attrs")
    return dict(vgprs=out[0], scratch_bytes=out[1], static_lds=out[2], max_threads=out[3], dynamic_lds=out[4])


def sdm_gx_strerror(code: int) -> str:
    return strerror(code)


def sdm_gx_last_hip_error() -> int:
    return load().sdm_gx_last_hip_error()


def sdm_gx_abi_version() -> int:
    return load().sdm_gx_abi_version()


# ---- Phase A (sdm_gx_pa2.h) ---------------------------------------------------------------------------------------------
def _iptr(t, name: str) -> int:
    """Device address of an int32 tensor (or a plain integer)."""
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or not t.is_cuda:
        raise TypeError(f"{name}: an int32 GPU tensor or a device address")
    return t.data_ptr()


def pa2_args(grad, bank, snap, ssr, d_u, beta, kpay, rec, bpre, out_eff, out_g, P, C, W, hd=None,
             ld_u=None) -> sdm_pa2_args_t:
    """An sdm_pa2_args_t from torch tensors: grad, bank [slots, hd]; snap [rows, hd]; d_u [N*C, ld_u] (a [N, C, hd]
    view with row stride ld_u also works); beta [N*C]; kpay [N, n], rec [N, n, 4], bpre [N, nb+1] int32 (bpre None
    for per-entry rows); out_eff, out_g [planes, plane]. Sizes are read from the tensors' shapes and strides."""
    a = sdm_pa2_args_t()
    hd = int(grad.shape[-1]) if hd is None else int(hd)
    a.grad, a.bank, a.snap = _ptr(grad, "grad"), _ptr(bank, "bank"), _ptr(snap, "snap")
    a.slots, a.snap_rows, a.ssr = int(grad.shape[0]), int(snap.numel() // max(1, int(snap.shape[-1]))), int(ssr)
    a.d_u, a.beta = _ptr(d_u, "d_u"), _ptr(beta, "beta")
    a.ld_u = int(ld_u if ld_u is not None else d_u.stride(-2))
    a.kpay, a.rec, a.bpre = _iptr(kpay, "kpay"), _iptr(rec, "rec"), _iptr(bpre, "bpre")
    a.out_eff, a.out_g = _ptr(out_eff, "out_eff"), _ptr(out_g, "out_g")
    a.planes, a.plane = int(out_eff.shape[0]), int(out_eff.shape[1])
    a.N, a.P, a.C, a.W, a.hd = int(kpay.shape[0]), int(P), int(C), int(W), hd
    return a


def make_pa2_plan(slices_per_wave, waves_per_wg, tile_len) -> sdm_pa2_plan_t:
    p = sdm_pa2_plan_t()
    p.slices_per_wave, p.waves_per_wg, p.tile_len = slices_per_wave, waves_per_wg, tile_len
    return p


def sdm_pa2_check(args: sdm_pa2_args_t, ti) -> int:
    """The status code (no exception); no device access."""
    return load().sdm_pa2_check(ctypes.byref(args), int(ti))


def sdm_pa2_plan_for(args: sdm_pa2_args_t, num_cus=256, lds_limit=160 * 1024) -> sdm_pa2_plan_t:
    p = sdm_pa2_plan_t()
    _raise(load().sdm_pa2_plan_for(ctypes.byref(args), int(num_cus), int(lds_limit), ctypes.byref(p)), "sdm_pa2_plan_for")
    return p


def sdm_pa2_step(args: sdm_pa2_args_t, ti, plan=None, stream=None) -> None:
    _raise(load().sdm_pa2_step(ctypes.byref(args), int(ti), ctypes.byref(plan) if plan is not None else None,
                               _stream(stream)), "sdm_pa2_step")


def sdm_pa2_steps(args: sdm_pa2_args_t, ti_begin, ti_end, mode=SDM_GX_STEPS_FORWARD, plan=None, stream=None) -> None:
    _raise(load().sdm_pa2_steps(ctypes.byref(args), int(ti_begin), int(ti_end), int(mode),
                                ctypes.byref(plan) if plan is not None else None, _stream(stream)), "sdm_pa2_steps")
