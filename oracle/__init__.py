"""CPU oracles of the deterministic backward step (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may import this package. It wraps two
plain C loops, and shares no code with the HIP library and imports nothing from it:
  * ``gx_gemm_oracle.c``: the per-step d_u update (plain ``fmaf`` in the fixed j order, then one separate add), which
    follows the page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_gemm_cuda.py", module docstring and
    the j-chain / epilogue of ``gx_gemm_kernel``;
  * ``gx_pa2_oracle.c``: Phase A, the consumer of the updated d_u (the record walk, group chains, per-lane dots and
    fixed-order butterfly of ``gx_pa2_kernel`` on the page "sparse-delta-memory 2.0.0 --
    sparse_delta_memory/cuda/gx_pa2_cuda.py"), for float32 rows.

Arrays are numpy float32 on the host:
  x    shape (N, C, C)            x[n, j, i]
  d_dv shape (N, C, ld_dv)        d_dv[n, j, c], columns c < hd used
  d_u  shape (N, C, ld_u)         updated in place for the chunks of the requested steps, columns c < hd
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gx_gemm_oracle.c")
LIB_PATH = os.path.join(_HERE, "libsdm_gx_oracle.so")
PA2_SRC = os.path.join(_HERE, "gx_pa2_oracle.c")
PA2_LIB_PATH = os.path.join(_HERE, "libsdm_pa2_oracle.so")

# -O2 without -ffast-math, no contraction: the C source's fmaf and + are exactly what runs.
CFLAGS = ("-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11")

_lib = None
_lib_lock = threading.Lock()


def build(src: str = _SRC, out: str = LIB_PATH, extra: tuple = ()) -> str:
    """Compile an oracle source with gcc into ``out`` (always recompiles; by default both oracles). Returns the output
    path."""
    if src == _SRC and out == LIB_PATH and not extra:
        _compile(PA2_SRC, PA2_LIB_PATH, ())
    return _compile(src, out, extra)


def _compile(src, out, extra):
    cmd = ["gcc", *CFLAGS, *extra, "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load an oracle library (building the default one if it is missing) and declare its signatures."""
    if path == LIB_PATH and not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    lib.sdm_gx_oracle_step.restype = ctypes.c_int
    lib.sdm_gx_oracle_step.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int64]
    lib.sdm_gx_oracle_fpenv_ok.restype = ctypes.c_int
    lib.sdm_gx_oracle_fpenv_ok.argtypes = []
    return lib


def _default_lib() -> ctypes.CDLL:
    global _lib
    with _lib_lock:
        if _lib is None:
            _lib = load()
        return _lib


def _check_arrays(d_u, x, d_dv):
    for name, a in (("d_u", d_u), ("x", x), ("d_dv", d_dv)):
        if not isinstance(a, np.ndarray) or a.dtype != np.float32 or a.ndim != 3 or not a.flags.c_contiguous:
            raise TypeError(f"oracle: {name} must be a C-contiguous float32 ndarray of rank 3")
    if not d_u.flags.writeable:
        raise TypeError("oracle: d_u must be writeable")
    N, C, C2 = x.shape
    if C2 != C or d_u.shape[:2] != (N, C) or d_dv.shape[:2] != (N, C):
        raise ValueError("oracle: x (N, C, C), d_dv (N, C, ld_dv), d_u (N, C, ld_u)")
    return N, C


def gx_gemm_step(d_u: np.ndarray, x: np.ndarray, d_dv: np.ndarray, ti: int, P: int, hd: int | None = None,
                 lib: ctypes.CDLL | None = None) -> None:
    """Step ti in place on d_u: chunks n = ti*P .. ti*P + P - 1, columns c < hd (default: all of d_u's columns)."""
    N, C = _check_arrays(d_u, x, d_dv)
    ld_u, ld_dv = d_u.shape[2], d_dv.shape[2]
    hd = ld_u if hd is None else int(hd)
    lib = lib or _default_lib()
    rc = lib.sdm_gx_oracle_step(d_u.ctypes.data, ld_u, x.ctypes.data, d_dv.ctypes.data, ld_dv, N, int(ti), int(P),
                                C, hd)
    if rc == -2:
        raise RuntimeError("oracle: host FP environment flushes subnormals or does not round to nearest")
    if rc != 0:
        raise ValueError(f"oracle: invalid step arguments (ti={ti}, P={P}, N={N}, C={C}, hd={hd})")


def gx_gemm_steps(d_u, x, d_dv, P: int, ti_list, hd: int | None = None, lib=None) -> None:
    """Steps in the given order, each in place on d_u."""
    for ti in ti_list:
        gx_gemm_step(d_u, x, d_dv, ti, P, hd, lib)


def gx_gemm_chunks(d_u, x, d_dv, n0: int, n1: int, hd: int | None = None, threads: int = 1, lib=None) -> int:
    """The update for chunks n0 .. n1 - 1 (any step), split over ``threads`` host threads by chunk. Each thread calls
    the unchanged scalar oracle on its own disjoint chunk range (as one step of P = its chunk count); ctypes releases
    the GIL during the call. Returns the number of threads used."""
    N, C = _check_arrays(d_u, x, d_dv)
    if not 0 <= n0 <= n1 <= N:
        raise ValueError("oracle: chunk range")
    ld_u, ld_dv = d_u.shape[2], d_dv.shape[2]
    hd = ld_u if hd is None else int(hd)
    lib = lib or _default_lib()
    if n1 == n0:
        return 0
    threads = max(1, min(int(threads), n1 - n0))
    bounds = [n0 + (n1 - n0) * k // threads for k in range(threads + 1)]
    errs = []

    def run(a, b):
        cnt = b - a
        if cnt <= 0:
            return
        rc = lib.sdm_gx_oracle_step(d_u[a:b].ctypes.data, ld_u, x[a:b].ctypes.data, d_dv[a:b].ctypes.data, ld_dv,
                                    cnt, 0, cnt, C, hd)
        if rc != 0:
            errs.append(rc)

    ts = [threading.Thread(target=run, args=(bounds[k], bounds[k + 1])) for k in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    if errs:
        raise RuntimeError(f"oracle: chunk range failed with codes {errs}")
    return threads


def fpenv_ok(lib=None) -> bool:
    return bool((lib or _default_lib()).sdm_gx_oracle_fpenv_ok())


# ---- Phase A --------------------------------------------------------------------------------------------------------
_pa2_lib = None


def load_pa2(path: str = PA2_LIB_PATH) -> ctypes.CDLL:
    """Load a Phase A oracle library (building the default one if it is missing)."""
    if path == PA2_LIB_PATH and not os.path.exists(path):
        _compile(PA2_SRC, PA2_LIB_PATH, ())
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.sdm_pa2_oracle_step.restype = ctypes.c_int
    lib.sdm_pa2_oracle_step.argtypes = [vp, vp, i64, vp, i64, i64, vp, i64, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                        i64, i64]
    lib.sdm_pa2_oracle_fpenv_ok.restype = ctypes.c_int
    lib.sdm_pa2_oracle_fpenv_ok.argtypes = []
    return lib


def _default_pa2() -> ctypes.CDLL:
    global _pa2_lib
    with _lib_lock:
        if _pa2_lib is None:
            _pa2_lib = load_pa2()
        return _pa2_lib


def _f32(a, name, ndim):
    if not isinstance(a, np.ndarray) or a.dtype != np.float32 or a.ndim != ndim or not a.flags.c_contiguous:
        raise TypeError(f"oracle: {name} must be a C-contiguous float32 ndarray of rank {ndim}")
    return a


def pa2_step(grad, bank, snap, ssr, du, beta, rec, out_eff, out_g, ti, P, C, W, hd=None, lib=None) -> None:
    """Phase A step ti in place on grad, bank, out_eff and out_g.
    grad, bank (slots, hd); snap (rows, hd); du (N*C, ld_u) token rows, columns < hd used; beta (N*C,); rec int32
    (N, C*W, 4); out_eff, out_g (planes, plane); ssr < 0: dense snapshot rows, else per-entry rows of stride ssr."""
    _f32(grad, "grad", 2), _f32(bank, "bank", 2), _f32(snap, "snap", 2), _f32(du, "du", 2), _f32(beta, "beta", 1)
    _f32(out_eff, "out_eff", 2), _f32(out_g, "out_g", 2)
    if not isinstance(rec, np.ndarray) or rec.dtype != np.int32 or rec.ndim != 3 or rec.shape[2] != 4 or \
            not rec.flags.c_contiguous:
        raise TypeError("oracle: rec must be a C-contiguous int32 ndarray (N, C*W, 4)")
    hd = grad.shape[1] if hd is None else int(hd)
    if bank.shape != grad.shape or snap.shape[1] != hd or grad.shape[1] != hd or out_eff.shape != out_g.shape:
        raise ValueError("oracle: grad / bank (slots, hd), snap (rows, hd), out_eff / out_g the same planes")
    N = rec.shape[0]
    lib = lib or _default_pa2()
    rc = lib.sdm_pa2_oracle_step(grad.ctypes.data, bank.ctypes.data, grad.shape[0], snap.ctypes.data, snap.shape[0],
                                 int(ssr), du.ctypes.data, du.shape[1], beta.ctypes.data, rec.ctypes.data,
                                 out_eff.ctypes.data, out_g.ctypes.data, out_eff.shape[1], N, int(ti), int(P), int(C),
                                 int(W), hd)
    if rc == -2:
        raise RuntimeError("oracle: host FP environment flushes subnormals or does not round to nearest")
    if rc == -3:
        raise ValueError("oracle: a record of the step is outside the definition (token, write, slot or snapshot row)")
    if rc != 0:
        raise ValueError(f"oracle: invalid Phase A arguments (ti={ti}, P={P}, N={N}, C={C}, W={W}, hd={hd})")


def pa2_fpenv_ok(lib=None) -> bool:
    return bool((lib or _default_pa2()).sdm_pa2_oracle_fpenv_ok())
