"""Host floating-point control state for the oracle's environment-guard pin (x86-64, per calling thread).

``non_ieee_modes()`` yields the modes under which the oracle must refuse to run: flush-to-zero alone,
denormals-are-zero alone, a directed rounding mode in the SSE control register alone, and a directed rounding mode
in the x87 control word alone (the one the C library's ``fegetround`` reports). Each is entered on the calling thread
and always restored afterwards.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
import tempfile
import threading

_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fpenv_helper.c")
_lib = None
_lock = threading.Lock()

MXCSR_FTZ = 1 << 15
MXCSR_DAZ = 1 << 6
MXCSR_RC_UP = 2 << 13          # rounding control field: 00 nearest, 01 down, 10 up, 11 toward zero
X87_RC_MASK = 0xC00
X87_RC_DOWN = 0x400


def helper() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            out = os.path.join(tempfile.mkdtemp(prefix="fpenv_"), "libfpenv_helper.so")
            subprocess.run(["gcc", "-O2", "-shared", "-fPIC", "-o", out, _SRC], check=True)
            lib = ctypes.CDLL(out)
            lib.fpenv_get_mxcsr.restype = ctypes.c_uint
            lib.fpenv_get_x87cw.restype = ctypes.c_uint
            lib.fpenv_set_mxcsr.argtypes = [ctypes.c_uint]
            lib.fpenv_set_x87cw.argtypes = [ctypes.c_uint]
            _lib = lib
        return _lib


@contextlib.contextmanager
def mode(name: str):
    """Enter one named non-IEEE mode on this thread; restore both control registers on exit."""
    h = helper()
    csr, cw = h.fpenv_get_mxcsr(), h.fpenv_get_x87cw()
    try:
        if name == "flush_to_zero":
            h.fpenv_set_mxcsr(csr | MXCSR_FTZ)
        elif name == "denormals_are_zero":
            h.fpenv_set_mxcsr(csr | MXCSR_DAZ)
        elif name == "sse_round_up":
            h.fpenv_set_mxcsr((csr & ~(3 << 13)) | MXCSR_RC_UP)
        elif name == "x87_round_down":
            h.fpenv_set_x87cw((cw & ~X87_RC_MASK) | X87_RC_DOWN)
        else:
            raise ValueError(name)
        yield
    finally:
        h.fpenv_set_mxcsr(csr)
        h.fpenv_set_x87cw(cw)


MODES = ("flush_to_zero", "denormals_are_zero", "sse_round_up", "x87_round_down")
