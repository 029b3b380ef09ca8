"""Helpers for the GPU parity tests: place host inputs on the device at chosen alignments, run the library through
the C ABI, and compute the expected result with the CPU oracle."""

from __future__ import annotations

import os
import sys

import numpy as np

import oracle
from deterministic_fp32_gemm_amd import inputs
from deterministic_fp32_gemm_amd.step import aligned_empty
from tests.compare import mismatch_report, same_bits

ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def say(*a):
    """Name the case on stdout (flushed) before its GPU work starts."""
    print(*a, file=sys.stdout, flush=True)


class DeviceCase:
    """Host inputs (x (N,C,C), d_dv (N,C,ld_dv), d_u (N,C,ld_u)) copied to device buffers whose base addresses sit at
    the given byte residues modulo 256."""

    def __init__(self, x, dv, du, hd, res_u=0, res_x=0, res_v=0, device="cuda"):
        import torch
        self.x_h, self.dv_h, self.du_h = x, dv, du
        self.N, self.C = x.shape[0], x.shape[1]
        self.hd, self.ld_u, self.ld_dv = int(hd), du.shape[2], dv.shape[2]
        self.x = aligned_empty(x.size, res_x, device)
        self.dv = aligned_empty(dv.size, res_v, device)
        self.du = aligned_empty(du.size, res_u, device)
        self.x.copy_(torch.from_numpy(x.reshape(-1)))
        self.dv.copy_(torch.from_numpy(dv.reshape(-1)))
        self.du.copy_(torch.from_numpy(du.reshape(-1)))
        torch.cuda.synchronize()

    def reset(self):
        import torch
        self.du.copy_(torch.from_numpy(self.du_h.reshape(-1)))
        torch.cuda.synchronize()

    def result(self) -> np.ndarray:
        import torch
        torch.cuda.synchronize()
        return self.du.cpu().numpy().reshape(self.du_h.shape)

    def args(self):
        """(d_u, ld_u, x, d_dv, ld_dv, N) for the C entry points."""
        return self.du, self.ld_u, self.x, self.dv, self.ld_dv, self.N


def expected(x, dv, du, hd, n0, n1):
    """The oracle's d_u after updating chunks n0 .. n1-1 (any union of whole steps)."""
    want = du.copy()
    oracle.gx_gemm_chunks(want, x, dv, n0, n1, hd, threads=ORACLE_THREADS)
    return want


def assert_matches(got, want, du_before, hd, what=""):
    """Bit-exact on every non-NaN result, NaN class on NaN results, and the padding columns' bits untouched."""
    ok = same_bits(got, want)
    if not ok.all():
        raise AssertionError(f"{what}: " + mismatch_report(got, want, ok))
    if hd < got.shape[2]:
        pad_g = got.view(np.uint32)[:, :, hd:]
        pad_b = du_before.view(np.uint32)[:, :, hd:]
        if (pad_g != pad_b).any():
            raise AssertionError(f"{what}: padding columns were written")


def workload_case(key: int, pattern: str = "normal", res_x: int = 0):
    w = inputs.WORKLOADS[key]
    x, dv, du = inputs.workload_inputs(w, pattern)
    return w, DeviceCase(x, dv, du, w.hd, res_u=w.base_offset_bytes, res_v=w.base_offset_bytes, res_x=res_x)
