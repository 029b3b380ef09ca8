"""Seeded synthetic inputs for the per-step d_u update (shared by the tests and the benchmark).

This module only draws numbers and lays them out; it holds none of the update's arithmetic, and it imports neither
the HIP library nor the oracle. Every array is numpy float32 on the host:

  x    (N, C, C)       x[n, j, i]
  d_dv (N, C, ld)      columns c < hd are data, columns hd..ld-1 hold PAD_BITS
  d_u  (N, C, ld)      same layout as d_dv

Workloads (the five shapes the update is measured and checked on) and value patterns follow the recipes stated in
the repository's design notes; the page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_gemm_cuda.py"
contributes its qualification probe's pattern families (_probe_inputs: signed zeros, half-zero masks, wide
exponents with near-overflow spikes, subnormal accumulation, near-cancelling row pairs, scattered specials), which
are re-drawn here with numpy's generator rather than reproduced bit for bit.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_BASE = 20261020
# Padding columns hd..ld-1 of d_u and d_dv hold this quiet-NaN bit pattern; they must never be read into a result or
# written.
PAD_BITS = np.uint32(0x7FC5A5A5)


@dataclass(frozen=True)
class Workload:
    """One measured/checked shape: T steps of P chunks, C rows (= chain length), hd columns, row stride ld of d_u
    and d_dv, and the byte offset of the d_u / d_dv base pointers from a 256-byte boundary on the device."""
    key: int
    T: int
    P: int
    C: int
    hd: int
    ld: int
    base_offset_bytes: int
    dist: str            # "normal" or "tril" (x ~ U(-1,1) masked to x[n,j,i]=0 for j<i; d_dv, d_u ~ N(0, 0.1))
    description: str

    @property
    def N(self) -> int:
        return self.T * self.P

    @property
    def flops_per_step(self) -> int:
        """2 flops per fused multiply-add of the chain plus the final add, over the step's P chunks."""
        return self.P * (2 * self.C * self.C * self.hd + self.C * self.hd)

    @property
    def bytes_per_step(self) -> int:
        """Algorithmic HBM bytes of one step: x and d_dv read once, d_u read and written once (padding excluded)."""
        return 4 * self.P * (self.C * self.C + 3 * self.C * self.hd)


WORKLOADS = {
    1: Workload(1, 1, 2, 16, 16, 16, 0, "normal", "single step ti=0, P=2, C=16, hd=16"),
    2: Workload(2, 16, 8, 64, 64, 64, 0, "normal", "T=16 steps x P=8 chunks, C=64, hd=64"),
    3: Workload(3, 8, 32, 64, 128, 128, 0, "normal", "T=8 steps x P=32, C=64, hd=128, six value patterns"),
    4: Workload(4, 4, 128, 128, 128, 128, 0, "tril", "T=4 steps x P=128, C=128, hd=128, lower-triangular masked x"),
    5: Workload(5, 2, 512, 64, 256, 260, 4, "normal", "T=2 steps x P=512, C=64, hd=256, row stride 260, base +4 B"),
}

# The six value patterns every step is checked on.
PATTERNS = ("normal", "zeros", "large", "denormal", "inf", "nan")
# The qualification probe's pattern families, re-drawn.
PROBE_PATTERNS = ("probe_normal", "probe_zeros", "probe_large", "probe_denormal", "probe_cancel", "probe_special")
ALL_PATTERNS = PATTERNS + PROBE_PATTERNS


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([SEED_BASE, *[int(k) for k in key]])


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _pad(a: np.ndarray, ld: int) -> np.ndarray:
    """(N, C, hd) -> (N, C, ld) with PAD_BITS in columns hd..ld-1."""
    N, C, hd = a.shape
    out = np.empty((N, C, ld), dtype=np.float32)
    out.view(np.uint32)[:, :, hd:] = PAD_BITS
    out[:, :, :hd] = a
    return out


def _inject(rng: np.random.Generator, a: np.ndarray, frac: float, values: np.ndarray) -> None:
    """Overwrite round(frac * a.size) distinct random elements of a with values drawn from ``values``."""
    flat = a.reshape(-1)
    k = max(1, int(round(frac * flat.size)))
    idx = rng.choice(flat.size, size=k, replace=False)
    flat[idx] = rng.choice(values, size=k)


def raw(N: int, C: int, hd: int, pattern: str, seed_key: tuple, dist: str = "normal"):
    """x (N, C, C), d_dv (N, C, hd), d_u (N, C, hd) in one value pattern, drawn in the order x, d_dv, d_u."""
    rng = _rng(*seed_key)
    if pattern == "normal":
        if dist == "tril":
            x = rng.uniform(-1.0, 1.0, size=(N, C, C))
            j = np.arange(C)[:, None]
            i = np.arange(C)[None, :]
            x = np.where(j < i, 0.0, x)               # x[n, j, i] = 0 for j < i
            dv = rng.normal(0.0, 0.1, size=(N, C, hd))
            du = rng.normal(0.0, 0.1, size=(N, C, hd))
            return _f32(x), _f32(dv), _f32(du)
        x = rng.standard_normal((N, C, C), dtype=np.float32)
        dv = rng.standard_normal((N, C, hd), dtype=np.float32)
        du = rng.standard_normal((N, C, hd), dtype=np.float32)
        return _f32(x), _f32(dv), _f32(du)
    if pattern == "zeros":
        return (np.zeros((N, C, C), np.float32), np.zeros((N, C, hd), np.float32), np.zeros((N, C, hd), np.float32))
    if pattern == "large":
        return tuple(_f32(rng.uniform(-1e30, 1e30, size=s)) for s in ((N, C, C), (N, C, hd), (N, C, hd)))
    if pattern == "denormal":
        return tuple(_f32(rng.uniform(-1e-40, 1e-40, size=s)) for s in ((N, C, C), (N, C, hd), (N, C, hd)))
    if pattern in ("inf", "nan"):
        arrs = [rng.standard_normal(s, dtype=np.float32) for s in ((N, C, C), (N, C, hd), (N, C, hd))]
        vals = np.array([np.inf, -np.inf] if pattern == "inf" else [np.nan], dtype=np.float32)
        for a in arrs:
            _inject(rng, a, 0.01, vals)
        return tuple(_f32(a) for a in arrs)
    if pattern.startswith("probe_"):
        return _probe(rng, N, C, hd, pattern[len("probe_"):])
    raise ValueError(f"unknown pattern {pattern!r}")


def _probe(rng, N, C, hd, kind):
    x = rng.standard_normal((N, C, C)).astype(np.float32) * np.float32(0.25)
    dv = rng.standard_normal((N, C, hd)).astype(np.float32)
    du = rng.standard_normal((N, C, hd)).astype(np.float32)
    if kind == "normal":                  # signed zeros sprinkled at fixed strides
        x.reshape(-1)[::7] = -0.0
        dv.reshape(-1)[::11] = 0.0
        du.reshape(-1)[::13] = -0.0
    elif kind == "zeros":                 # half of the entries zero, x's zeros negative
        x *= (rng.random(x.shape) < 0.5)
        x[x == 0] = -0.0
        dv *= (rng.random(dv.shape) < 0.5)
        du[rng.random(du.shape) < 0.5] = -0.0
    elif kind == "large":                 # exponents spread over 2^-60 .. 2^60, near-overflow spikes
        for a in (x, dv, du):
            a *= np.exp2(rng.integers(-60, 61, size=a.shape)).astype(np.float32)
        x.reshape(-1)[::17] = 3.0e38
        dv.reshape(-1)[::19] = -3.0e38
    elif kind == "denormal":              # products land in the subnormal range and accumulate there
        x *= np.float32(1e-20)
        dv *= np.float32(1e-19)
        du *= np.float32(1e-38)
        du.reshape(-1)[::5] = np.float32(1e-41)
    elif kind == "cancel":                # odd rows of d_dv nearly cancel the even rows above them
        x = (np.sign(rng.standard_normal(x.shape)) * (1.0 + rng.random(x.shape))).astype(np.float32)
        dv *= np.float32(1e4)
        h = C // 2
        if h:
            jitter = (1.0 + 1e-3 * rng.standard_normal((N, h, hd))).astype(np.float32)
            dv[:, 1:2 * h:2, :] = -dv[:, 0:2 * h:2, :] * jitter
        du *= np.float32(1e-3)
    elif kind == "special":               # NaN, +-Inf, -0, a subnormal and +-near-max at random slots
        specials = np.array([np.nan, np.inf, -np.inf, -0.0, 1e-41, 3.4e38, -3.4e38], dtype=np.float32)
        for a, k in ((dv, 64), (x, 16), (du, 32)):
            flat = a.reshape(-1)
            k = min(k, flat.size)
            flat[rng.permutation(flat.size)[:k]] = specials[np.arange(k) % specials.size]
    else:
        raise ValueError(kind)
    return _f32(x), _f32(dv), _f32(du)


def workload_inputs(w: Workload | int, pattern: str = "normal"):
    """The whole workload's host inputs: x (N, C, C), d_dv (N, C, ld), d_u (N, C, ld) with padding columns set to
    PAD_BITS. Seeded by (workload key, pattern index)."""
    if not isinstance(w, Workload):
        w = WORKLOADS[int(w)]
    x, dv, du = raw(w.N, w.C, w.hd, pattern, (w.key, ALL_PATTERNS.index(pattern)), w.dist)
    return x, _pad(dv, w.ld), _pad(du, w.ld)


def shape_inputs(N: int, C: int, hd: int, ld: int | None = None, pattern: str = "normal", seed: int = 0,
                 dist: str = "normal"):
    """Inputs for an arbitrary shape (tests of ragged tiles and edge cases)."""
    ld = hd if ld is None else int(ld)
    x, dv, du = raw(N, C, hd, pattern, (1000 + int(seed), N, C, hd, ALL_PATTERNS.index(pattern)), dist)
    return x, _pad(dv, ld), _pad(du, ld)


def small_int_inputs(N: int, C: int, hd: int, ld: int | None = None, lo: int = -8, hi: int = 8, seed: int = 0):
    """Integer-valued float32 inputs in [lo, hi] (so every partial result of the chain is an exact integer)."""
    ld = hd if ld is None else int(ld)
    rng = _rng(7, N, C, hd, seed)
    x = rng.integers(lo, hi + 1, size=(N, C, C)).astype(np.float32)
    dv = rng.integers(lo, hi + 1, size=(N, C, hd)).astype(np.float32)
    du = rng.integers(lo, hi + 1, size=(N, C, hd)).astype(np.float32)
    return x, _pad(dv, ld), _pad(du, ld)
