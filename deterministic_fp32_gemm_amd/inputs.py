"""Seeded synthetic inputs for the per-step d_u update (shared by the tests and the benchmark).

This module only draws numbers and lays them out; it holds none of the update's arithmetic, and it imports neither
the HIP library nor the oracle. Every array is numpy float32 on the host:

  x    (N, C, C)       x[n, j, i]
  d_dv (N, C, ld)      columns c < hd are data, columns hd..ld-1 hold PAD_BITS
  d_u  (N, C, ld)      same layout as d_dv

Workloads (the five shapes the update is measured and checked on) and the six value patterns follow the recipes
stated in the repository's design notes. The hazard families target the same floating-point hazards as the
qualification probe on the page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_gemm_cuda.py" (signed
zeros, sparse operands, wide exponents with overflow, subnormal accumulation, cancellation, special values); their
recipes (rates, scales, structure) are this module's own.
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
# Hazard families, one floating-point hazard of the chain each (the same hazards the page's qualification probe
# targets; these recipes are this module's own).
HAZARD_PATTERNS = ("hazard_signed_zero", "hazard_sparse", "hazard_wide", "hazard_subnormal", "hazard_cancel",
                   "hazard_special")
ALL_PATTERNS = PATTERNS + HAZARD_PATTERNS


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
    if pattern.startswith("hazard_"):
        return _hazard(rng, N, C, hd, pattern[len("hazard_"):])
    raise ValueError(f"unknown pattern {pattern!r}")


def _signs(rng, shape) -> np.ndarray:
    return np.where(rng.random(shape) < 0.5, np.float32(-1.0), np.float32(1.0))


def _hazard(rng, N, C, hd, kind):
    """Inputs that stress one floating-point hazard of the fixed chain at a time (x, d_dv, d_u)."""
    sx, sv, su = (N, C, C), (N, C, hd), (N, C, hd)
    if kind == "signed_zero":
        # N(0,1) with one element in eight replaced by a zero of random sign: -0 products meet +0 and -0 sums
        out = []
        for s in (sx, sv, su):
            a = rng.standard_normal(s, dtype=np.float32)
            z = rng.random(s) < 0.125
            a[z] = np.float32(0.0) * _signs(rng, s)[z]
            out.append(a)
        return tuple(out)
    if kind == "sparse":
        # most products vanish: x zero (random sign) with probability 0.6, d_dv with 0.3, d_u is -0 with 0.3
        x = rng.standard_normal(sx, dtype=np.float32)
        x = np.where(rng.random(sx) < 0.6, np.float32(0.0) * _signs(rng, sx), x)
        dv = rng.standard_normal(sv, dtype=np.float32)
        dv = np.where(rng.random(sv) < 0.3, np.float32(0.0) * _signs(rng, sv), dv)
        du = rng.standard_normal(su, dtype=np.float32)
        du = np.where(rng.random(su) < 0.3, np.float32(-0.0), du)
        return _f32(x), _f32(dv), _f32(du)
    if kind == "wide":
        # sign * m * 2^e, m in [1, 2): x and d_dv exponents over [-70, 70] (products from the subnormal range to
        # overflow), d_u over [-40, 40]; one x and d_dv element in 500 at +-m * 2^126 (overflows against most rows)
        def draw(s, lo, hi):
            m = (1.0 + rng.random(s)) * _signs(rng, s)
            return _f32(np.ldexp(m, rng.integers(lo, hi + 1, size=s)))
        x, dv, du = draw(sx, -70, 70), draw(sv, -70, 70), draw(su, -40, 40)
        for a in (x, dv):
            flat = a.reshape(-1)
            k = max(1, flat.size // 500)
            idx = rng.choice(flat.size, size=k, replace=False)
            flat[idx] = _f32(np.ldexp((1.0 + rng.random(k)) * _signs(rng, k), 126))
        return x, dv, du
    if kind == "subnormal":
        # every product is subnormal (|x d| about 2^-132) and the chain accumulates below 2^-126; d_u subnormal,
        # with one element in seven at k * 2^-149 (k = 1 .. 7, the smallest subnormals)
        x = _f32(np.ldexp(rng.standard_normal(sx), -64))
        dv = _f32(np.ldexp(rng.standard_normal(sv), -68))
        du = _f32(np.ldexp(rng.standard_normal(su), -128))
        flat = du.reshape(-1)
        idx = np.flatnonzero(rng.random(flat.size) < 1.0 / 7.0)
        flat[idx] = _f32(np.ldexp(rng.integers(1, 8, size=idx.size) * _signs(rng, idx.size), -149))
        return x, dv, du
    if kind == "cancel":
        # mirrored chain rows: row C-1-j of x repeats row j and row C-1-j of d_dv is row j negated and perturbed
        # by a relative 2^-11 or less, so the late half of every chain undoes the early half (magnitudes near 2^12)
        # and what is left depends on the order of the steps
        x = _f32(rng.choice(np.array([0.5, 1.0, 1.5, 2.0], np.float32), size=sx) * _signs(rng, sx))
        dv = _f32(np.ldexp(rng.standard_normal(sv), 12))
        h = C // 2
        if h:
            lo = np.arange(h)
            hi = C - 1 - lo
            x[:, hi, :] = x[:, lo, :]
            delta = _f32(1.0 + np.ldexp(rng.uniform(-1.0, 1.0, size=(N, h, hd)), -11))
            dv[:, hi, :] = -dv[:, lo, :] * delta
        du = _f32(np.ldexp(rng.standard_normal(su), -6))
        return _f32(x), _f32(dv), du
    if kind == "special":
        # N(0,1) with scattered specials: quiet NaNs (two payloads), +-Inf, +-0, +-2^-149, +-FLT_MAX, 2^-126; one
        # element in 256 of d_dv, 384 of d_u, 512 of x (at least one each)
        vals = np.array([0x7FC00000, 0xFFC12345, 0x7F800000, 0xFF800000, 0x00000000, 0x80000000, 0x00000001,
                         0x80000001, 0x7F7FFFFF, 0xFF7FFFFF, 0x00800000], dtype=np.uint32).view(np.float32)
        out = []
        for s, every in ((sx, 512), (sv, 256), (su, 384)):
            a = rng.standard_normal(s, dtype=np.float32)
            flat = a.reshape(-1)
            k = max(1, flat.size // every)
            idx = rng.choice(flat.size, size=k, replace=False)
            flat[idx] = vals[rng.integers(0, vals.size, size=k)]
            out.append(a)
        return tuple(out)
    raise ValueError(kind)


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
