"""Seeded synthetic inputs for Phase A of the deterministic backward step (the consumer of the updated d_u).

This module only draws numbers and lays out the record structures; it holds none of Phase A's arithmetic, and it
imports neither the HIP library nor the oracle. The record format is the one the page "sparse-delta-memory 2.0.0 --
sparse_delta_memory/cuda/gx_pa2_cuda.py" reads (gx_pa2_kernel, the payload constants and snap_back): per chunk k, n =
C*W records, each the int32 quadruple {payload, slot, sck bits, cpe bits}; payload bit 31 FIRST (a group's first
record), bit 30 LAST (its last), bit 17 INVALID, bits 18-29 the distance back to the group's FIRST (4095: that far or
farther), bits 9-16 the token t < C, bits 0-7 the write w < W; kpay[k, j] is record j's payload, and bpre[k, b] is the
number of valid FIRST records among records 0 .. 32b-1 of chunk k (b = 0 .. ceil(n/32)).

How records are drawn (the forward that produces them is not on the pages; this is the plainest structure the walk
reads): the chunk's C*W (token, write) entries are shuffled and cut into groups whose sizes are drawn from a geometric
distribution of the given mean (capped at max_group); each group lists its entries in (token, write) order; every group
of a step gets its own slot (distinct across the step's P chunks, so no two groups of a step touch the same grad or
bank row; different steps may reuse slots); a record is INVALID with the given probability; sck ~ N(0, 1) and
cpe ~ U(0.5, 1.5). Snapshot rows: dense (row k*n + ordinal of the group's FIRST among the chunk's valid FIRSTs) or
per-entry (row ti*ssr + p*C*W + t*W + w of the FIRST record, ssr = P*C*W).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_BASE = 20261020
FIRST = np.uint32(0x80000000)
LAST = np.uint32(0x40000000)
INVALID = np.uint32(0x00020000)
DIST_SHIFT = 18
DIST_MAX = 4095
# rows and columns no record reaches hold this quiet-NaN pattern
PAD_BITS = np.uint32(0x7FC5A5A5)


@dataclass(frozen=True)
class Pa2Workload:
    """T steps of P chunks of C tokens with W writes each; head of hd columns; d_u rows of stride ld_u whose base sits
    du_offset_bytes past a 256-byte boundary; `slots` grad / bank rows; dense or per-entry snapshot rows."""
    key: str
    T: int
    P: int
    C: int
    W: int
    hd: int
    ld_u: int
    du_offset_bytes: int
    slots: int
    dense: bool
    mean_group: float
    invalid_frac: float
    description: str
    max_group: int = 1 << 16

    @property
    def N(self) -> int:
        return self.T * self.P

    @property
    def n(self) -> int:
        return self.C * self.W

    @property
    def nsl(self) -> int:
        return 1 + (self.hd - 1) // 128


PA2_WORKLOADS = {
    "a1": Pa2Workload("a1", 1, 2, 16, 4, 16, 16, 0, 256, True, 3.0, 0.05, "1 step x P=2, C=16, W=4, hd=16, dense snapshot"),
    "a3": Pa2Workload("a3", 8, 32, 64, 8, 128, 128, 0, 1 << 14, True, 4.0, 0.02,
                      "T=8 x P=32, C=64, W=8, hd=128 (workload 3's d_u), dense snapshot rows"),
    "a5": Pa2Workload("a5", 2, 512, 64, 8, 256, 260, 4, 1 << 17, False, 4.0, 0.02,
                      "T=2 x P=512, C=64, W=8, hd=256 in two slices (workload 5's d_u: ld 260, base +4 B), per-entry "
                      "snapshot rows"),
}


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng([SEED_BASE, 77, *[int(k) for k in key]])


def _group_sizes(rng, n, mean, cap):
    sizes = []
    left = n
    while left > 0:
        s = int(min(rng.geometric(1.0 / mean) if mean > 1 else 1, cap, left))
        sizes.append(s)
        left -= s
    return sizes


def chunk_records(rng, C, W, mean_group, invalid_frac, max_group=1 << 16):
    """One chunk's records without slots: (payload uint32 [n], group index of each record [n], groups)."""
    n = C * W
    order = rng.permutation(n)
    sizes = _group_sizes(rng, n, mean_group, max_group)
    pay = np.empty(n, np.uint32)
    grp = np.empty(n, np.int64)
    pos = 0
    for g, s in enumerate(sizes):
        ent = np.sort(order[pos:pos + s])              # the group's entries in (token, write) order
        t, w = ent // W, ent % W
        dist = np.minimum(np.arange(s), DIST_MAX).astype(np.uint32)
        p = (t.astype(np.uint32) << np.uint32(9)) | w.astype(np.uint32) | (dist << np.uint32(DIST_SHIFT))
        p[0] |= FIRST
        p[-1] |= LAST
        pay[pos:pos + s] = p
        grp[pos:pos + s] = g
        pos += s
    pay[rng.random(n) < invalid_frac] |= INVALID
    return pay, grp, len(sizes)


def bpre_of(kpay: np.ndarray) -> np.ndarray:
    """Per chunk: the count of valid FIRST records before each 32-record block (blocks 0 .. ceil(n/32))."""
    N, n = kpay.shape
    nb = (n + 31) // 32
    p = kpay.view(np.uint32)
    vf = ((p & FIRST) != 0) & ((p & INVALID) == 0)
    pad = np.zeros((N, nb * 32), bool)
    pad[:, :n] = vf
    blk = pad.reshape(N, nb, 32).sum(axis=2)
    out = np.zeros((N, nb + 1), np.int32)
    out[:, 1:] = np.cumsum(blk, axis=1)
    return out


def _values(rng, shape, pattern):
    if pattern == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if pattern == "integer":                            # small integers: every partial result exact in binary32
        return rng.integers(-4, 5, size=shape).astype(np.float32)
    if pattern == "special":                            # N(0,1) with scattered NaN, +-Inf, -0, subnormal and huge values
        a = rng.standard_normal(shape, dtype=np.float32)
        flat = a.reshape(-1)
        vals = np.array([0x7FC00000, 0x7F800000, 0xFF800000, 0x80000000, 0x00000003, 0x7F7FFFFF, 0xFF7FFFFF],
                        dtype=np.uint32).view(np.float32)
        k = max(1, flat.size // 300)
        idx = rng.choice(flat.size, size=k, replace=False)
        flat[idx] = vals[rng.integers(0, vals.size, size=k)]
        return a
    if pattern == "subnormal":                          # products and sums below 2^-126
        return np.ldexp(rng.standard_normal(shape), -66).astype(np.float32)
    raise ValueError(pattern)


def inputs(w: Pa2Workload, pattern: str = "normal", seed: int = 0):
    """Host arrays of one workload: dict with grad, bank [slots, hd]; snap [rows, hd]; du [N*C, ld_u]; beta [N*C];
    rec int32 [N, n, 4]; kpay int32 [N, n]; bpre int32 [N, nb+1]; ssr (-1 for dense rows); planes."""
    rng = _rng(int.from_bytes(w.key.encode(), "little"), seed, ("normal", "integer", "special", "subnormal").index(pattern))
    N, n, C, W, hd = w.N, w.n, w.C, w.W, w.hd
    rec = np.zeros((N, n, 4), np.int32)
    for ti in range(w.T):
        chunks = [chunk_records(rng, C, W, w.mean_group, w.invalid_frac, w.max_group) for _ in range(w.P)]
        total = sum(c[2] for c in chunks)
        if total > w.slots:
            raise ValueError(f"{total} groups in step {ti} need more than {w.slots} slots")
        step_slots = rng.choice(w.slots, size=total, replace=False).astype(np.int32)
        base = 0
        for p, (pay, grp, ng) in enumerate(chunks):
            k = ti * w.P + p
            rec[k, :, 0] = pay.view(np.int32)
            rec[k, :, 1] = step_slots[base + grp]
            base += ng
    if pattern == "integer":                             # exact products: sck and cpe small integers too
        rec[:, :, 2] = rng.integers(-3, 4, size=(N, n)).astype(np.float32).view(np.int32)
        rec[:, :, 3] = rng.integers(1, 3, size=(N, n)).astype(np.float32).view(np.int32)
    else:
        rec[:, :, 2] = rng.standard_normal((N, n), dtype=np.float32).view(np.int32)
        rec[:, :, 3] = rng.uniform(0.5, 1.5, size=(N, n)).astype(np.float32).view(np.int32)
    kpay = np.ascontiguousarray(rec[:, :, 0])
    rows = N * n
    snap = np.empty((rows, hd), np.float32)
    snap.view(np.uint32)[:] = PAD_BITS
    # the rows some group may read: every dense row of a chunk up to its valid-FIRST count, or every entry row of a
    # FIRST record (per-entry layout, ssr = P*C*W)
    bpre = bpre_of(kpay)
    if w.dense:
        used = np.concatenate([k * n + np.arange(bpre[k, -1]) for k in range(N)]) if N else np.zeros(0, int)
        ssr = -1
    else:
        ssr = w.P * n
        p = kpay.view(np.uint32)
        isf = (p & FIRST) != 0
        t = ((p >> np.uint32(9)) & np.uint32(0xFF)).astype(np.int64)
        wr = (p & np.uint32(0xFF)).astype(np.int64)
        kk = np.arange(N)[:, None]
        used = ((kk // w.P) * ssr + (kk % w.P) * n + t * W + wr)[isf]
    snap[used] = _values(rng, (used.size, hd), pattern)
    du = np.empty((N * C, w.ld_u), np.float32)
    du.view(np.uint32)[:] = PAD_BITS
    du[:, :hd] = _values(rng, (N * C, hd), pattern)
    beta = rng.uniform(0.0, 1.0, size=N * C).astype(np.float32)
    if pattern == "integer":
        beta = rng.integers(0, 3, size=N * C).astype(np.float32)
    grad = _values(rng, (w.slots, hd), pattern)
    bank = np.empty((w.slots, hd), np.float32)
    bank.view(np.uint32)[:] = PAD_BITS
    return dict(grad=grad, bank=bank, snap=snap, du=du, beta=beta, rec=rec, kpay=kpay, bpre=bpre, ssr=ssr,
                planes=w.nsl if w.nsl > 1 else 1)
