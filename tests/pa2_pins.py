"""Independent pins of the Phase A oracle (oracle/gx_pa2_oracle.c).

Each pin checks the oracle against something other than itself: hand-derived worked examples (tests/golden/pa2),
integer inputs whose every partial result is exact (checked against an order-free int64 formulation of each group),
an exact-rational evaluation with a hand-written binary32 rounding (tests/exact.py) on tiny inputs with wild values,
the split of a head into column slices (each slice's plane equals a one-slice run on its columns), the forward error
bound of the dot products against float64, the floating-point environment guard, and the refusal of records outside
the definition. Every pin takes an oracle library handle so that broken builds of the oracle can be run through the
same battery (tests/test_pa2_mutants.py).
"""

from __future__ import annotations

import os

import numpy as np

import oracle
from deterministic_fp32_gemm_amd import pa2_inputs as PI
from tests import exact
from tests.compare import mismatch_report, same_bits

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pa2")


class PinFailure(AssertionError):
    pass


def _check(got, want, what):
    ok = same_bits(got, want)
    if not ok.all():
        raise PinFailure(what + ": " + mismatch_report(got, want, ok))


def _tok(t: str) -> float:
    return float.fromhex(t) if "0x" in t.lower() else float(t)


def load_fixture(path: str) -> dict:
    d = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            key, *vals = line.split()
            d[key] = vals
    dims = dict(v.split("=") for v in d["dims"])
    dims = {k: int(v) for k, v in dims.items()}
    f32 = lambda k: np.array([_tok(v) for v in d[k]], dtype=np.float32)   # noqa: E731
    N, C, W, hd, slots, rows = dims["N"], dims["C"], dims["W"], dims["hd"], dims["slots"], dims["rows"]
    n = C * W
    raw = d["rec"]
    rec = np.zeros((N, n, 4), np.int32)
    for j in range(N * n):
        pay, slot, sck, cpe = raw[4 * j:4 * j + 4]
        r = rec.reshape(-1, 4)[j]
        r[0] = np.uint32(int(pay, 16)).view(np.int32)
        r[1] = int(slot)
        r[2] = np.float32(_tok(sck)).view(np.int32)
        r[3] = np.float32(_tok(cpe)).view(np.int32)
    planes = 1 + (hd - 1) // 128
    return dict(dims=dims, du=f32("du").reshape(N * C, hd), beta=f32("beta"), rec=rec,
                grad=f32("grad").reshape(slots, hd), snap=f32("snap").reshape(rows, hd),
                bank=f32("bank").reshape(slots, hd), expect_grad=f32("expect_grad").reshape(slots, hd),
                expect_bank=f32("expect_bank").reshape(slots, hd), expect_eff=f32("expect_eff").reshape(planes, -1),
                expect_g=f32("expect_g").reshape(planes, -1), name=os.path.basename(path))


def fixtures() -> list:
    return [load_fixture(os.path.join(GOLDEN_DIR, f)) for f in sorted(os.listdir(GOLDEN_DIR)) if f.endswith(".txt")]


def run(d, dims, lib=None, planes=None):
    """The oracle on fixture-like arrays (copies of grad and bank); returns grad, bank, out_eff, out_g."""
    N, P, ti, C, W, hd = (dims[k] for k in ("N", "P", "ti", "C", "W", "hd"))
    n = C * W
    planes = planes or (1 + (hd - 1) // 128)
    grad, bank = d["grad"].copy(), d["bank"].copy()
    eff = np.full((planes, N * n), 77.0, np.float32)
    g = np.full((planes, N * n), 77.0, np.float32)
    oracle.pa2_step(grad, bank, d["snap"], dims.get("ssr", -1), d["du"], d["beta"], d["rec"], eff, g, ti, P, C, W,
                    hd, lib=lib)
    return grad, bank, eff, g


# ---- pin 1: hand-derived worked examples --------------------------------------------------------------------------
def pin_golden(lib=None):
    for fx in fixtures():
        grad, bank, eff, g = run(fx, fx["dims"], lib)
        _check(grad, fx["expect_grad"], fx["name"] + " grad")
        _check(bank, fx["expect_bank"], fx["name"] + " bank")
        _check(eff, fx["expect_eff"], fx["name"] + " out_eff")
        _check(g, fx["expect_g"], fx["name"] + " out_g")


# ---- pin 2: integer inputs, order-free int64 evaluation --------------------------------------------------------------
def _groups(pay):
    """(start, end) record ranges of a chunk's groups: from each FIRST to the record before the next FIRST."""
    firsts = np.flatnonzero(pay & PI.FIRST)
    ends = list(firsts[1:]) + [pay.size]
    return list(zip(firsts, ends))


def integer_expectation(d, w: PI.Pa2Workload, ti: int):
    """Expected grad, bank and output planes of step ti when every value is a small integer (exact in binary32, in
    any order): the group's grad row is gdw * cpe(LAST) + sum of sck * x over its records, its bank row the snapshot
    row, a record's dot the sum over the head's columns of a slice of x * sn, g that of gdw * sn."""
    N, n, C, W, hd, P = w.N, w.n, w.C, w.W, w.hd, w.P
    nsl = w.nsl
    slw = 4 * (((hd + 3) // 4 + nsl - 1) // nsl)
    grad = d["grad"].astype(np.int64)
    bank = d["bank"].copy()
    g64 = d["grad"].astype(np.int64)
    eff = np.zeros((nsl, N * n), np.float64)
    gout = np.zeros((nsl, N * n), np.float64)
    for p in range(P):
        k = ti * P + p
        rec = d["rec"][k]
        pay = rec[:, 0].view(np.uint32)
        sck = rec[:, 2].view(np.float32).astype(np.int64)
        cpe = rec[:, 3].view(np.float32).astype(np.int64)
        valid = (pay & PI.INVALID) == 0
        t = ((pay >> np.uint32(9)) & np.uint32(0xFF)).astype(np.int64)
        wr = (pay & np.uint32(0xFF)).astype(np.int64)
        ordinal = 0
        for s, e in _groups(pay):
            if valid[s]:
                srow = k * n + ordinal if w.dense else ti * (P * n) + p * n + t[s] * W + wr[s]
                ordinal += 1
                sn = d["snap"][srow].astype(np.int64)
                gdw = g64[rec[s, 1]]
            else:
                sn = np.zeros(hd, np.int64)
                gdw = np.zeros(hd, np.int64)
            x = d["du"][k * C + t[s:e], :hd].astype(np.int64)
            acc = (sck[s:e, None] * x).sum(axis=0)
            for sl in range(nsl):
                cols = slice(sl * slw, min(hd, (sl + 1) * slw))
                dots = (x[:, cols] * sn[cols]).sum(axis=1)
                gg = (gdw[cols] * sn[cols]).sum()
                o = k * n + t[s:e] * W + wr[s:e]
                v = valid[s:e]
                if nsl == 1:
                    beta = d["beta"][k * C + t[s:e]].astype(np.float64)
                    eff[0, o] = np.where(v, -beta * dots, 0.0)
                    gout[0, o] = np.where(v, cpe[s:e] * gg, 0.0)
                else:
                    eff[sl, o] = np.where(v, dots, 0.0)
                    gout[sl, o] = np.where(v, gg, 0.0)
            last = e - 1
            if valid[last] and (pay[last] & PI.LAST):
                grad[rec[last, 1]] = gdw * cpe[last] + acc
                bank[rec[last, 1]] = sn.astype(np.float32)
    return grad.astype(np.float32), bank, eff.astype(np.float32), gout.astype(np.float32)


INT_CASES = (
    PI.Pa2Workload("i1", 2, 2, 8, 3, 12, 12, 0, 64, True, 2.5, 0.1, "dense, one slice"),
    PI.Pa2Workload("i2", 1, 3, 5, 4, 136, 140, 0, 64, False, 3.0, 0.1, "per-entry, two slices of 68 columns"),
    PI.Pa2Workload("i3", 1, 1, 16, 8, 7, 9, 0, 256, True, 6.0, 0.2, "hd % 4 != 0, long groups"),
)


def pin_integer(lib=None):
    for w in INT_CASES:
        d = PI.inputs(w, "integer")
        for ti in range(w.T):
            dims = dict(N=w.N, P=w.P, ti=ti, C=w.C, W=w.W, hd=w.hd, ssr=d["ssr"])
            got = run(d, dims, lib, w.nsl)
            want = integer_expectation(d, w, ti)
            for name, a, b in zip(("grad", "bank", "out_eff", "out_g"), got, want):
                if name.startswith("out"):     # outputs of the step's chunks only (others keep their 77s)
                    k0, k1 = ti * w.P * w.n, (ti + 1) * w.P * w.n
                    a, b = a[:, k0:k1], b[:, k0:k1]
                _check(a, b, f"integer {w.key} step {ti} {name}")


# ---- pin 3: exact-rational evaluation of the walk ---------------------------------------------------------------------
def _tree(v):
    v = list(v)
    span = 1
    while span < 32:
        for i in range(0, 32, 2 * span):
            v[i] = exact.add(v[i], v[i + span])
        span *= 2
    return v[0]


def _dot4(a, b):
    s = exact.mul(a[0], b[0])
    for i in (1, 2, 3):
        s = exact.fma(a[i], b[i], s)
    return s


def rational_walk(d, dims):
    """The walk with every operation evaluated exactly and rounded once by the hand-written binary32 rounding."""
    N, P, ti, C, W, hd, ssr = (dims[k] for k in ("N", "P", "ti", "C", "W", "hd", "ssr"))
    n = C * W
    nsl = 1 + (hd - 1) // 128
    slw = 4 * (((hd + 3) // 4 + nsl - 1) // nsl)
    grad = [[float(v) for v in r] for r in d["grad"]]
    bank = [[float(v) for v in r] for r in d["bank"]]
    eff = [[float(v) for v in r] for r in np.full((nsl, N * n), 77.0, np.float32)]
    gout = [[float(v) for v in r] for r in np.full((nsl, N * n), 77.0, np.float32)]
    for p in range(P):
        k = ti * P + p
        for sl in range(nsl):
            cols = [sl * slw + c for c in range(128)]
            on = [c < slw and cols[c] < hd for c in range(128)]
            acc, gdw, sn, gp = [0.0] * 128, [0.0] * 128, [0.0] * 128, [0.0] * 32
            ordinal = 0
            for j in range(n):
                pay, slot, sckb, cpeb = (int(v) for v in d["rec"][k, j])
                pay &= 0xFFFFFFFF
                t, w = (pay >> 9) & 0xFF, pay & 0xFF
                valid = not (pay & 0x20000)
                sck = exact.from_bits(sckb & 0xFFFFFFFF)
                cpe = exact.from_bits(cpeb & 0xFFFFFFFF)
                x = [float(d["du"][k * C + t, cols[c]]) if on[c] else 0.0 for c in range(128)]
                if pay & 0x80000000:
                    acc = [0.0] * 128
                    if valid:
                        srow = k * n + ordinal if ssr < 0 else ti * ssr + p * n + t * W + w
                        ordinal += 1
                        gdw = [float(d["grad"][slot, cols[c]]) if on[c] else 0.0 for c in range(128)]
                        sn = [float(d["snap"][srow, cols[c]]) if on[c] else 0.0 for c in range(128)]
                    else:
                        gdw, sn = [0.0] * 128, [0.0] * 128
                    gp = [_dot4(gdw[4 * q:4 * q + 4], sn[4 * q:4 * q + 4]) for q in range(32)]
                acc = [exact.fma(sck, x[c], acc[c]) for c in range(128)]
                dot = _tree([_dot4(x[4 * q:4 * q + 4], sn[4 * q:4 * q + 4]) for q in range(32)])
                g = _tree(gp)
                if (pay & 0x40000000) and valid:
                    for c in range(128):
                        if on[c]:
                            grad[slot][cols[c]] = exact.fma(gdw[c], cpe, acc[c])
                            bank[slot][cols[c]] = sn[c]
                o = k * n + t * W + w
                if nsl == 1:
                    eff[0][o] = exact.mul(-float(d["beta"][k * C + t]), dot) if valid else 0.0
                    gout[0][o] = exact.mul(cpe, g) if valid else 0.0
                else:
                    eff[sl][o] = dot if valid else 0.0
                    gout[sl][o] = g if valid else 0.0
    f = lambda a: np.array(a, dtype=np.float32)    # noqa: E731
    return f(grad), f(bank), f(eff), f(gout)


def _wild(rng, shape):
    """float32 values over the whole binary32 range: random exponents (subnormal to near overflow), specials."""
    n = int(np.prod(shape))
    out = rng.standard_normal(n).astype(np.float32)
    kind = rng.random(n)
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    expo = rng.integers(60, 200, size=n).astype(np.uint32)
    wild = ((bits & np.uint32(0x807FFFFF)) | (expo << np.uint32(23))).view(np.float32)
    out = np.where(kind < 0.3, wild, out)
    sub = (bits & np.uint32(0x807FFFFF)).view(np.float32)
    out = np.where((kind >= 0.3) & (kind < 0.38), sub, out)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 2.0 ** 120, -(2.0 ** -149)], dtype=np.float32)
    out = np.where((kind >= 0.38) & (kind < 0.42), specials[rng.integers(0, specials.size, n)], out)
    return out.reshape(shape).astype(np.float32)


RATIONAL_CASES = (
    PI.Pa2Workload("r1", 1, 2, 2, 3, 8, 8, 0, 16, True, 2.0, 0.15, "dense, one slice"),
    PI.Pa2Workload("r2", 1, 1, 2, 2, 133, 133, 0, 8, False, 2.0, 0.1, "per-entry, two slices, hd % 4 != 0"),
)


def pin_exact(lib=None):
    rng = np.random.default_rng([20261020, 404])
    for trial, w in enumerate(RATIONAL_CASES * 2):
        d = PI.inputs(w, "normal", seed=trial)
        for key in ("grad", "snap"):
            used = d[key]
            d[key] = _wild(rng, used.shape) if trial % 2 == 0 else used
        d["du"][:, :w.hd] = _wild(rng, (w.N * w.C, w.hd)) if trial % 2 == 0 else d["du"][:, :w.hd]
        d["rec"][:, :, 2] = _wild(rng, d["rec"].shape[:2]).view(np.int32)
        d["beta"] = _wild(rng, d["beta"].shape)
        dims = dict(N=w.N, P=w.P, ti=0, C=w.C, W=w.W, hd=w.hd, ssr=d["ssr"])
        got = run(d, dims, lib, w.nsl)
        want = rational_walk(d, dims)
        for name, a, b in zip(("grad", "bank", "out_eff", "out_g"), got, want):
            _check(a, b, f"exact-rational {w.key} trial {trial} {name}")


# ---- pin 4: slices -------------------------------------------------------------------------------------------------------
def pin_slices(lib=None):
    """A head of nsl slices gives, in plane s, the raw dot and g of slice s; a one-slice run on that slice's columns
    with beta = -1 and cpe = 1 gives the same values through -beta * dot and cpe * g, exactly; grad and bank rows are
    the one-slice runs' rows on those columns."""
    w = PI.Pa2Workload("s", 1, 2, 6, 4, 200, 200, 0, 64, True, 3.0, 0.1, "two slices of 100 columns")
    d = PI.inputs(w, "normal", seed=3)
    dims = dict(N=w.N, P=w.P, ti=0, C=w.C, W=w.W, hd=w.hd, ssr=-1)
    grad, bank, eff, g = run(d, dims, lib, 2)
    for s in range(2):
        cols = slice(100 * s, 100 * s + 100)
        e = dict(d)
        e["grad"] = np.ascontiguousarray(d["grad"][:, cols])
        e["bank"] = np.ascontiguousarray(d["bank"][:, cols])
        e["snap"] = np.ascontiguousarray(d["snap"][:, cols])
        e["du"] = np.ascontiguousarray(d["du"][:, cols])
        e["beta"] = np.full_like(d["beta"], -1.0)
        e["rec"] = d["rec"].copy()
        e["rec"][:, :, 3] = np.float32(1.0).view(np.int32)
        sub = run(e, dict(dims, hd=100), lib, 1)
        # grad rows differ through cpe (fmaf(gdw, cpe, acc)): compare bank rows and outputs
        _check(bank[:, cols], sub[1], f"slice {s} bank")
        _check(eff[s:s + 1], sub[2], f"slice {s} dot plane")
        _check(g[s:s + 1], sub[3], f"slice {s} g plane")
    # and grad rows with cpe = 1 on both sides
    d2 = dict(d)
    d2["rec"] = d["rec"].copy()
    d2["rec"][:, :, 3] = np.float32(1.0).view(np.int32)
    grad2 = run(d2, dims, lib, 2)[0]
    for s in range(2):
        cols = slice(100 * s, 100 * s + 100)
        e = dict(d2)
        for key in ("grad", "bank", "snap", "du"):
            e[key] = np.ascontiguousarray(d2[key][:, cols])
        _check(grad2[:, cols], run(e, dict(dims, hd=100), lib, 1)[0], f"slice {s} grad")


# ---- pin 5: error bound of the dot products -------------------------------------------------------------------------
def pin_error_bound(lib=None):
    w = PI.Pa2Workload("b", 1, 2, 8, 4, 128, 128, 0, 64, True, 3.0, 0.0, "bound")
    d = PI.inputs(w, "normal", seed=5)
    d["beta"] = np.full_like(d["beta"], -1.0)
    d["rec"][:, :, 3] = np.float32(1.0).view(np.int32)
    dims = dict(N=w.N, P=w.P, ti=0, C=w.C, W=w.W, hd=w.hd, ssr=-1)
    eff = run(d, dims, lib, 1)[2][0].astype(np.float64)
    u = 2.0 ** -24
    gam = 9 * u / (1 - 9 * u)                 # at most 4 + 5 roundings along any term's path (chain, then tree)
    worst = 0.0
    for k in range(w.N):
        pay = d["rec"][k, :, 0].view(np.uint32)
        ordinal = 0
        for s, e in _groups(pay):
            valid = (pay[s] & PI.INVALID) == 0
            sn = d["snap"][k * w.n + ordinal].astype(np.float64) if valid else np.zeros(w.hd)
            ordinal += int(valid)
            for j in range(s, e):
                if pay[j] & PI.INVALID:
                    continue
                t, wr = (pay[j] >> 9) & 0xFF, pay[j] & 0xFF
                x = d["du"][k * w.C + t, :w.hd].astype(np.float64)
                ex = (x * sn).sum()
                mag = np.abs(x * sn).sum()
                err = abs(eff[k * w.n + t * w.W + wr] - ex)
                if err > gam * mag + 1e-12 * mag + 1e-300:
                    raise PinFailure(f"dot bound: record {j} of chunk {k}: error {err} > {gam * mag}")
                worst = max(worst, err / (mag or 1))
    if worst == 0.0:
        raise PinFailure("every dot is exact: the inputs cannot tell a float32 evaluation from a float64 one")


# ---- pin 6: floating-point environment guard --------------------------------------------------------------------------
def pin_fpenv(lib=None):
    from tests import fpenv
    fx = fixtures()[0]
    for m in fpenv.MODES:
        grad = fx["grad"].copy()
        with fpenv.mode(m):
            usable = oracle.pa2_fpenv_ok(lib)
            try:
                dims = fx["dims"]
                eff = np.zeros((1, 4), np.float32)
                oracle.pa2_step(grad, fx["bank"].copy(), fx["snap"], -1, fx["du"], fx["beta"], fx["rec"], eff,
                                eff.copy(), 0, dims["P"], dims["C"], dims["W"], dims["hd"], lib=lib)
                refused = False
            except RuntimeError:
                refused = True
        if usable or not refused:
            raise PinFailure(f"Phase A fpenv guard: runs in mode {m}")
        _check(grad, fx["grad"], f"Phase A fpenv guard: grad written in mode {m}")


# ---- pin 7: records outside the definition are refused, nothing written -----------------------------------------------
def pin_bad_records(lib=None):
    fx = fixtures()[0]
    dims = fx["dims"]
    for field, value in (("token", 2 << 9), ("write", 2), ("slot", None)):
        d = dict(fx)
        d["rec"] = fx["rec"].copy()
        if field == "slot":
            d["rec"][0, 2, 1] = dims["slots"]
        else:
            d["rec"][0, 3, 0] = np.int32(np.uint32(0x80000000 | value).view(np.int32))   # a valid FIRST past C or W
        grad = d["grad"].copy()
        eff = np.full((1, 4), 77.0, np.float32)
        try:
            oracle.pa2_step(grad, d["bank"].copy(), d["snap"], -1, d["du"], d["beta"], d["rec"], eff, eff.copy(), 0,
                            dims["P"], dims["C"], dims["W"], dims["hd"], lib=lib)
            refused = False
        except ValueError:
            refused = True
        if not refused:
            raise PinFailure(f"a record with its {field} out of range was accepted")
        _check(grad, d["grad"], f"bad {field}: grad written")
        _check(eff, np.full((1, 4), 77.0, np.float32), f"bad {field}: outputs written")


ALL_PINS = (pin_golden, pin_integer, pin_exact, pin_slices, pin_error_bound, pin_fpenv, pin_bad_records)


def run_all(lib=None) -> dict:
    out = {}
    for pin in ALL_PINS:
        try:
            pin(lib)
            out[pin.__name__] = None
        except (PinFailure, AssertionError, ValueError, RuntimeError, IndexError) as e:
            out[pin.__name__] = str(e)[:400]
    return out
