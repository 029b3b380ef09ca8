"""Independent pins of the CPU oracle.

Each pin checks the oracle against something other than itself: hand-derived worked examples (tests/golden), an
integer sum computed in int64 (exact, any order), closed forms for zero and identity x, an exact-rational IEEE
binary32 evaluation on tiny inputs (tests/exact.py), and the forward error bound against float64. Every pin takes an
oracle library handle so that the same battery can be run against deliberately broken builds of the oracle
(tests/test_oracle_mutants.py), which must each fail at least one pin.
"""

from __future__ import annotations

import math
import os

import numpy as np

import oracle
from deterministic_fp32_gemm_amd import inputs
from tests import exact
from tests.compare import same_bits, mismatch_report

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


class PinFailure(AssertionError):
    pass


def _tok(t: str) -> float:
    t = t.strip()
    if "0x" in t.lower():
        return float.fromhex(t)
    return float(t)          # decimal, inf, -inf, nan


def load_fixture(path: str) -> dict:
    d = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            d[key] = vals
    N, P, ti, C, hd = (int(d[k][0]) for k in ("N", "P", "ti", "C", "hd"))
    ld = int(d["ld"][0]) if "ld" in d else hd
    arr = lambda k, shape: np.array([_tok(v) for v in d[k]], dtype=np.float32).reshape(shape)  # noqa: E731
    return dict(N=N, P=P, ti=ti, C=C, hd=hd, ld=ld, x=arr("x", (N, C, C)), d_dv=arr("d_dv", (N, C, ld)),
                d_u=arr("d_u", (N, C, ld)), expect=arr("expect", (N, C, ld)), name=os.path.basename(path))


def fixtures() -> list:
    return [load_fixture(os.path.join(GOLDEN_DIR, f)) for f in sorted(os.listdir(GOLDEN_DIR)) if f.endswith(".txt")]


def _check(ok: np.ndarray, got, want, what: str):
    if not ok.all():
        raise PinFailure(what + ": " + mismatch_report(got, want, ok))


# ---- pin 1: hand-derived worked examples -------------------------------------------------------------------------
def pin_golden(lib=None):
    for fx in fixtures():
        du = fx["d_u"].copy()
        oracle.gx_gemm_step(du, fx["x"], fx["d_dv"], fx["ti"], fx["P"], fx["hd"], lib=lib)
        _check(same_bits(du, fx["expect"]), du, fx["expect"], "golden " + fx["name"])


# ---- pin 2: integer inputs, exact int64 sum ----------------------------------------------------------------------
INT_CASES = (  # N, P, ti, C, hd, ld
    (6, 2, 1, 5, 7, 9),
    (3, 3, 0, 16, 4, 4),
    (5, 2, 1, 3, 2, 2),        # N % P != 0: chunk 4 belongs to no step
    (2, 1, 1, 64, 33, 40),
    (4, 4, 0, 1, 1, 1),
)


def pin_integer(lib=None):
    for (N, P, ti, C, hd, ld) in INT_CASES:
        x, dv, du = inputs.small_int_inputs(N, C, hd, ld, seed=N * 7 + C)
        got = du.copy()
        oracle.gx_gemm_step(got, x, dv, ti, P, hd, lib=lib)
        want = du.copy()
        xi = x.astype(np.int64)
        di = dv[:, :, :hd].astype(np.int64)
        s = np.einsum("nji,njc->nic", xi, di)          # sum over j of x[n, j, i] * d_dv[n, j, c], exact
        rows = slice(ti * P, ti * P + P)
        want[rows, :, :hd] = (du[rows, :, :hd].astype(np.int64) + s[rows]).astype(np.float32)
        _check(same_bits(got, want), got, want, f"integer N={N} P={P} ti={ti} C={C} hd={hd} ld={ld}")
        if (got.view(np.uint32)[:, :, hd:] != du.view(np.uint32)[:, :, hd:]).any():
            raise PinFailure(f"integer N={N} C={C} hd={hd} ld={ld}: padding columns were written")


# ---- pin 3: zero x ------------------------------------------------------------------------------------------------
def pin_zero_x(lib=None):
    N, P, ti, C, hd, ld = 4, 2, 1, 9, 6, 8
    _, dv, du = inputs.shape_inputs(N, C, hd, ld, "hazard_signed_zero", seed=3)   # finite, with signed zeros
    x = np.zeros((N, C, C), np.float32)
    x.reshape(-1)[::3] = -0.0
    got = du.copy()
    oracle.gx_gemm_step(got, x, dv, ti, P, hd, lib=lib)
    want = du.copy()
    rows = slice(ti * P, ti * P + P)
    blk = want[rows, :, :hd]
    blk[blk == 0] = 0.0          # every acc is +0, so -0 + +0 = +0 and every other d_u is unchanged
    want[rows, :, :hd] = blk
    _check(same_bits(got, want), got, want, "zero x")
    # an infinite d_dv entry turns its column into NaN (0 * inf)
    dv2 = dv.copy()
    dv2[ti * P, 2, 1] = np.inf
    got2 = du.copy()
    oracle.gx_gemm_step(got2, x, dv2, ti, P, hd, lib=lib)
    if not np.isnan(got2[ti * P, :, 1]).all():
        raise PinFailure("zero x with an infinite d_dv entry must give NaN in that column")


# ---- pin 4: identity x --------------------------------------------------------------------------------------------
def pin_identity_x(lib=None):
    N, P, ti, C, hd, ld = 3, 1, 2, 7, 5, 5
    _, dv, du = inputs.shape_inputs(N, C, hd, ld, "hazard_signed_zero", seed=4)
    x = np.broadcast_to(np.eye(C, dtype=np.float32), (N, C, C)).copy()
    got = du.copy()
    oracle.gx_gemm_step(got, x, dv, ti, P, hd, lib=lib)
    n = ti * P
    acc = dv[n, :, :hd].copy()          # x[n, j, i] = [j == i]: acc = d_dv[n, i, c], except -0 -> +0
    acc[acc == 0] = 0.0
    want = du.copy()
    want[n, :, :hd] = (du[n, :, :hd] + acc).astype(np.float32)      # one IEEE binary32 add (numpy)
    _check(same_bits(got, want), got, want, "identity x")


# ---- pin 5: exact rational evaluation ------------------------------------------------------------------------------
def _wild_values(rng, shape):
    """float32 values mixing N(0,1), arbitrary exponents (subnormal to near-overflow) and specials."""
    n = int(np.prod(shape))
    out = rng.standard_normal(n).astype(np.float32)
    kind = rng.random(n)
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    exp = rng.integers(0, 255, size=n).astype(np.uint32)        # 0 = subnormal, 254 = largest finite binade
    wild = ((bits & np.uint32(0x807FFFFF)) | (exp << np.uint32(23))).view(np.float32)
    out = np.where(kind < 0.25, wild, out)
    sub = (bits & np.uint32(0x807FFFFF)).view(np.float32)           # subnormal (or zero)
    out = np.where((kind >= 0.25) & (kind < 0.35), sub, out)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 2.0 ** 127, -(2.0 ** -149)], dtype=np.float32)
    out = np.where((kind >= 0.35) & (kind < 0.40), specials[rng.integers(0, specials.size, n)], out)
    return out.reshape(shape).astype(np.float32)


def _tolist3(a):
    return [[[float(v) for v in row] for row in ch] for ch in a]


def pin_exact(lib=None, trials: int = 12):
    rng = np.random.default_rng([20261020, 99])
    shapes = [(4, 2, 1, 4, 3)] * (trials - 2) + [(2, 1, 1, 16, 4), (3, 3, 0, 2, 5)]   # N, P, ti, C, hd
    for t, (N, P, ti, C, hd) in enumerate(shapes):
        if t % 3 == 0:
            x = _wild_values(rng, (N, C, C))
            dv = _wild_values(rng, (N, C, hd))
            du = _wild_values(rng, (N, C, hd))
        else:        # mostly finite: long stretches of ordinary rounding and cancellation
            x = rng.standard_normal((N, C, C)).astype(np.float32)
            dv = (rng.standard_normal((N, C, hd)) * np.exp2(rng.integers(-30, 30, (N, C, hd)))).astype(np.float32)
            du = rng.standard_normal((N, C, hd)).astype(np.float32)
            if t % 3 == 2:   # push products into the subnormal range
                x *= np.float32(2.0 ** -70)
                dv *= np.float32(2.0 ** -70)
                du *= np.float32(2.0 ** -130)
        got = du.copy()
        oracle.gx_gemm_step(got, x, dv, ti, P, hd, lib=lib)
        want = np.array(exact.step(_tolist3(du), _tolist3(x), _tolist3(dv), ti, P, hd), dtype=np.float32)
        _check(same_bits(got, want), got, want, f"exact-rational trial {t} (N={N} P={P} ti={ti} C={C} hd={hd})")


# ---- pin 6: forward error bound versus float64 --------------------------------------------------------------------
def pin_error_bound(lib=None):
    N, P, ti, C, hd = 4, 2, 1, 64, 48
    x, dv, du = inputs.shape_inputs(N, C, hd, None, "normal", seed=6)
    got = du.copy()
    oracle.gx_gemm_step(got, x, dv, ti, P, hd, lib=lib)
    rows = slice(ti * P, ti * P + P)
    x64, d64, u64 = x[rows].astype(np.float64), dv[rows].astype(np.float64), du[rows].astype(np.float64)
    s = np.einsum("nji,njc->nic", x64, d64)
    mag = np.einsum("nji,njc->nic", np.abs(x64), np.abs(d64))
    u = 2.0 ** -24
    gamma = C * u / (1 - C * u)
    # chain error <= gamma * sum|x d|; the final add adds u * |d_u + acc|; float64 evaluation error is far smaller
    bound = gamma * mag + u * (np.abs(u64 + s) + gamma * mag) + 1e-12 * (mag + np.abs(u64))
    err = np.abs(got[rows].astype(np.float64) - (u64 + s))
    if not (err <= bound).all():
        k = np.argmax(err - bound)
        raise PinFailure(f"error bound violated: max excess {float((err - bound).reshape(-1)[k])}")
    # the untouched chunks are bit-identical
    others = [n for n in range(N) if not (ti * P <= n < ti * P + P)]
    _check(same_bits(got[others], du[others]), got[others], du[others], "untouched chunks")
    # and the chain is not computed in higher precision: at least one element differs from the float64 value
    # rounded once (a 64 x 48 x 2 block of N(0,1) chains essentially always has some double-rounding difference)
    once = (u64 + s).astype(np.float32)
    if same_bits(got[rows], once).all():
        raise PinFailure("result equals float64 evaluation rounded once: the chain is not binary32")


# ---- pin 7: the floating-point environment guard ----------------------------------------------------------------
def pin_fpenv_refusal(lib=None):
    """The oracle's results are IEEE binary32 with subnormals kept and round-to-nearest-even, the page's setting
    (plain fmaf and +; its qualification probe feeds subnormal accumulations). A host thread in flush-to-zero,
    denormals-are-zero or a directed rounding mode would silently give other bits, so the oracle must refuse there:
    the guard reports the environment as unusable, the step returns its environment status without touching d_u,
    and it runs again once the environment is restored. Each mode is entered alone, so every check of the guard is
    exercised on its own."""
    from tests import fpenv
    x, dv, du = inputs.shape_inputs(2, 4, 3, None, "hazard_subnormal", seed=8)
    for m in fpenv.MODES:
        got = du.copy()
        with fpenv.mode(m):
            usable = oracle.fpenv_ok(lib)
            try:
                oracle.gx_gemm_step(got, x, dv, 0, 2, lib=lib)
                refused = False
            except RuntimeError:
                refused = True
        if usable:
            raise PinFailure(f"fpenv guard: reports the host usable in mode {m}")
        if not refused:
            raise PinFailure(f"fpenv guard: the step ran in mode {m}")
        _check(same_bits(got, du), got, du, f"fpenv guard: d_u written while refusing in mode {m}")
    if not oracle.fpenv_ok(lib):
        raise PinFailure("fpenv guard: refuses the restored IEEE environment")
    got = du.copy()
    oracle.gx_gemm_step(got, x, dv, 0, 2, lib=lib)


ALL_PINS = (pin_golden, pin_integer, pin_zero_x, pin_identity_x, pin_exact, pin_error_bound, pin_fpenv_refusal)


def run_all(lib=None) -> dict:
    """{pin name: None if it passed, else the failure message}."""
    out = {}
    for pin in ALL_PINS:
        try:
            pin(lib)
            out[pin.__name__] = None
        except (PinFailure, AssertionError, ValueError, RuntimeError) as e:
            out[pin.__name__] = str(e)[:400]
    return out


def nan_safe_equal(a: float, b: float) -> bool:
    return (math.isnan(a) and math.isnan(b)) or (exact.bits(a) == exact.bits(b))
