"""The CPU oracle against its independent pins (no GPU involved)."""

import numpy as np
import pytest

import oracle
from deterministic_fp32_gemm_amd import inputs
from tests import exact, pins
from tests.compare import assert_same_bits


def test_fpenv_is_ieee(oracle_lib):
    assert oracle.fpenv_ok(oracle_lib)


@pytest.mark.parametrize("fx", pins.fixtures(), ids=lambda f: f["name"])
def test_golden_fixture(fx, oracle_lib):
    du = fx["d_u"].copy()
    oracle.gx_gemm_step(du, fx["x"], fx["d_dv"], fx["ti"], fx["P"], fx["hd"], lib=oracle_lib)
    assert_same_bits(du, fx["expect"], fx["name"])
    # padding columns keep their exact bits
    assert (du.view(np.uint32)[:, :, fx["hd"]:] == fx["d_u"].view(np.uint32)[:, :, fx["hd"]:]).all()


@pytest.mark.parametrize("fx", pins.fixtures(), ids=lambda f: f["name"])
def test_golden_fixture_matches_exact_rational(fx):
    """The hand derivations in tests/golden agree with the exact-rational IEEE evaluation (checks both)."""
    hd = fx["hd"]
    want = exact.step(pins._tolist3(fx["d_u"][:, :, :hd]), pins._tolist3(fx["x"]),
                      pins._tolist3(fx["d_dv"][:, :, :hd]), fx["ti"], fx["P"], hd)
    assert_same_bits(np.array(want, dtype=np.float32), fx["expect"][:, :, :hd], fx["name"])


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_exact_rounding_helper_against_known_values():
    """Spot checks of the exact-rational binary32 rounding itself (ties to even, subnormals, overflow)."""
    from fractions import Fraction
    assert exact.round_rational(Fraction(2 ** 24 + 1)) == 2.0 ** 24                 # tie -> even
    assert exact.round_rational(Fraction(2 ** 24 + 3)) == 2.0 ** 24 + 4             # tie -> even (up)
    assert exact.round_rational(Fraction(1, 2 ** 150)) == 0.0                       # half the min subnormal
    assert exact.round_rational(Fraction(3, 2 ** 151)) == 2.0 ** -149
    assert exact.round_rational(Fraction(-1, 2 ** 151)) == 0.0
    assert np.signbit(exact.round_rational(Fraction(-1, 2 ** 151)))                 # underflow keeps the sign
    big = Fraction(2 ** 24 - 1) * Fraction(2) ** 104                                # FLT_MAX
    assert exact.round_rational(big) == float(np.finfo(np.float32).max)
    assert exact.round_rational(big + Fraction(2) ** 103) == np.inf                 # tie at FLT_MAX + half ulp
    assert exact.round_rational(big + Fraction(2) ** 102) == float(np.finfo(np.float32).max)
    # fma agrees with numpy's binary32 arithmetic wherever the product is exact in binary32
    rng = np.random.default_rng(5)
    a = rng.integers(-2 ** 11, 2 ** 11, 200).astype(np.float32)
    b = rng.integers(-2 ** 11, 2 ** 11, 200).astype(np.float32)
    c = rng.standard_normal(200).astype(np.float32)
    for ai, bi, ci in zip(a, b, c):
        assert exact.fma(float(ai), float(bi), float(ci)) == float(np.float32(ai * bi) + ci)


def test_step_order_and_chunk_split_invariance(oracle_lib):
    """Steps update disjoint chunks: forward, reverse and all-chunks-at-once (threaded) give identical bits."""
    w = inputs.Workload(0, 6, 3, 12, 10, 13, 0, "normal", "invariance")
    x, dv, du = inputs.shape_inputs(w.N, w.C, w.hd, w.ld, "hazard_cancel", seed=11)
    fwd, rev, once = du.copy(), du.copy(), du.copy()
    oracle.gx_gemm_steps(fwd, x, dv, w.P, range(w.T), w.hd, lib=oracle_lib)
    oracle.gx_gemm_steps(rev, x, dv, w.P, reversed(range(w.T)), w.hd, lib=oracle_lib)
    oracle.gx_gemm_chunks(once, x, dv, 0, w.N, w.hd, threads=4, lib=oracle_lib)
    assert_same_bits(rev, fwd, "reverse order")
    assert_same_bits(once, fwd, "threaded chunks")
    assert (fwd.view(np.uint32)[:, :, w.hd:] == du.view(np.uint32)[:, :, w.hd:]).all()


def test_reversed_chain_differs_on_cancellation(oracle_lib):
    """Negative control: running the chain in reversed j order (by reversing the j axis of x and d_dv) changes bits
    on cancellation-heavy input, so the j order is material and the pins can see it."""
    x, dv, du = inputs.shape_inputs(4, 32, 16, None, "hazard_cancel", seed=12)
    fwd, rev = du.copy(), du.copy()
    oracle.gx_gemm_step(fwd, x, dv, 0, 4, lib=oracle_lib)
    oracle.gx_gemm_step(rev, np.ascontiguousarray(x[:, ::-1, :]), np.ascontiguousarray(dv[:, ::-1, :]), 0, 4,
                        lib=oracle_lib)
    assert (fwd.view(np.uint32) != rev.view(np.uint32)).any()


def test_baddbmm_within_error_bound(oracle_lib):
    """A library batched GEMM (torch.baddbmm on the CPU, its own summation order) lands within the chain's error
    bound of the oracle; bits may differ."""
    torch = pytest.importorskip("torch")
    N, C, hd = 3, 48, 40
    x, dv, du = inputs.shape_inputs(N, C, hd, None, "normal", seed=13)
    got = du.copy()
    oracle.gx_gemm_step(got, x, dv, 0, N, lib=oracle_lib)
    ref = torch.baddbmm(torch.from_numpy(du.copy()), torch.from_numpy(x).transpose(1, 2).contiguous(),
                        torch.from_numpy(dv)).numpy()
    mag = np.einsum("nji,njc->nic", np.abs(x.astype(np.float64)), np.abs(dv.astype(np.float64)))
    u = 2.0 ** -24
    bound = 2 * (C * u / (1 - C * u)) * mag + 2 * u * (np.abs(du) + mag)
    assert (np.abs(got.astype(np.float64) - ref.astype(np.float64)) <= bound).all()


@pytest.mark.parametrize("args", [
    dict(ti=2, P=2),      # ti >= N / P (N = 4)
    dict(ti=-1, P=2),
    dict(ti=0, P=5),      # P > N
    dict(ti=0, P=0),
])
def test_invalid_step_arguments(args, oracle_lib):
    x, dv, du = inputs.shape_inputs(4, 4, 4)
    with pytest.raises(ValueError):
        oracle.gx_gemm_step(du, x, dv, args["ti"], args["P"], lib=oracle_lib)


def test_invalid_hd(oracle_lib):
    x, dv, du = inputs.shape_inputs(4, 4, 4)
    with pytest.raises(ValueError):
        oracle.gx_gemm_step(du, x, dv, 0, 4, hd=5, lib=oracle_lib)   # hd > ld
