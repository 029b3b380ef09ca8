"""Seeded random sweep over shapes, strides, base-address residues, step ranges and plans (the planner's and
explicit ones of both engines), every result compared with the oracle bit for bit. Complements the hand-picked
cases: C in 1..256, hd in 1..600, row strides with every residue mod 4, bases at 4-byte residues mod 64."""

import numpy as np
import pytest

import deterministic_fp32_gemm_amd as g
from deterministic_fp32_gemm_amd import inputs
from tests.gpu_util import DeviceCase, assert_matches, expected, say

pytestmark = pytest.mark.gpu

EXPLICIT = [None, None, None,
            ("mfma", 1, 2, 3, 0, 1, 0, 0, 16, 32), ("mfma", 2, 4, 3, 0, 1, 3, 0, 16, 16), ("mfma", 1, 8, 8, 0, 2, 0, 0, 16),
            ("mfma", 1, 4, 4, 0, 1, 5, 0, 32), ("mfma", 2, 2, 4, 4, 4, 0), ("mfma", 1, 2, 4, 2, 2, 7),
            ("valu", 4, 1, 8, 1, 1), ("valu", 8, 4, 8, 0, 0), ("valu", 2, 2, 4, 1, 0)]


def random_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        C = int(rng.choice([int(rng.integers(1, 257)), 32, 64, 96, 128, 256, int(rng.integers(30, 70))]))
        hd = int(rng.choice([int(rng.integers(1, 601)), 16, 64, 128, 256, int(rng.integers(1, 40))]))
        ld = hd + int(rng.choice([0, 0, 1, 2, 3, 4, int(rng.integers(0, 20))]))
        P = int(rng.integers(1, 6))
        T = int(rng.integers(1, 4))
        N = P * T + int(rng.integers(0, 3))             # trailing chunks belong to no step
        res = tuple(int(4 * rng.integers(0, 16)) for _ in range(3))
        plan = EXPLICIT[int(rng.integers(0, len(EXPLICIT)))]
        if plan is not None and plan[0] == "valu" and plan[1] > C:
            plan = None
        mode = int(rng.integers(0, 3))
        out.append((k, N, P, C, hd, ld, res, plan, mode))
    return out


@pytest.mark.parametrize("case", random_cases(40, 20261202), ids=lambda c: f"case{c[0]}")
def test_random_shape(case):
    k, N, P, C, hd, ld, res, plan, mode = case
    x, dv, du = inputs.shape_inputs(N, C, hd, ld, ("normal", "hazard_cancel", "hazard_special")[k % 3], seed=1000 + k)
    dc = DeviceCase(x, dv, du, hd, res_u=res[0], res_x=res[1], res_v=res[2])
    p = None
    if plan is not None:
        p = g.make_mfma_plan(*plan[1:]) if plan[0] == "mfma" else g.make_plan(*plan[1:])
    say(f"random case {k}: N={N} P={P} C={C} hd={hd} ld={ld} res={res} plan={plan} mode={mode}")
    g.sdm_gx_gemm_steps(dc.du, ld, dc.x, dc.dv, ld, N, P, C, hd, 0, N // P, mode, p)
    want = expected(x, dv, du, hd, 0, (N // P) * P)
    assert_matches(dc.result(), want, du, hd, f"random case {k}")
