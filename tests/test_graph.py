"""HIP graphs of prepared step ranges: replays give the oracle's bits every time (each replay applies the update
again), with the program's own eager work and synchronisations between replays; per-step and fused graphs; both
engines; the empty range."""

import numpy as np
import pytest

import deterministic_fp32_gemm_amd as g
from deterministic_fp32_gemm_amd import inputs
from tests.gpu_util import DeviceCase, assert_matches, expected, say

pytestmark = pytest.mark.gpu

SHAPES = [  # N, P, C, hd, ld, residues, engine expected from the planner
    (16, 4, 64, 64, 64, (0, 0, 0), g.SDM_GX_ENGINE_MFMA),
    (12, 3, 100, 96, 99, (4, 8, 12), g.SDM_GX_ENGINE_MFMA),
    (8, 2, 16, 40, 41, (8, 4, 0), g.SDM_GX_ENGINE_VALU),
    (6, 2, 64, 256, 260, (4, 0, 4), g.SDM_GX_ENGINE_MFMA),      # rows 4 bytes past a 16-byte boundary
    (6, 2, 64, 200, 201, (4, 0, 4), g.SDM_GX_ENGINE_VALU),
]


@pytest.mark.parametrize("N,P,C,hd,ld,res,engine", SHAPES)
@pytest.mark.parametrize("mode", [g.SDM_GX_STEPS_FORWARD, g.SDM_GX_STEPS_REVERSE, g.SDM_GX_STEPS_FUSED])
def test_graph_replays_match_the_oracle(N, P, C, hd, ld, res, engine, mode):
    import torch
    x, dv, du = inputs.shape_inputs(N, C, hd, ld, "hazard_cancel", seed=N + C + hd + mode)
    case = DeviceCase(x, dv, du, hd, res_u=res[0], res_x=res[1], res_v=res[2])
    step = g.make_step(case.du.view(N, C, ld)[:, :, :hd], case.x.view(N, C, C), case.dv.view(N, C, ld)[:, :, :hd], P)
    assert step.geom["fused"]["engine"] == engine
    graph = step.graph(0, N // P, mode)
    assert graph.nodes == (1 if mode == g.SDM_GX_STEPS_FUSED else N // P)
    side = torch.zeros(1 << 20, device="cuda")
    want = du.copy()
    for replay in range(3):
        say(f"graph N={N} C={C} hd={hd} mode={mode} replay {replay}")
        graph.launch()
        side.add_(1.0)                                   # the program's own eager work between replays
        torch.cuda.synchronize()
        want = expected(x, dv, want, hd, 0, (N // P) * P)
        assert_matches(case.result(), want, du, hd, f"graph mode {mode} replay {replay}")
    assert float(side[0]) == 3.0
    graph.close()
    with pytest.raises(ValueError):
        graph.launch()


def test_graph_of_a_step_subrange_and_empty_range():
    N, P, C, hd = 12, 3, 64, 128
    x, dv, du = inputs.shape_inputs(N, C, hd, None, "normal", seed=31)
    case = DeviceCase(x, dv, du, hd)
    step = g.make_step(case.du.view(N, C, hd), case.x.view(N, C, C), case.dv.view(N, C, hd), P)
    empty = step.graph(2, 2, g.SDM_GX_STEPS_FORWARD)
    assert empty.nodes == 0
    empty.launch()
    sub = step.graph(1, 3, g.SDM_GX_STEPS_REVERSE)      # steps 2 then 1
    sub.launch()
    import torch
    torch.cuda.synchronize()
    assert_matches(case.result(), expected(x, dv, du, hd, 1 * P, 3 * P), du, hd, "graph steps 1..2")
    with pytest.raises(ValueError):
        step.graph(0, N // P + 1)
    with pytest.raises(ValueError):
        step.graph(2, 1)
