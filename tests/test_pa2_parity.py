"""GPU parity of Phase A (sdm_pa2_*, through the C ABI) against its CPU oracle, element by element.

Bar: grad, bank, out_eff and out_g bit-identical to the oracle wherever the oracle's value is not NaN, NaN where it
is NaN; rows no valid LAST names and outputs of other chunks keep their bytes.
"""

import numpy as np
import pytest

import deterministic_fp32_gemm_amd as g
from deterministic_fp32_gemm_amd import pa2_inputs as PI
from deterministic_fp32_gemm_amd.step import aligned_empty
from tests.compare import mismatch_report, same_bits
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the parity tests need an MI355X")
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    g.load()
    yield
    torch.cuda.synchronize()


class Pa2Case:
    """A workload's host arrays on the device (d_u at the workload's byte offset), and the oracle beside it."""

    def __init__(self, w: PI.Pa2Workload, pattern="normal", seed=0, d=None):
        import torch
        self.w = w
        self.h = d if d is not None else PI.inputs(w, pattern, seed)
        h = self.h
        dev = "cuda"
        self.grad = torch.from_numpy(h["grad"]).to(dev)
        self.bank = torch.from_numpy(h["bank"]).to(dev)
        self.snap = torch.from_numpy(h["snap"]).to(dev)
        du = aligned_empty(h["du"].size, w.du_offset_bytes)
        du.copy_(torch.from_numpy(h["du"].reshape(-1)))
        self.du = du.view(h["du"].shape)
        self.beta = torch.from_numpy(h["beta"]).to(dev)
        self.kpay = torch.from_numpy(h["kpay"]).to(dev)
        self.rec = torch.from_numpy(h["rec"]).to(dev)
        self.bpre = torch.from_numpy(h["bpre"]).to(dev) if h["ssr"] < 0 else None
        shape = (h["planes"], w.N * w.n)
        self.eff0 = np.full(shape, 77.0, np.float32)
        self.eff = torch.from_numpy(self.eff0).to(dev)
        self.gout = torch.from_numpy(self.eff0).to(dev)
        self.args = g.pa2_args(self.grad, self.bank, self.snap, h["ssr"], self.du, self.beta, self.kpay, self.rec,
                               self.bpre, self.eff, self.gout, w.P, w.C, w.W, w.hd, ld_u=w.ld_u)
        torch.cuda.synchronize()

    def expect(self, steps):
        import oracle
        h, w = self.h, self.w
        grad, bank = h["grad"].copy(), h["bank"].copy()
        eff, gout = self.eff0.copy(), self.eff0.copy()
        for ti in steps:
            oracle.pa2_step(grad, bank, h["snap"], h["ssr"], h["du"], h["beta"], h["rec"], eff, gout, ti, w.P, w.C,
                            w.W, w.hd)
        return grad, bank, eff, gout

    def result(self):
        import torch
        torch.cuda.synchronize()
        return self.grad.cpu().numpy(), self.bank.cpu().numpy(), self.eff.cpu().numpy(), self.gout.cpu().numpy()


def assert_same(got, want, what):
    for name, a, b in zip(("grad", "bank", "out_eff", "out_g"), got, want):
        ok = same_bits(a, b)
        if not ok.all():
            raise AssertionError(f"{what} {name}: " + mismatch_report(a, b, ok))


@pytest.mark.parametrize("key,pattern", [("a1", "normal"), ("a1", "special"), ("a1", "subnormal"), ("a3", "normal"),
                                         ("a3", "special"), ("a5", "normal"), ("a5", "special")])
def test_workload_steps_in_order(key, pattern):
    """Every step of the workload in order (steps reuse grad rows: each reads what earlier steps wrote)."""
    w = PI.PA2_WORKLOADS[key]
    say(f"phase A workload {key} pattern {pattern}: T={w.T} P={w.P} C={w.C} W={w.W} hd={w.hd}")
    c = Pa2Case(w, pattern)
    g.sdm_pa2_steps(c.args, 0, w.T, g.SDM_GX_STEPS_FORWARD)
    assert_same(c.result(), c.expect(range(w.T)), f"{key} {pattern}")


def test_reverse_steps():
    """The backward's order: steps descending, each in place."""
    w = PI.PA2_WORKLOADS["a3"]
    c = Pa2Case(w, "normal", seed=4)
    say("phase A a3 reverse")
    g.sdm_pa2_steps(c.args, 0, w.T, g.SDM_GX_STEPS_REVERSE)
    assert_same(c.result(), c.expect(reversed(range(w.T))), "a3 reverse")


EDGE = [
    # key, T, P, C, W, hd, ld_u, offset, slots, dense, mean group, invalid, max group
    ("hd7", 1, 3, 16, 8, 7, 9, 4, 256, True, 3.0, 0.1, 1 << 16),        # hd % 4 != 0, one lane partly used
    ("hd133", 1, 2, 12, 6, 133, 140, 8, 128, False, 2.0, 0.1, 1 << 16),  # two slices, the second ragged
    ("hd300", 2, 2, 8, 5, 300, 300, 0, 128, True, 4.0, 0.05, 1 << 16),   # three slices: a pair and a single
    ("c200", 1, 2, 200, 2, 256, 260, 4, 1024, True, 3.0, 0.05, 1 << 16),  # C > 128 with two slices: one per wave
    ("long", 1, 1, 64, 80, 36, 36, 0, 64, True, 1e9, 0.0, 1 << 16),       # one group of 5120 records (scan back)
    ("long2", 1, 2, 64, 72, 20, 20, 0, 64, False, 2500.0, 0.01, 4500),   # groups around 4095 records
    ("w1", 2, 3, 1, 1, 128, 128, 0, 16, True, 1.0, 0.0, 1 << 16),        # one record per chunk
    ("c256", 1, 1, 256, 3, 64, 64, 0, 512, True, 8.0, 0.3, 1 << 16),     # C = 256, many invalid records
]


@pytest.mark.parametrize("case", EDGE, ids=lambda e: e[0])
def test_edge_shapes(case):
    key, T, P, C, W, hd, ld, off, slots, dense, mean, inv, mg = case
    w = PI.Pa2Workload(key, T, P, C, W, hd, ld, off, slots, dense, mean, inv, key, max_group=mg)
    for pattern in ("normal", "special"):
        say(f"phase A edge {key} {pattern}")
        c = Pa2Case(w, pattern)
        g.sdm_pa2_steps(c.args, 0, w.T, g.SDM_GX_STEPS_FORWARD)
        assert_same(c.result(), c.expect(range(w.T)), f"edge {key} {pattern}")


def test_every_plan_gives_the_same_bits():
    """Slices per wavefront, wavefronts per workgroup and tile lengths (1 record .. the whole chunk) regroup the same
    walk: the bits never change."""
    import torch
    w = PI.Pa2Workload("plans", 1, 3, 24, 6, 260, 264, 4, 256, True, 3.0, 0.1, "plans")
    c = Pa2Case(w, "special", seed=9)
    want = c.expect([0])
    n = 0
    for sg in (1, 2):
        for waves in (4, 8, 16):
            for L in (1, 3, 8, 31, 64, 100, w.n):
                plan = g.make_pa2_plan(sg, waves, L)
                plan.stage_out = 1                      # an output of the plan's completion: the input is ignored
                c.grad.copy_(torch.from_numpy(c.h["grad"]))
                c.bank.copy_(torch.from_numpy(c.h["bank"]))
                c.eff.fill_(77.0)
                c.gout.fill_(77.0)
                say(f"phase A plan sg={sg} waves={waves} L={L}")
                g.sdm_pa2_step(c.args, 0, plan)
                assert_same(c.result(), want, f"plan sg={sg} waves={waves} L={L}")
                n += 1
    assert n == 42


@pytest.mark.parametrize("mode", ["forward", "reverse"])
def test_gathered_outputs_over_steps(mode):
    """Outputs gathered in LDS (one workgroup per chunk, two slices, d_u rows off a 16-byte boundary), over three
    steps in either order; the outputs of the chunks a step does not cover keep their bytes."""
    w = PI.Pa2Workload("gather", 3, 2, 16, 8, 256, 260, 4, 256, False, 3.0, 0.05, "gather")
    c = Pa2Case(w, "special", seed=5)
    # 16 tiles of 8 records: one workgroup holds each chunk; its 4 output planes (2 KiB) add an eighth to the 16 KiB
    # of token rows, so they are gathered in LDS
    plan = g.make_pa2_plan(2, 16, 8)
    say(f"phase A gathered outputs {mode}")
    order = range(w.T) if mode == "forward" else reversed(range(w.T))
    g.sdm_pa2_steps(c.args, 0, w.T, g.SDM_GX_STEPS_FORWARD if mode == "forward" else g.SDM_GX_STEPS_REVERSE, plan)
    assert_same(c.result(), c.expect(order), f"gathered outputs {mode}")


def test_planner_plans():
    for key, sg in (("a1", 1), ("a3", 1), ("a5", 2)):
        w = PI.PA2_WORKLOADS[key]
        c = Pa2Case(w)
        p = g.sdm_pa2_plan_for(c.args)
        say(f"phase A plan {key}: {p.as_dict()}")
        assert p.slices_per_wave == sg and p.grid == w.P * p.npair * p.ctas


def test_errors_launch_nothing():
    import torch
    w = PI.PA2_WORKLOADS["a1"]
    c = Pa2Case(w)
    before = c.result()
    bad = g.pa2_args(c.grad, c.bank, c.snap, -1, c.du, c.beta, c.kpay, c.rec, c.bpre, c.eff, c.gout, w.P, w.C, w.W,
                     w.hd, ld_u=w.ld_u)
    bad.out_g = bad.grad                                       # written arrays overlap
    with pytest.raises(ValueError):
        g.sdm_pa2_step(bad, 0)
    with pytest.raises(ValueError):
        g.sdm_pa2_step(c.args, 1)                             # ti >= N / P
    torch.cuda.synchronize()
    for a, b in zip(c.result(), before):
        assert (a.view(np.uint32) == b.view(np.uint32)).all()
