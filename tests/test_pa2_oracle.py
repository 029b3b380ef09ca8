"""The Phase A CPU oracle against its independent pins (no GPU involved)."""

import numpy as np
import pytest

import oracle
from deterministic_fp32_gemm_amd import pa2_inputs as PI
from tests import pa2_pins
from tests.compare import assert_same_bits


@pytest.fixture(scope="session")
def pa2_lib():
    return oracle.load_pa2()


def test_fpenv_is_ieee(pa2_lib):
    assert oracle.pa2_fpenv_ok(pa2_lib)


@pytest.mark.parametrize("pin", pa2_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, pa2_lib):
    pin(pa2_lib)


def test_fixtures_load():
    names = [f["name"] for f in pa2_pins.fixtures()]
    assert names == ["group_walk.txt", "tree_and_rounding.txt"]


def test_record_generator_structure():
    """The generator's records: every (token, write) pair once per chunk, groups opened by FIRST and closed by LAST,
    distance fields back to the group's FIRST, distinct slots per group within a step, kpay equal to the payloads,
    and bpre the valid-FIRST counts before each 32-record block."""
    w = PI.Pa2Workload("g", 2, 3, 40, 7, 24, 24, 0, 4096, True, 5.0, 0.1, "structure", max_group=300)
    d = PI.inputs(w)
    pay = d["rec"][:, :, 0].view(np.uint32)
    assert (d["kpay"] == d["rec"][:, :, 0]).all()
    for k in range(w.N):
        t = (pay[k] >> 9) & 0xFF
        wr = pay[k] & 0xFF
        assert sorted((t * w.W + wr).tolist()) == list(range(w.n))
        first = (pay[k] & PI.FIRST) != 0
        last = (pay[k] & PI.LAST) != 0
        assert first[0] and last[-1]
        starts = np.flatnonzero(first)
        ends = np.flatnonzero(last)
        assert (starts[1:] == ends[:-1] + 1).all() and starts.size == ends.size
        dist = (pay[k] >> 18) & 0xFFF
        for s, e in zip(starts, ends):
            assert (dist[s:e + 1] == np.minimum(np.arange(e + 1 - s), 4095)).all()
            assert (d["rec"][k, s:e + 1, 1] == d["rec"][k, s, 1]).all()
        vf = first & ((pay[k] & PI.INVALID) == 0)
        for b in range(d["bpre"].shape[1]):
            assert d["bpre"][k, b] == vf[:32 * b].sum()
    for ti in range(w.T):
        ks = range(ti * w.P, (ti + 1) * w.P)
        slots = [d["rec"][k, s, 1] for k in ks for s in np.flatnonzero(pay[k] & PI.FIRST)]
        assert len(slots) == len(set(slots))


def test_long_groups_set_the_far_distance():
    w = PI.Pa2Workload("l", 1, 1, 64, 80, 4, 4, 0, 16, True, 1e9, 0.0, "one group of all 5120 records")
    d = PI.inputs(w)
    pay = d["rec"][0, :, 0].view(np.uint32)
    assert ((pay >> 18) & 0xFFF).max() == 4095


def test_steps_in_order_chain_through_grad_rows(pa2_lib):
    """Steps reuse slots: a group of step 1 reads (at its FIRST) the grad row a group of step 0 wrote (at its LAST),
    so the steps run in order, each in place."""
    w = PI.Pa2Workload("o", 2, 2, 6, 3, 8, 8, 0, 40, True, 3.0, 0.0, "order")
    d = PI.inputs(w)
    grad, bank = d["grad"].copy(), d["bank"].copy()
    eff = np.zeros((1, w.N * w.n), np.float32)
    g = eff.copy()
    for ti in range(w.T):
        oracle.pa2_step(grad, bank, d["snap"], -1, d["du"], d["beta"], d["rec"], eff, g, ti, w.P, w.C, w.W, w.hd,
                        lib=pa2_lib)
    g1 = d["grad"].copy()
    oracle.pa2_step(g1, d["bank"].copy(), d["snap"], -1, d["du"], d["beta"], d["rec"], eff.copy(), g.copy(), 1,
                    w.P, w.C, w.W, w.hd, lib=pa2_lib)
    shared = set(d["rec"][:w.P, :, 1].ravel()) & set(d["rec"][w.P:, :, 1].ravel())
    assert shared                                     # the two steps share slots (40 slots, ~12 groups a step)
    assert not np.array_equal(grad.view(np.uint32), g1.view(np.uint32))


def test_invalid_arguments(pa2_lib):
    fx = pa2_pins.fixtures()[0]
    dims = fx["dims"]
    eff = np.zeros((1, 4), np.float32)
    for kw in (dict(ti=1), dict(P=2), dict(C=3), dict(W=3)):
        a = dict(ti=0, P=dims["P"], C=dims["C"], W=dims["W"])
        a.update(kw)
        with pytest.raises(ValueError):
            oracle.pa2_step(fx["grad"].copy(), fx["bank"].copy(), fx["snap"], -1, fx["du"], fx["beta"], fx["rec"],
                            eff, eff.copy(), a["ti"], a["P"], a["C"], a["W"], dims["hd"], lib=pa2_lib)


def test_outputs_of_other_chunks_untouched(pa2_lib):
    w = PI.PA2_WORKLOADS["a1"]
    d = PI.inputs(w)
    eff = np.full((1, w.N * w.n), 77.0, np.float32)
    g = eff.copy()
    grad = d["grad"].copy()
    oracle.pa2_step(grad, d["bank"].copy(), d["snap"], d["ssr"], d["du"], d["beta"], d["rec"], eff, g, 0, 1, w.C,
                    w.W, w.hd, lib=pa2_lib)
    assert_same_bits(eff[:, w.n:], np.full((1, w.n), 77.0, np.float32), "chunk 1 outputs")
    assert (eff[:, :w.n] != 77.0).all()
