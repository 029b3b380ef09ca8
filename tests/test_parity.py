"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle, element by element.

Bar: every non-NaN output bit-identical to the oracle, NaN outputs NaN on both sides, padding columns and chunks
outside the requested steps untouched (bit for bit).
"""

import numpy as np
import pytest

import deterministic_fp32_gemm_amd as g
from deterministic_fp32_gemm_amd import inputs
from tests.gpu_util import DeviceCase, assert_matches, expected, say, workload_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the parity tests need an MI355X")
    arch = torch.cuda.get_device_properties(0).gcnArchName
    assert arch.startswith("gfx950"), arch
    g.load()
    yield
    torch.cuda.synchronize()


def run_steps(case: DeviceCase, P, ti_begin, ti_end, mode, plan=None):
    du, ld_u, x, dv, ld_dv, N = case.args()
    g.sdm_gx_gemm_steps(du, ld_u, x, dv, ld_dv, N, P, case.C, case.hd, ti_begin, ti_end, mode, plan)
    return case.result()


# ---- the five workloads ----------------------------------------------------------------------------------------------
WORKLOAD_PATTERNS = [(1, p) for p in inputs.ALL_PATTERNS] + [(2, p) for p in inputs.ALL_PATTERNS] + \
    [(3, p) for p in inputs.ALL_PATTERNS] + [(4, "normal"), (4, "hazard_special"), (4, "hazard_subnormal")] + \
    [(5, "normal"), (5, "hazard_special"), (5, "nan")]


@pytest.mark.parametrize("key,pattern", WORKLOAD_PATTERNS, ids=lambda v: str(v))
def test_workload_steps_in_order(key, pattern):
    """All T steps in order ti = 0..T-1 (one launch per step), then the whole d_u against the oracle."""
    w, case = workload_case(key, pattern)
    say(f"workload {key} pattern {pattern}: N={w.N} P={w.P} C={w.C} hd={w.hd} ld={w.ld}")
    got = run_steps(case, w.P, 0, w.T, g.SDM_GX_STEPS_FORWARD)
    want = expected(case.x_h, case.dv_h, case.du_h, w.hd, 0, w.N)
    assert_matches(got, want, case.du_h, w.hd, f"workload {key} {pattern}")


@pytest.mark.parametrize("pattern", inputs.PATTERNS)
def test_workload3_after_every_step(pattern):
    """The six value patterns, compared with the oracle after every one of the T steps."""
    w, case = workload_case(3, pattern)
    want = case.du_h.copy()
    import oracle
    for ti in range(w.T):
        say(f"workload 3 pattern {pattern} step {ti}")
        g.sdm_gx_gemm_ex(*case.args()[:5], w.N, ti, w.P, w.C, w.hd)
        oracle.gx_gemm_chunks(want, case.x_h, case.dv_h, ti * w.P, (ti + 1) * w.P, w.hd, threads=8)
        assert_matches(case.result(), want, case.du_h, w.hd, f"workload 3 {pattern} after step {ti}")


@pytest.mark.parametrize("key", [1, 2, 3, 4, 5])
def test_workload_bench_launch(key):
    """The launch configuration the benchmark times (a prepared launch, all T steps fused into one launch, repeated
    three times back to back so d_u accumulates) against the oracle applying the same three sweeps."""
    import torch
    w, case = workload_case(key)
    say(f"workload {key} fused x3")
    N, C, hd = w.N, w.C, w.hd
    du_t = case.du.view(N, C, w.ld)[:, :, :hd]
    dv_t = case.dv.view(N, C, w.ld)[:, :, :hd]
    x_t = case.x.view(N, C, C)
    step = g.make_step(du_t, x_t, dv_t, w.P)
    for _ in range(3):
        step.fused(0, w.T)
    torch.cuda.synchronize()
    want = case.du_h.copy()
    for _ in range(3):
        want = expected(case.x_h, case.dv_h, want, hd, 0, N)
    assert_matches(case.result(), want, case.du_h, hd, f"workload {key} fused x3")


@pytest.mark.parametrize("key,pattern", [(k, p) for k in (2, 3, 4, 5) for p in inputs.PATTERNS + ("hazard_subnormal",)
                                         if p != "normal"], ids=lambda v: str(v))
def test_workload_bench_launch_patterns(key, pattern):
    """The benchmark's launch configuration (prepared launch, all T steps in one fused launch, the planner's plan
    for the whole workload) on the six value patterns and the subnormal-accumulation probe, against the oracle."""
    import torch
    w, case = workload_case(key, pattern)
    say(f"workload {key} pattern {pattern} fused")
    N, C, hd = w.N, w.C, w.hd
    step = g.make_step(case.du.view(N, C, w.ld)[:, :, :hd], case.x.view(N, C, C), case.dv.view(N, C, w.ld)[:, :, :hd],
                       w.P)
    step.fused(0, w.T)
    torch.cuda.synchronize()
    want = expected(case.x_h, case.dv_h, case.du_h, hd, 0, N)
    assert_matches(case.result(), want, case.du_h, hd, f"workload {key} {pattern} fused")


@pytest.mark.parametrize("key,res_x", [(k, 0) for k in (1, 2, 3, 4, 5)] + [(5, 8), (3, 4), (4, 12)])
def test_prepared_plan_is_the_planners(key, res_x):
    """The plan a prepared launch stores (and runs) is the plan sdm_gx_plan reports for the same strides and
    placements, unaligned-row instance included."""
    w, case = workload_case(key, res_x=res_x)
    N, C, hd = w.N, w.C, w.hd
    step = g.make_step(case.du.view(N, C, w.ld)[:, :, :hd], case.x.view(N, C, C), case.dv.view(N, C, w.ld)[:, :, :hd],
                       w.P)
    xm, dm = case.x.data_ptr() % 16, case.dv.data_ptr() % 16
    for which, nchunks in (("step", w.P), ("fused", N)):
        want = g.sdm_gx_plan(nchunks, C, hd, w.ld, w.ld, xm, dm).as_dict()
        got = dict(step.geom[which])
        want.pop("wgs_per_cu")
        got.pop("wgs_per_cu")
        assert got == want, (which, got, want)
    if key == 5:
        assert (step.geom["fused"]["mf_block"], step.geom["fused"]["mf_aln"]) == (32, 4 if res_x == 0 else 3)


# ---- every plan gives the same bits --------------------------------------------------------------------------------
def all_plans(C, hd=64):
    """Every plan the library has a kernel instance for (plans without one are rejected by the library): every
    vector-ALU tile and staging, and every matrix-core instance with one workgroup per CU and with two workgroups in
    all (so that each walks several work items)."""
    for ri in (1, 2, 4, 8, 16, 32):
        if ri > C:
            continue
        for rc in (1, 2, 4):
            for waves in (1, 2, 4, 8, 16):
                for staging in (0, 1):
                    for xcd in (0, 1):
                        slab = (0, 5) if staging else (0,)
                        for sj in slab:
                            plan = g.make_plan(ri, rc, waves, staging, xcd, sj)
                            try:
                                g.sdm_gx_plan_complete(type(plan).from_buffer_copy(plan), 1, C, hd)
                            except ValueError:
                                continue
                            yield plan
    for rw in (1, 2):
        for cw in (1, 2, 4, 8):
            for stages, rs, lw, blk, j in ((4, 2, 2, 32, 16), (4, 2, 4, 32, 16), (4, 4, 2, 32, 16), (4, 4, 4, 32, 16),
                                           (4, 0, 1, 32, 16), (8, 0, 2, 32, 16), (3, 0, 1, 16, 16), (8, 0, 2, 16, 16),
                                           (3, 0, 1, 16, 32), (3, 0, 1, 32, 32), (3, 0, 2, 32, 32)):
                for de in (0, 1):
                    for wgs in (0, 2):
                        plan = g.make_mfma_plan(rw, cw, stages, rs, lw, wgs, de, blk, j)
                        try:
                            g.sdm_gx_plan_complete(type(plan).from_buffer_copy(plan), 1, C, hd)
                        except ValueError:
                            continue
                        yield plan


def dma_plans():
    """Matrix-core plans whose slabs go straight to LDS (mf_reg_slabs 0), several work items per workgroup."""
    return [g.make_mfma_plan(rw, cw, s, 0, lw, wgs, 0) for rw, cw in ((1, 1), (1, 2), (1, 4), (1, 8), (2, 1), (2, 2),
                                                                      (2, 4)) for s, lw, wgs in ((4, 1, 3), (8, 2, 0))] \
        + [g.make_mfma_plan(2, 4, 4, 0, 1, 5, 1)] \
        + [g.make_mfma_plan(rw, cw, s, 0, lw, wgs, 0, 16, j) for rw, cw in ((1, 2), (1, 4), (1, 8), (2, 2), (2, 4))
           for s, lw, wgs, j in ((3, 1, 3, 16), (8, 2, 0, 16), (3, 1, 2, 32))] \
        + [g.make_mfma_plan(1, 4, 3, 0, 1, 0, 0, 16, 16, 1), g.make_mfma_plan(2, 2, 3, 0, 1, 3, 0, 16, 32, 1)] \
        + [g.make_mfma_plan(1, 4, 3, 0, 1, 3, 0, 32, 32), g.make_mfma_plan(1, 4, 3, 0, 2, 3, 0, 32, 32)]


@pytest.mark.parametrize("C,hd,ld,res", [(37, 150, 157, 4), (64, 256, 260, 4), (16, 16, 16, 0), (5, 300, 301, 8),
                                        (100, 72, 76, 0), (36, 40, 44, 0)])
def test_every_plan_is_bit_identical(C, hd, ld, res):
    N, P = 6, 3
    x, dv, du = inputs.shape_inputs(N, C, hd, ld, "hazard_cancel", seed=C + hd)
    case = DeviceCase(x, dv, du, hd, res_u=res, res_v=res, res_x=(res * 3) % 256)
    want = expected(x, dv, du, hd, 0, N)
    n = 0
    for plan in all_plans(C):
        case.reset()
        say(f"plan {plan} C={C} hd={hd} ld={ld}")
        got = run_steps(case, P, 0, N // P, g.SDM_GX_STEPS_FORWARD, plan)
        assert_matches(got, want, du, hd, f"plan {plan}")
        n += 1
    assert n > 100



@pytest.mark.parametrize("res_v", [4, 8, 12])
def test_unaligned_dv_rows_with_aligned_x(res_v):
    """x on a 16-byte boundary and d_dv (and d_u) off it, as in workload 5: the instances that move d_dv rows by 4-byte
    DMA (the 64 x 128 items of 32-column wavefronts with two loader wavefronts, the 16-column ones) and those that
    read them from the boundary below, each against the oracle; ragged C and hd tails, several items per
    workgroup."""
    N, P, C, hd, ld = 12, 4, 60, 250, 252
    x, dv, du = inputs.shape_inputs(N, C, hd, ld, "hazard_cancel", seed=res_v)
    case = DeviceCase(x, dv, du, hd, res_u=res_v, res_v=res_v, res_x=0)
    want = expected(x, dv, du, hd, 0, N)
    plans = [None, g.make_mfma_plan(1, 4, 3, 0, 2, 3, 0, 32, 32), g.make_mfma_plan(1, 4, 3, 0, 1, 3, 0, 32, 32),
             g.make_mfma_plan(1, 4, 3, 0, 1, 3, 0, 16, 32), g.make_mfma_plan(1, 4, 3, 0, 1, 3, 0, 16, 16),
             g.make_mfma_plan(1, 8, 3, 0, 1, 3, 0, 16, 32)]
    seen = set()
    for plan in plans:
        case.reset()
        say(f"unaligned d_dv +{res_v}: plan {plan}")
        got = run_steps(case, P, 0, N // P, g.SDM_GX_STEPS_FUSED, plan)
        assert_matches(got, want, du, hd, f"d_dv +{res_v} plan {plan}")
        geom = g.sdm_gx_plan_complete(type(plan).from_buffer_copy(plan), N, C, hd, ld_u=ld, ld_dv=ld,
                                      dv_mod16=res_v % 16) if plan is not None else None
        if geom is not None:
            seen.add((geom.mf_block, geom.mf_loader_waves, geom.mf_aln))
    assert (32, 2, 4) in seen and (32, 1, 2) in seen and (16, 1, 4) in seen

@pytest.mark.parametrize("C", [1, 5, 16, 17, 20, 33, 64, 65, 128, 130])
def test_signed_zero_through_padded_steps(C):
    """Products that round to -0 keep the accumulator at -0, and -0 + -0 stays -0 in d_u. The matrix-core engine
    pads the last slab's chain rows (and items' missing rows) with a -0 product, which must leave such an
    accumulator untouched; a +0 padding product would turn the result into +0."""
    N, P, hd, ld = 4, 2, 40, 44
    x = np.full((N, C, C), -1e-30, np.float32)
    dv = np.full((N, C, ld), 1e-30, np.float32)
    du = np.full((N, C, ld), -0.0, np.float32)
    du[:, :, hd:] = np.float32(3.5)                            # padding columns: must stay untouched
    want = expected(x, dv, du, hd, 0, N)
    assert (np.signbit(want[:, :, :hd])).all() and (want[:, :, :hd] == 0).all()
    plans = [None, g.make_mfma_plan(1, 2, 4, 4, 2), g.make_mfma_plan(2, 1, 4, 2, 4, 1), g.make_plan(1, 1, 2, 1, 1),
             g.make_mfma_plan(1, 2, 4, 0, 1), g.make_mfma_plan(2, 1, 8, 0, 2, 1),
             g.make_mfma_plan(1, 4, 3, 0, 1, 0, 0, 16, 16)]
    for res in ((4, 8, 12), (0, 0, 0)):             # direct-to-LDS slabs need the aligned layout
        case = DeviceCase(x, dv, du, hd, res_u=res[0], res_v=res[1], res_x=res[2])
        for plan in plans:
            case.reset()
            say(f"signed zero C={C} res {res} plan {plan}")
            got = run_steps(case, P, 0, N // P, g.SDM_GX_STEPS_FUSED, plan)
            assert_matches(got, want, du, hd, f"signed zero C={C} res {res} plan {plan}")


@pytest.mark.parametrize("C,plan", [(2, (1, 2, 4, 4, 2)),                                  # 32x32x1, register ring
                                    (4, (1, 4, 3, 0, 1, 0, 0, 16, 32))])                  # 16x16x1, direct to LDS
def test_mfma_engine_single_rounding(C, plan):
    """Two-step chains on near-cancelling inputs: acc = fma(x1, d1, fl(x0*d0)), where a fused and an unfused second
    step round differently for a large share of the outputs. The matrix-core engine (one K=1 MFMA per step, each
    MFMA shape) must give the fused result: the oracle's fmaf chain, bit for bit. With C = 4 the chain's last two
    steps have x = 0 (slabs straight to LDS need C % 4 == 0)."""
    rng = np.random.default_rng(2026)
    N, P, hd = 512, 8, 64
    x = rng.standard_normal((N, C, C)).astype(np.float32)
    x[:, 2:, :] = 0
    dv = rng.standard_normal((N, C, hd)).astype(np.float32)
    # row 1 nearly cancels row 0's product for output row 0: x[n,1,0]*dv[n,1,c] ~ -x[n,0,0]*dv[n,0,c]
    dv[:, 1, :] = (-(x[:, 0, 0:1].astype(np.float64) * dv[:, 0, :]) / x[:, 1, 0:1]).astype(np.float32)
    du = np.zeros((N, C, hd), np.float32)
    want = expected(x, dv, du, hd, 0, N)
    p0 = (x[:, 0, 0:1] * dv[:, 0, :]).astype(np.float32)                 # fl(x0*d0): float32 products
    unfused = (p0 + (x[:, 1, 0:1] * dv[:, 1, :]).astype(np.float32)).astype(np.float32)
    differ = unfused.view(np.uint32) != want[:, 0, :].view(np.uint32)
    assert differ.mean() > 0.2, differ.mean()                             # the test has teeth
    case = DeviceCase(x, dv, du, hd)
    got = run_steps(case, P, 0, N // P, g.SDM_GX_STEPS_FUSED, g.make_mfma_plan(*plan))
    assert_matches(got, want, du, hd, f"mfma single rounding C={C} plan {plan}")


@pytest.mark.parametrize("C,hd,ld,res", [(148, 70, 76, (0, 0, 0)), (64, 64, 64, (0, 0, 0)), (128, 128, 128, (4, 0, 0)),
                                        (36, 100, 104, (0, 0, 0)), (64, 128, 131, (0, 4, 0)), (148, 70, 76, (0, 0, 8)),
                                        (64, 256, 260, (4, 4, 0)), (64, 64, 68, (0, 12, 4)), (36, 100, 104, (8, 4, 12)),
                                        (100, 33, 36, (0, 8, 0)), (128, 40, 44, (12, 0, 4))])
def test_mfma_direct_to_lds_plans(C, hd, ld, res):
    """Slabs moved straight from memory into LDS (mf_reg_slabs 0): ragged rows, columns and last slabs (C % 16 != 0
    runs only the chain's own steps), several items per workgroup, per step and fused. Rows that start 4, 8 or 12
    bytes past a 16-byte boundary (x or d_dv base off, C and ld multiples of 4) load from the boundary below and
    skip the first floats of each LDS row (the unaligned-row instances); with ld 131 the rows cannot share one offset
    and the launch takes the register ring. Same bits in every case."""
    N, P = 12, 4
    x, dv, du = inputs.shape_inputs(N, C, hd, ld, "hazard_cancel", seed=C * 3 + hd)
    case = DeviceCase(x, dv, du, hd, res_u=res[0], res_v=res[1], res_x=res[2])
    want = expected(x, dv, du, hd, 0, N)
    for plan in dma_plans():
        for mode in (g.SDM_GX_STEPS_FORWARD, g.SDM_GX_STEPS_FUSED):
            case.reset()
            say(f"direct-to-LDS C={C} hd={hd} ld={ld} res={res} plan {plan} mode {mode}")
            got = run_steps(case, P, 0, N // P, mode, plan)
            assert_matches(got, want, du, hd, f"direct-to-LDS plan {plan} mode {mode}")


@pytest.mark.parametrize("C,ld,plan", [
    (1, None, None), (3, None, None),
    (32, 1 << 20, ("mfma", 1, 4, 3, 0, 1, 0, 0, 16, 16)),     # direct-to-LDS (rows 16-byte aligned)
    (32, None, ("mfma", 1, 4, 3, 0, 1, 0, 0, 16, 32)),        # ld = hd = 2^20 - 1: runs through the register ring
    (33, None, ("valu", 4, 4, 8, 0)),
])
def test_widest_hd(C, ld, plan):
    """hd = 2^20 - 1, the largest row the checks accept, on both engines; the oracle runs on a sample of columns
    (each output column's chain reads only that column of d_dv), including the last ones."""
    N, P, hd = 2, 1, (1 << 20) - 1
    ld = ld or hd
    x, dv, du = inputs.shape_inputs(N, C, hd, ld, "normal", seed=C + ld)
    case = DeviceCase(x, dv, du, hd)
    if plan is not None:
        plan = g.make_mfma_plan(*plan[1:]) if plan[0] == "mfma" else g.make_plan(*plan[1:])
    say(f"widest hd C={C} ld={ld} plan {plan}")
    got = run_steps(case, P, 0, N // P, g.SDM_GX_STEPS_FUSED, plan)
    rng = np.random.default_rng(C)
    cols = np.unique(np.concatenate([rng.integers(0, hd, 1500), np.arange(hd - 70, hd), np.arange(0, 70)]))
    want = expected(x, np.ascontiguousarray(dv[:, :, cols]), np.ascontiguousarray(du[:, :, cols]), len(cols), 0, N)
    assert_matches(np.ascontiguousarray(got[:, :, cols]), want, du[:, :, cols], len(cols), f"widest hd C={C}")
    if ld > hd:
        assert (got.view(np.uint32)[:, :, hd:] == du.view(np.uint32)[:, :, hd:]).all(), "padding column written"


def test_mfma_engine_many_items_per_workgroup():
    """Persistent matrix-core workgroups walking long ranges of work items (chunks x row groups x column groups),
    ragged in rows and columns, per step and fused."""
    N, P, C, hd, ld = 30, 5, 150, 70, 73
    x, dv, du = inputs.shape_inputs(N, C, hd, ld, "hazard_cancel", seed=77)
    case = DeviceCase(x, dv, du, hd, res_u=4, res_v=0, res_x=8)
    want = expected(x, dv, du, hd, 0, N)
    for plan in (g.make_mfma_plan(2, 2, 4, 4, 4, 3), g.make_mfma_plan(1, 1, 4, 2, 2, 7),
                 g.make_mfma_plan(1, 8, 4, 2, 2, 1), g.make_mfma_plan(2, 4, 4, 4, 4, 0),
                 g.make_mfma_plan(2, 4, 4, 2, 4, 5, 1), g.make_mfma_plan(1, 4, 4, 2, 4, 0, 1)):
        for mode in (g.SDM_GX_STEPS_FORWARD, g.SDM_GX_STEPS_FUSED):
            case.reset()
            say(f"mfma items plan {plan} mode {mode}")
            got = run_steps(case, P, 0, N // P, mode, plan)
            assert_matches(got, want, du, hd, f"mfma plan {plan} mode {mode}")


# ---- driver modes ----------------------------------------------------------------------------------------------------
def test_driver_modes_agree():
    N, P, C, hd, ld = 14, 4, 24, 70, 72              # N % P != 0: chunks 12, 13 belong to no step
    x, dv, du = inputs.shape_inputs(N, C, hd, ld, "hazard_wide", seed=5)
    case = DeviceCase(x, dv, du, hd, res_u=12, res_v=20, res_x=4)
    want = expected(x, dv, du, hd, 0, (N // P) * P)
    for mode in (g.SDM_GX_STEPS_FORWARD, g.SDM_GX_STEPS_REVERSE, g.SDM_GX_STEPS_FUSED):
        case.reset()
        say(f"mode {mode}")
        assert_matches(run_steps(case, P, 0, N // P, mode), want, du, hd, f"mode {mode}")
    # prepared launches: per step in reverse (the backward's order), and fused
    import torch
    du_t = case.du.view(N, C, ld)[:, :, :hd]
    dv_t = case.dv.view(N, C, ld)[:, :, :hd]
    step = g.make_step(du_t, case.x.view(N, C, C), dv_t, P)
    case.reset()
    for ti in reversed(range(N // P)):
        step(ti)
    assert_matches(case.result(), want, du, hd, "prepared per step")
    case.reset()
    step.fused(0, 1)
    step.fused(1, N // P)
    assert_matches(case.result(), want, du, hd, "prepared fused")
    torch.cuda.synchronize()


def test_contiguous_entry_point():
    """sdm_gx_gemm (no N, rows of hd floats) on step ti: only that step's chunks change."""
    N, P, C, hd, ti = 9, 3, 32, 96, 2
    x, dv, du = inputs.shape_inputs(N, C, hd, None, "normal", seed=6)
    case = DeviceCase(x, dv, du, hd)
    g.sdm_gx_gemm(case.du, case.x, case.dv, ti, P, C, hd)
    want = expected(x, dv, du, hd, ti * P, (ti + 1) * P)
    assert_matches(case.result(), want, du, hd, "sdm_gx_gemm")


# ---- edge shapes and alignment -------------------------------------------------------------------------------------
EDGE = [  # N, P, C, hd, ld, res_u, res_x, res_v, pattern
    (1, 1, 1, 1, 1, 0, 0, 0, "normal"),
    (2, 1, 1, 5, 7, 4, 8, 12, "hazard_special"),
    (3, 3, 3, 5, 5, 4, 4, 4, "normal"),
    (2, 2, 256, 1, 1, 0, 0, 0, "normal"),            # longest chain, one column
    (2, 2, 256, 260, 263, 4, 0, 8, "hazard_cancel"),  # longest chain, ragged columns
    (4, 2, 17, 4100, 4100, 0, 0, 0, "normal"),       # many column blocks with a tail
    (5, 2, 63, 129, 131, 252, 248, 244, "hazard_sparse"),
    (7, 7, 100, 3, 3, 8, 4, 0, "hazard_subnormal"),
    (3, 1, 33, 255, 255, 4, 4, 4, "inf"),
]


@pytest.mark.parametrize("N,P,C,hd,ld,ru,rx,rv,pattern", EDGE)
def test_edge_shapes(N, P, C, hd, ld, ru, rx, rv, pattern):
    x, dv, du = inputs.shape_inputs(N, C, hd, ld, pattern, seed=N + C + hd)
    case = DeviceCase(x, dv, du, hd, res_u=ru, res_x=rx, res_v=rv)
    say(f"edge N={N} P={P} C={C} hd={hd} ld={ld} res=({ru},{rx},{rv}) {pattern}")
    got = run_steps(case, P, 0, N // P, g.SDM_GX_STEPS_FUSED)
    want = expected(x, dv, du, hd, 0, (N // P) * P)
    assert_matches(got, want, du, hd, "edge")


@pytest.mark.parametrize("res", [(0, 0, 0), (4, 0, 0), (0, 4, 0), (0, 0, 4), (4, 8, 12), (12, 4, 8), (60, 124, 252),
                                 (128, 64, 32)])
def test_alignment_classes(res):
    """Every 4-byte residue class of the three base pointers (mod 256) gives the same bits; a 16-byte-aligned row
    stride keeps the class, an odd stride walks through all of them across rows."""
    N, P, C, hd = 4, 2, 32, 128
    for ld in (128, 129):
        x, dv, du = inputs.shape_inputs(N, C, hd, ld, "normal", seed=ld)
        case = DeviceCase(x, dv, du, hd, res_u=res[0], res_x=res[1], res_v=res[2])
        say(f"alignment {res} ld={ld}")
        got = run_steps(case, P, 0, N // P, g.SDM_GX_STEPS_FORWARD)
        assert_matches(got, expected(x, dv, du, hd, 0, N), du, hd, f"alignment {res} ld {ld}")


def test_repeated_runs_are_identical():
    w, case = workload_case(3, "hazard_cancel")
    first = run_steps(case, w.P, 0, w.T, g.SDM_GX_STEPS_FUSED)
    for _ in range(3):
        case.reset()
        again = run_steps(case, w.P, 0, w.T, g.SDM_GX_STEPS_FUSED)
        assert (again.view(np.uint32) == first.view(np.uint32)).all()


# ---- errors reach the caller and launch nothing --------------------------------------------------------------------
def test_errors_launch_nothing():
    import torch
    N, P, C, hd = 4, 2, 8, 8
    x, dv, du = inputs.shape_inputs(N, C, hd, None, "normal", seed=9)
    case = DeviceCase(x, dv, du, hd)
    with pytest.raises(ValueError):
        g.sdm_gx_gemm_ex(case.du, hd, case.x, case.dv, hd, N, 2, P, C, hd)           # ti >= N / P
    with pytest.raises(ValueError):
        g.sdm_gx_gemm_ex(case.du, hd, case.du, case.dv, hd, N, 0, P, C, hd)          # d_u overlaps x
    host = torch.zeros(N * C * hd)
    with pytest.raises(RuntimeError):                                               # a host pointer
        g.sdm_gx_gemm_ex(host.data_ptr(), hd, case.x, case.dv, hd, N, 0, P, C, hd)
    step = g.make_step(case.du.view(N, C, hd), case.x.view(N, C, C), case.dv.view(N, C, hd), P)
    with pytest.raises(ValueError):
        step(2)
    with pytest.raises(ValueError):
        g.sdm_gx_launch(step.prepared, 5)
    bad = g.sdm_gx_launch_t()
    with pytest.raises(ValueError):
        g.sdm_gx_launch(bad, 0)
    torch.cuda.synchronize()
    assert (case.result().view(np.uint32) == du.view(np.uint32)).all()


def test_no_kernel_instance_spills():
    """Every kernel instance runs without private (scratch) memory, and its workgroup fits one CU's registers."""
    seen = set()
    for plan in all_plans(256, 4096):
        if plan.engine == g.SDM_GX_ENGINE_MFMA:
            key = ("mfma", plan.mf_row_waves, plan.mf_col_waves, plan.mf_stages, plan.mf_reg_slabs,
                   plan.mf_loader_waves, plan.mf_du_at_end, plan.mf_block, plan.slab_rows)
            waves = plan.mf_row_waves * plan.mf_col_waves + plan.mf_loader_waves
        else:
            key = ("valu", plan.rows_per_wave, plan.cols_per_lane, plan.waves_per_wg, plan.staging)
            waves = plan.waves_per_wg
        if key in seen:
            continue
        seen.add(key)
        attrs = g.sdm_gx_kernel_attrs(plan)
        assert attrs["scratch_bytes"] == 0, (key, attrs)
        assert attrs["vgprs"] * -(-waves // 4) <= 512, (key, attrs)
    assert len([k for k in seen if k[0] == "valu"]) > 100 and len([k for k in seen if k[0] == "mfma"]) == 60    # 92 instances: the 32 unaligned-row twins are chosen for a layout, not by plan fields


def test_kernel_attrs_report_no_scratch():
    for key in (1, 2, 3, 4, 5):
        w = inputs.WORKLOADS[key]
        plan = g.sdm_gx_plan(w.N, w.C, w.hd, w.ld, w.ld, 0, w.base_offset_bytes % 16)
        attrs = g.sdm_gx_kernel_attrs(plan)
        say(f"workload {key}: {plan} {attrs}")
        assert attrs["scratch_bytes"] == 0
        assert 0 < attrs["vgprs"] <= 512
