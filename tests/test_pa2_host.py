"""Host logic of Phase A's C ABI that needs no GPU: sdm_pa2_check's status codes and sdm_pa2_plan_for's plans.

Neither entry point touches the arrays, so the arguments carry made-up, well-separated addresses.
"""

import pytest

from deterministic_fp32_gemm_amd import _binding as B

MiB = 1 << 20


def args(P=32, N=256, C=64, W=8, hd=128, ld_u=None, slots=1 << 14, ssr=-1, snap_rows=None, planes=None, plane=None,
         **addr):
    """sdm_pa2_args_t for N chunks of C tokens x W writes, each array at its own 256 MiB-aligned address."""
    a = B.sdm_pa2_args_t()
    n = C * W
    nsl = 1 + (hd - 1) // 128
    base = {"grad": 1, "bank": 2, "snap": 3, "d_u": 4, "beta": 5, "kpay": 6, "rec": 7, "bpre": 8, "out_eff": 9,
            "out_g": 10}
    for name, k in base.items():
        setattr(a, name, addr.get(name, k * 256 * MiB * 16))
    a.slots = slots
    a.snap_rows = snap_rows if snap_rows is not None else (N * n if ssr < 0 else (N // P) * ssr + P * n)
    a.ssr = ssr
    a.ld_u = ld_u if ld_u is not None else hd
    a.plane = plane if plane is not None else N * n
    a.planes = planes if planes is not None else (1 if nsl == 1 else nsl)
    a.N, a.P, a.C, a.W, a.hd = N, P, C, W, hd
    return a


def check(a, ti=0):
    return B.load().sdm_pa2_check(B.ctypes.byref(a), int(ti))


def plan(a, cus=256, lds=160 * 1024):
    p = B.sdm_pa2_plan_t()
    st = B.load().sdm_pa2_plan_for(B.ctypes.byref(a), cus, lds, B.ctypes.byref(p))
    return st, p


def test_valid_arguments_pass():
    assert check(args()) == B.SDM_GX_OK
    assert check(args(), ti=7) == B.SDM_GX_OK
    assert check(args(P=512, N=1024, hd=256, ld_u=260, slots=1 << 17, ssr=512 * 512), ti=1) == B.SDM_GX_OK


@pytest.mark.parametrize("field", ["grad", "bank", "snap", "d_u", "beta", "kpay", "rec", "out_eff", "out_g"])
def test_null_arrays(field):
    assert check(args(**{field: 0})) == B.SDM_GX_ERR_NULL


def test_bpre_needed_only_for_dense_rows():
    assert check(args(bpre=0)) == B.SDM_GX_ERR_NULL
    assert check(args(bpre=0, ssr=32 * 512)) == B.SDM_GX_OK


@pytest.mark.parametrize("kw", [dict(C=0), dict(C=257), dict(W=0), dict(W=257), dict(hd=0), dict(hd=1 << 20),
                                dict(slots=0), dict(planes=2), dict(hd=256, planes=1), dict(plane=256 * 512 - 1),
                                dict(snap_rows=32 * 512 - 1)])
def test_shapes(kw):
    assert check(args(**kw)) == B.SDM_GX_ERR_SHAPE


def test_snapshot_rows_cover_the_step():
    """Dense rows: (ti + 1) * P * n; per-entry rows: ti * ssr + P * n (a later step needs more rows)."""
    a = args(snap_rows=4 * 32 * 512)
    assert check(a, 3) == B.SDM_GX_OK and check(a, 4) == B.SDM_GX_ERR_SHAPE
    a = args(ssr=32 * 512, snap_rows=2 * 32 * 512 + 32 * 512)
    assert check(a, 2) == B.SDM_GX_OK and check(a, 3) == B.SDM_GX_ERR_SHAPE


def test_stride_and_steps():
    assert check(args(ld_u=127)) == B.SDM_GX_ERR_STRIDE
    assert check(args(), ti=8) == B.SDM_GX_ERR_STEP
    assert check(args(), ti=-1) == B.SDM_GX_ERR_STEP
    assert check(args(P=300)) == B.SDM_GX_ERR_STEP


def test_alignment():
    assert check(args(rec=7 * 256 * MiB * 16 + 4)) == B.SDM_GX_ERR_ALIGN     # records: 16 bytes
    assert check(args(grad=1 * 256 * MiB * 16 + 2)) == B.SDM_GX_ERR_ALIGN     # floats: 4 bytes
    assert check(args(d_u=4 * 256 * MiB * 16 + 4)) == B.SDM_GX_OK              # d_u rows may sit at any float


def test_written_arrays_must_not_overlap():
    a = args()
    assert check(args(out_g=a.grad)) == B.SDM_GX_ERR_OVERLAP                  # two written arrays
    assert check(args(bank=a.snap + 4)) == B.SDM_GX_ERR_OVERLAP               # written over a read array
    assert check(args(out_eff=a.d_u + 64)) == B.SDM_GX_ERR_OVERLAP
    assert check(args(bank=a.grad + (1 << 14) * 128 * 4)) == B.SDM_GX_OK       # adjacent, not overlapping


def test_planner_one_slice_small_chunks():
    """64 x 8 records per chunk, 32 chunks, 128 columns: 4-record tiles (at least 4; 2 would give 8 waves per SIMD),
    16 wavefronts per workgroup, one slice per wavefront."""
    st, p = plan(args())
    assert st == B.SDM_GX_OK
    assert (p.slices_per_wave, p.waves_per_wg, p.tile_len, p.ctas, p.npair) == (1, 16, 4, 8, 1)
    assert p.grid == 32 * 8 and p.lds_bytes == 64 * 16 * 32 + 64 * 4 and p.stage_out == 0


def test_planner_two_slices():
    """512 chunks of 64 x 8 records, 256 columns: two slices per wavefront, tiles of 32 records (16 per chunk: 32
    wavefronts per CU over 256 CUs), one workgroup per chunk."""
    st, p = plan(args(P=512, N=1024, hd=256, ld_u=260, slots=1 << 17, ssr=512 * 512))
    assert st == B.SDM_GX_OK
    assert (p.slices_per_wave, p.waves_per_wg, p.tile_len, p.ctas, p.npair) == (2, 16, 32, 1, 1)
    # one workgroup per chunk: its four output planes (2 slices x 2 outputs x 512 records) and a count go to LDS too
    assert p.grid == 512 and p.lds_bytes == 64 * 16 * 64 + 64 * 4 + 4 + 4 * 512 * 4 and p.stage_out == 1


def test_planner_stages_outputs_only_when_cheap():
    """Outputs go through LDS only with one workgroup per chunk, when they add at most a quarter to its LDS and the
    total fits the limit."""
    a = args(P=512, N=1024, hd=256, ld_u=260, slots=1 << 17, ssr=512 * 512)
    st, p = plan(a, lds=70000)                            # 73988 bytes with the outputs: left out
    assert st == B.SDM_GX_OK and p.ctas == 1 and p.lds_bytes == 64 * 16 * 64 + 64 * 4 and p.stage_out == 0
    st, p = plan(args(P=512, N=1024, C=4, W=256, hd=16, slots=1 << 17))   # outputs 4x the token rows: left out
    assert st == B.SDM_GX_OK and p.ctas == 1 and p.lds_bytes == 4 * 16 * 32 + 4 * 4 and p.stage_out == 0
    st, p = plan(args(), lds=0)                           # 8 workgroups per chunk: never staged
    assert st == B.SDM_GX_OK and p.ctas == 8 and p.lds_bytes == 64 * 16 * 32 + 64 * 4 and p.stage_out == 0


def test_planner_three_slices_and_wide_tokens():
    st, p = plan(args(P=4, N=8, hd=300))                  # three slices: a pair and a single
    assert st == B.SDM_GX_OK and p.slices_per_wave == 2 and p.npair == 2
    st, p = plan(args(P=4, N=8, C=200, hd=256))          # C > 128: one slice per wavefront
    assert st == B.SDM_GX_OK and p.slices_per_wave == 1 and p.npair == 2


def test_planner_falls_back_to_one_slice_then_refuses():
    a = args(P=4, N=8, C=128, hd=256)
    st, p = plan(a, lds=70000)                            # two slices' token rows (128 KiB) do not fit, one does
    assert st == B.SDM_GX_OK and p.slices_per_wave == 1 and p.lds_bytes == 128 * 16 * 32 + 128 * 4
    st, _ = plan(a, lds=40000)
    assert st == B.SDM_GX_ERR_LIMIT


def test_planner_rejects_bad_shapes_and_arguments():
    assert plan(args(C=0))[0] == B.SDM_GX_ERR_SHAPE
    assert plan(args(hd=1 << 20))[0] == B.SDM_GX_ERR_SHAPE
    p = B.sdm_pa2_plan_t()
    assert B.load().sdm_pa2_plan_for(None, 256, 0, B.ctypes.byref(p)) == B.SDM_GX_ERR_ARG


def test_planner_tiles_never_exceed_the_chunk():
    st, p = plan(args(P=1, N=1, C=1, W=1, hd=4, slots=4))
    assert st == B.SDM_GX_OK and p.tile_len == 1 and p.ctas == 1 and p.waves_per_wg == 4
