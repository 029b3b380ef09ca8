"""C ABI tests that need no GPU: the library loads and exports every function the header declares, the ctypes
structs match the C layout, argument checks return the documented status codes, and the planner only emits plans
the kernels support."""

import ctypes
import os
import re
import subprocess

import pytest

import deterministic_fp32_gemm_amd as g
from deterministic_fp32_gemm_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdm_gx_gemm.h")
HEADERS = (HEADER, os.path.join(ROOT, "include", "sdm_gx_pa2.h"))


def header_functions():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"SDM_GX_API\s+(?:const\s+)?\w+\*?\s+\*?(sdm_(?:gx|pa2)_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = header_functions()
    assert "sdm_gx_gemm" in names and "sdm_gx_gemm_steps" in names and len(names) >= 14


def test_library_exports_every_declared_function():
    lib = B.load()
    for name in header_functions():
        assert hasattr(lib, name), name
    assert sorted(B.EXPORTS) == header_functions()


def test_only_the_c_abi_is_exported():
    """Exported functions are exactly the C ABI (kernel handle variables, type V, are the HIP runtime's)."""
    out = subprocess.run(["nm", "-D", "--defined-only", B.lib_path()], capture_output=True, text=True, check=True)
    exported = {ln.split()[-1] for ln in out.stdout.splitlines() if ln.split() and ln.split()[1] in ("T", "W")}
    assert exported == set(header_functions()), exported ^ set(header_functions())


def test_abi_version():
    assert g.sdm_gx_abi_version() == 4


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "sdm_gx_gemm.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(sdm_gx_plan_t), offsetof(sdm_gx_plan_t, grid),
         sizeof(sdm_gx_launch_t), offsetof(sdm_gx_launch_t, ti_max), offsetof(sdm_gx_launch_t, plan_step),
         offsetof(sdm_gx_launch_t, plan_fused), offsetof(sdm_gx_plan_t, slab_rows),
         offsetof(sdm_gx_plan_t, mf_row_waves), offsetof(sdm_gx_plan_t, mf_workgroups),
         offsetof(sdm_gx_plan_t, mf_du_at_end), offsetof(sdm_gx_plan_t, mf_block),
         offsetof(sdm_gx_plan_t, mf_stream_du), offsetof(sdm_gx_plan_t, mf_aln));
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert vals == [ctypes.sizeof(g.sdm_gx_plan_t), g.sdm_gx_plan_t.grid.offset, ctypes.sizeof(g.sdm_gx_launch_t),
                    g.sdm_gx_launch_t.ti_max.offset, g.sdm_gx_launch_t.plan_step.offset,
                    g.sdm_gx_launch_t.plan_fused.offset, g.sdm_gx_plan_t.slab_rows.offset,
                    g.sdm_gx_plan_t.mf_row_waves.offset, g.sdm_gx_plan_t.mf_workgroups.offset,
                    g.sdm_gx_plan_t.mf_du_at_end.offset, g.sdm_gx_plan_t.mf_block.offset,
                    g.sdm_gx_plan_t.mf_stream_du.offset, g.sdm_gx_plan_t.mf_aln.offset]



def test_phase_a_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout_pa2.c"
    fields_a = [f for f, _ in B.sdm_pa2_args_t._fields_]
    fields_p = [f for f, _ in B.sdm_pa2_plan_t._fields_]
    body = " ".join(f'printf("%zu ", offsetof(sdm_pa2_args_t, {f}));' for f in fields_a)
    body += " ".join(f'printf("%zu ", offsetof(sdm_pa2_plan_t, {f}));' for f in fields_p)
    src.write_text(f"""
#include <stdio.h>
#include <stddef.h>
#include "sdm_gx_pa2.h"
int main(void) {{
  printf("%zu %zu ", sizeof(sdm_pa2_args_t), sizeof(sdm_pa2_plan_t));
  {body}
  return 0;
}}
""")
    exe = tmp_path / "layout_pa2"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(B.sdm_pa2_args_t), ctypes.sizeof(B.sdm_pa2_plan_t)]
    want += [getattr(B.sdm_pa2_args_t, f).offset for f in fields_a] + [getattr(B.sdm_pa2_plan_t, f).offset for f in fields_p]
    assert vals == want


def test_c_program_links_and_calls_the_host_entry_points(tmp_path):
    """A plain C program, linked against the library, calls the entry points that need no device: the ABI version,
    the argument checks and both planners, with made-up device addresses (nothing is dereferenced)."""
    src = tmp_path / "use.c"
    src.write_text(r"""
#include <stdint.h>
#include <stdio.h>
#include "sdm_gx_gemm.h"
#include "sdm_gx_pa2.h"
int main(void) {
  float* du = (float*)(uintptr_t)(1ull << 32);
  const float* x = (const float*)(uintptr_t)(2ull << 32);
  const float* dv = (const float*)(uintptr_t)(3ull << 32);
  sdm_gx_plan_t plan;
  int ok = sdm_gx_check(du, 260, x, dv, 260, 1024, 1, 512, 64, 256);
  int bad = sdm_gx_check(du, 255, x, dv, 260, 1024, 1, 512, 64, 256);
  int pl = sdm_gx_plan_for(512, 64, 256, 260, 260, 0, 4, -1, 256, 160 * 1024, &plan);
  sdm_pa2_args_t a = {0};
  a.grad = (float*)(uintptr_t)(4ull << 32); a.bank = (float*)(uintptr_t)(5ull << 32); a.slots = 1 << 17;
  a.snap = (const float*)(uintptr_t)(6ull << 32); a.snap_rows = 2 * 512 * 512; a.ssr = 512 * 512;
  a.d_u = x; a.ld_u = 260; a.beta = (const float*)(uintptr_t)(7ull << 32);
  a.kpay = (const int32_t*)(uintptr_t)(8ull << 32); a.rec = (const int32_t*)(uintptr_t)(9ull << 32);
  a.out_eff = (float*)(uintptr_t)(10ull << 32); a.out_g = (float*)(uintptr_t)(11ull << 32);
  a.N = 1024; a.P = 512; a.C = 64; a.W = 8; a.hd = 256; a.planes = 2; a.plane = 1024 * 512;
  sdm_pa2_plan_t q;
  int pa = sdm_pa2_check(&a, 1);
  int pq = sdm_pa2_plan_for(&a, 256, 160 * 1024, &q);
  printf("%d %d %d %d %d %d %d %d %d %s\n", sdm_gx_abi_version(), ok, bad, pl, plan.engine, pa, pq, q.slices_per_wave,
         q.ctas, sdm_gx_strerror(bad));
  return 0;
}
""")
    exe = tmp_path / "use"
    libdir = os.path.dirname(B.lib_path())
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe), "-L", libdir,
                    "-l:" + os.path.basename(B.lib_path()), f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True, timeout=120).stdout.split(maxsplit=9)
    assert [int(v) for v in out[:9]] == [g.sdm_gx_abi_version(), B.SDM_GX_OK, B.SDM_GX_ERR_STRIDE, B.SDM_GX_OK,
                                         B.SDM_GX_ENGINE_MFMA, B.SDM_GX_OK, B.SDM_GX_OK, 2, 1]
    assert out[9].strip() == g.sdm_gx_strerror(B.SDM_GX_ERR_STRIDE)

def test_strerror_covers_every_code():
    for code in range(0, -12, -1):
        assert g.sdm_gx_strerror(code) != "unknown status"
    assert g.sdm_gx_strerror(-99) == "unknown status"


# ---- argument checks (addresses are plain integers: nothing is dereferenced) -------------------------------------
U, X, V = 1 << 32, 1 << 36, 1 << 40        # far-apart fake device addresses


def chk(**kw):
    a = dict(d_u=U, ld_u=64, x=X, d_dv=V, ld_dv=64, N=8, ti=0, P=4, C=64, hd=64)
    a.update(kw)
    return g.sdm_gx_check(a["d_u"], a["ld_u"], a["x"], a["d_dv"], a["ld_dv"], a["N"], a["ti"], a["P"], a["C"],
                          a["hd"])


@pytest.mark.parametrize("kw,code", [
    ({}, g.SDM_GX_OK),
    (dict(ti=1), g.SDM_GX_OK),
    (dict(d_u=0), g.SDM_GX_ERR_NULL),
    (dict(x=0), g.SDM_GX_ERR_NULL),
    (dict(d_dv=0), g.SDM_GX_ERR_NULL),
    (dict(C=0), g.SDM_GX_ERR_SHAPE),
    (dict(C=257), g.SDM_GX_ERR_SHAPE),
    (dict(C=256, ld_u=64, hd=64), g.SDM_GX_OK),
    (dict(hd=0), g.SDM_GX_ERR_SHAPE),
    (dict(hd=1 << 20, ld_u=1 << 20, ld_dv=1 << 20), g.SDM_GX_ERR_SHAPE),
    (dict(hd=(1 << 20) - 1, ld_u=1 << 20, ld_dv=1 << 20, N=1, P=1), g.SDM_GX_OK),
    (dict(N=0), g.SDM_GX_ERR_SHAPE),
    (dict(N=1 << 31), g.SDM_GX_ERR_SHAPE),
    (dict(P=0), g.SDM_GX_ERR_SHAPE),
    (dict(ld_u=63), g.SDM_GX_ERR_STRIDE),
    (dict(ld_dv=63), g.SDM_GX_ERR_STRIDE),
    (dict(ld_u=1 << 31), g.SDM_GX_ERR_STRIDE),
    (dict(P=9), g.SDM_GX_ERR_STEP),
    (dict(ti=-1), g.SDM_GX_ERR_STEP),
    (dict(ti=2), g.SDM_GX_ERR_STEP),
    (dict(ti=(1 << 62)), g.SDM_GX_ERR_STEP),
    (dict(N=9, P=4, ti=2), g.SDM_GX_ERR_STEP),      # the trailing chunk 8 belongs to no step
    (dict(d_u=U + 2), g.SDM_GX_ERR_ALIGN),
    (dict(x=X + 1), g.SDM_GX_ERR_ALIGN),
    (dict(d_dv=V + 6), g.SDM_GX_ERR_ALIGN),
    (dict(d_u=U + 4), g.SDM_GX_OK),                  # 4-byte alignment is enough
    (dict(x=U + 4 * 100), g.SDM_GX_ERR_OVERLAP),
    (dict(d_dv=U + 4 * (8 * 64 * 64 - 1)), g.SDM_GX_ERR_OVERLAP),
    (dict(d_dv=U + 4 * 8 * 64 * 64), g.SDM_GX_OK),   # adjacent, not overlapping
    (dict(x=U - 4 * 8 * 64 * 64), g.SDM_GX_OK),      # x ends exactly where d_u starts
    (dict(x=U - 4 * 8 * 64 * 64 + 4), g.SDM_GX_ERR_OVERLAP),
    (dict(ld_u=100, d_dv=U + 4 * ((8 * 64 - 1) * 100 + 64)), g.SDM_GX_OK),   # extent ends at the last row's hd
])
def test_check_codes(kw, code):
    assert chk(**kw) == code


def cdiv(a, b):
    return -(-a // b)


def mfma_grid(items, workgroups=256):
    if items == 0:
        return 0
    per = cdiv(items, min(items, workgroups))
    return cdiv(items, per)


def dma_ok(C, ld):
    return C % 4 == 0 and ld % 4 == 0 and (C + 32) * ld * 4 < 2 ** 31


def test_plan_for_emits_supported_plans():
    shapes = [(C, hd) for C in (1, 2, 3, 4, 5, 16, 17, 31, 32, 64, 100, 128, 200, 256)
              for hd in (1, 3, 4, 63, 64, 65, 100, 128, 129, 200, 256, 257, 1000, 4100)]
    for nchunks in (0, 1, 7, 128, 4096):
        for C, hd in shapes:
            p = g.sdm_gx_plan_for(nchunks, C, hd)
            assert p.mf_aln == 0                       # rows on 16-byte boundaries (ld = hd, aligned bases)
            # engine rule: matrix cores for 32 <= C when slabs can go straight to LDS (C and the row stride, taken
            # as hd here, multiples of 4), or for hd <= 128 through the register ring
            assert p.engine == (g.SDM_GX_ENGINE_MFMA if C >= 32 and (dma_ok(C, hd) or hd <= 128)
                                else g.SDM_GX_ENGINE_VALU)
            if p.engine == g.SDM_GX_ENGINE_MFMA and dma_ok(C, hd):
                # 16-column wavefronts, slabs straight to LDS, items of 64 or 128 rows by 64 columns (32 when hd <= 32
                # or when 64-column items would leave CUs idle; 64 x 128 when C > 64 and hd is a multiple of 128 with
                # items for every CU), 8 compute wavefronts per CU unless the items are many (4 or more per CU),
                # 32-row stages when each CU holds one workgroup that walks several items
                assert p.mf_reg_slabs == 0 and p.mf_stages == 3 and p.mf_du_at_end == 0
                rw0 = 2 if C > 64 else 1
                wide = hd > 32 and nchunks * cdiv(C, 64 * rw0) * cdiv(hd, 64) >= 256
                long_rows = wide and C > 64 and hd % 128 == 0 and nchunks * cdiv(C, 64) * (hd // 128) >= 256
                rw, cw = (1, 8) if long_rows else (rw0, 4 if wide else 2)
                items = nchunks * cdiv(cdiv(C, 64), rw) * cdiv(hd, 16 * cw)
                two = rw * cw < 8 and items < 4 * 256
                grid16 = mfma_grid(items, 512 if two else 256)
                # one workgroup per CU walking several items, hd a multiple of 128: 64 x 128 items on four 32-column
                # wavefronts, 3 stages of 32 rows
                items32 = nchunks * cdiv(C, 64) * (hd // 128)
                if grid16 <= 256 and items > grid16 and hd % 128 == 0 and items32 > 256:
                    assert (p.mf_block, p.mf_row_waves, p.mf_col_waves, p.slab_rows, p.mf_loader_waves) == (32, 1, 4, 32, 2)
                    assert p.mf_workgroups == 256 and p.grid == mfma_grid(items32, 256) and p.mf_stream_du == 0
                    assert p.lds_bytes == 16 * 3 * 32 * (16 + 8 * 4)
                    continue
                assert p.mf_block == 16 and (p.mf_row_waves, p.mf_col_waves) == (rw, cw) and p.mf_loader_waves == 1
                assert p.mf_workgroups == (512 if two else 256)
                assert p.grid == grid16
                assert p.slab_rows == (32 if p.grid <= 256 and items > p.grid else 16)
                assert p.mf_stream_du == (0 if p.grid <= 256 else 1)
                assert p.lds_bytes == 16 * 3 * p.slab_rows * (16 * p.mf_row_waves + 4 * p.mf_col_waves)
                continue
            if p.engine == g.SDM_GX_ENGINE_MFMA:
                # register ring, 32-column wavefronts, one work item per chunk up to 128 x 128
                assert p.mf_block == 32 and p.mf_stages == 4
                assert p.mf_row_waves == (2 if C > 64 else 1)
                assert p.mf_col_waves == (4 if cdiv(hd, 32) > 2 else cdiv(hd, 32))
                big = (p.mf_row_waves, p.mf_col_waves) == (2, 4)      # 128 x 128 items: two workgroups per CU
                assert p.mf_reg_slabs == (2 if big else 4)
                assert p.mf_du_at_end == (1 if big else 0) and p.mf_workgroups == (512 if big else 256)
                assert p.mf_loader_waves == (2 if p.mf_row_waves * p.mf_col_waves <= 2 else 4)
                items = nchunks * cdiv(cdiv(C, 64), p.mf_row_waves) * cdiv(hd, 32 * p.mf_col_waves)
                assert p.grid == mfma_grid(items, p.mf_workgroups)
                assert p.lds_bytes == 16 * 4 * 16 * (16 * p.mf_row_waves + 8 * p.mf_col_waves)
                continue
            assert p.rows_per_wave in (1, 2, 4, 8, 16) and p.rows_per_wave <= C
            assert p.cols_per_lane in (1, 2, 4) and p.rows_per_wave * p.cols_per_lane <= 64
            assert p.waves_per_wg in (1, 2, 4, 8)
            nrb = cdiv(C, p.rows_per_wave)
            nrg = cdiv(nrb, p.waves_per_wg)
            ncb = cdiv(hd, 64 * p.cols_per_lane)
            assert p.grid == nchunks * nrg * ncb
            assert p.lds_bytes <= 64 * 1024


@pytest.mark.parametrize("bad", [
    dict(rows_per_wave=3), dict(rows_per_wave=64), dict(cols_per_lane=3), dict(waves_per_wg=3),
    dict(waves_per_wg=32), dict(staging=2), dict(xcd_remap=2), dict(slab_rows=-1),
    dict(rows_per_wave=32), dict(rows_per_wave=16, cols_per_lane=4, waves_per_wg=16), dict(engine=2),
    dict(engine=-1),
])
def test_plan_complete_rejects(bad):
    p = g.make_plan(8, 1, 4)
    for k, v in bad.items():
        setattr(p, k, v)
    with pytest.raises(ValueError):
        g.sdm_gx_plan_complete(p, 4, 64, 64)


@pytest.mark.parametrize("bad", [
    dict(mf_row_waves=3), dict(mf_row_waves=0), dict(mf_col_waves=3), dict(mf_col_waves=16),
    dict(mf_row_waves=2, mf_col_waves=8), dict(mf_stages=3), dict(mf_stages=2), dict(mf_reg_slabs=3),
    dict(mf_loader_waves=1), dict(mf_loader_waves=8), dict(mf_workgroups=-1),
    dict(mf_col_waves=8, mf_reg_slabs=4, mf_loader_waves=2),        # left out of the table: it spills
    dict(mf_row_waves=2, mf_col_waves=4, mf_reg_slabs=4, mf_loader_waves=2),
    dict(mf_du_at_end=2), dict(mf_du_at_end=1),                       # d_u at the end: only 2 reg slabs, 4 loaders
    dict(mf_du_at_end=1, mf_reg_slabs=2, mf_loader_waves=2),
])
def test_mfma_plan_complete_rejects(bad):
    p = g.make_mfma_plan(1, 4)
    for k, v in bad.items():
        setattr(p, k, v)
    with pytest.raises(ValueError):
        g.sdm_gx_plan_complete(p, 4, 64, 64)


MFMA_TILES = [(rw, cw) for rw in (1, 2) for cw in (1, 2, 4, 8) if not (rw == 2 and cw == 8)]
MFMA_INSTANCES = [(rw, cw, 4, rs, lw, 0, 32, 16) for rw, cw in MFMA_TILES for rs in (2, 4) for lw in (2, 4)
                  if (rw, cw, rs, lw) not in ((1, 8, 4, 2), (2, 4, 4, 2))] + \
                 [(2, 4, 4, 2, 4, 1, 32, 16), (1, 4, 4, 2, 4, 1, 32, 16)] + \
                 [(rw, cw, s, 0, lw, 0, 32, 16) for rw, cw in MFMA_TILES for s, lw in ((4, 1), (8, 2))] + \
                 [(2, 4, 4, 0, 1, 1, 32, 16), (1, 4, 3, 0, 1, 0, 32, 32), (1, 4, 3, 0, 2, 0, 32, 32)] + \
                 [(rw, cw, s, 0, lw, 0, 16, j) for rw, cw in ((1, 2), (1, 4), (1, 8), (2, 2), (2, 4))
                  for s, lw, j in ((3, 1, 16), (8, 2, 16), (3, 1, 32))]
# and, for each 16-column (3 stages, 1 loader) instance, twins for rows off a 16-byte boundary, picked at launch


@pytest.mark.parametrize("rw,cw,s,rs,lw,de,blk,j", MFMA_INSTANCES)
def test_mfma_plan_complete_geometry(rw, cw, s, rs, lw, de, blk, j):
    for nchunks, C, hd, wgs in ((512, 128, 128, 0), (7, 200, 33, 3), (1, 1, 1, 0), (1000, 64, 256, 100), (0, 64, 64, 0)):
        ld = cdiv(hd, 4) * 4                    # a stride direct-to-LDS slabs can take
        p = g.sdm_gx_plan_complete(g.make_mfma_plan(rw, cw, s, rs, lw, wgs, de, blk, j), nchunks, C, hd,
                                   ld_u=ld, ld_dv=ld)
        ers, es, ej, eblk, ecw = rs, s, j, blk, cw
        if rs == 0 and not dma_ok(C, ld):       # C not a multiple of 4: the register-ring form of the plan
            ers, es, ej, eblk, ecw = 2, 4, 16, 32, (cw // 2 if blk == 16 else cw)
        items = nchunks * cdiv(cdiv(C, 64), rw) * cdiv(hd, eblk * ecw)
        assert p.grid == mfma_grid(items, wgs or 256)
        assert p.lds_bytes == 16 * es * ej * (16 * rw + eblk // 4 * ecw)
        assert (p.mf_block, p.slab_rows, p.mf_reg_slabs, p.mf_col_waves) == (eblk, ej, ers, ecw)


def test_mfma_block_zero_means_32():
    p = g.sdm_gx_plan_complete(g.make_mfma_plan(1, 2, 4, 4, 2, 0, 0, 0), 8, 64, 64)
    assert p.mf_block == 32 and p.slab_rows == 16 and p.grid == 8


def test_mfma_direct_to_lds_fallback_instances_exist():
    """A direct-to-LDS plan whose launch finds unaligned x or d_dv rows runs the same work items through the register
    ring with 4 stages of 16 rows, 2 register slabs and 4 loader wavefronts of 32-column wavefronts (half as many
    column wavefronts for a 16-column plan): that instance exists for every direct-to-LDS one."""
    for rw, cw, s, rs, lw, de, blk, j in MFMA_INSTANCES:
        if rs == 0:
            fcw = cw // 2 if blk == 16 else cw
            assert (rw, fcw, 4, 2, 4, de, 32, 16) in MFMA_INSTANCES
            g.sdm_gx_plan_complete(g.make_mfma_plan(rw, fcw, 4, 2, 4, 0, de), 4, 64, 64)


def test_mfma_direct_to_lds_rejects_missing_instances():
    for s, rs, lw in ((8, 0, 1), (4, 0, 2), (2, 0, 1), (8, 2, 4)):
        with pytest.raises(ValueError):
            g.sdm_gx_plan_complete(g.make_mfma_plan(2, 4, s, rs, lw), 4, 128, 128)
    for rw, cw, s, rs, lw, blk, j in ((1, 1, 3, 0, 1, 16, 0), (1, 2, 4, 4, 2, 16, 0), (1, 2, 3, 0, 1, 8, 0),
                                      (1, 2, 3, 0, 1, 64, 0), (1, 2, 4, 0, 1, 32, 32), (1, 2, 8, 0, 2, 16, 32),
                                      (1, 2, 4, 4, 2, 32, 32), (1, 2, 3, 0, 1, 16, 24), (1, 2, 4, 0, 1, 16, 16),
                                      (1, 2, 3, 0, 1, 32, 16)):
        with pytest.raises(ValueError):
            g.sdm_gx_plan_complete(g.make_mfma_plan(rw, cw, s, rs, lw, 0, 0, blk, j), 4, 64, 64)

def test_plan_resolves_the_layout():
    """The planner takes the row strides and the placement of x and d_dv, and reports the instance that a launch with
    that layout runs (unaligned-row twins, or the register ring where the strides rule out direct-to-LDS slabs)."""
    # workload 5's layout: ld 260, d_u and d_dv at +4 bytes, x aligned: 64 x 128 items of 32-column wavefronts with
    # 32-row stages and 2 loader wavefronts, d_dv rows by 4-byte DMA (LDS rows exactly the item's 128 columns)
    p = g.sdm_gx_plan_for(1024, 64, 256, ld_u=260, ld_dv=260, x_mod16=0, dv_mod16=4)
    assert (p.engine, p.mf_reg_slabs, p.mf_block, p.mf_col_waves, p.slab_rows, p.mf_loader_waves, p.mf_aln) == \
        (g.SDM_GX_ENGINE_MFMA, 0, 32, 4, 32, 2, 4)
    assert p.lds_bytes == 16 * 3 * (32 * 16 + 32 * 32)
    # x off the boundary too: 1 loader wavefront, both from the 16-byte boundary below (one more group per LDS row)
    q = g.sdm_gx_plan_for(1024, 64, 256, ld_u=260, ld_dv=260, x_mod16=8, dv_mod16=4)
    assert (q.mf_reg_slabs, q.mf_block, q.mf_loader_waves, q.mf_aln) == (0, 32, 1, 3) and q.lds_bytes > p.lds_bytes
    # 16-column wavefronts (hd not a multiple of 128): d_dv rows by 4-byte DMA
    t = g.sdm_gx_plan_for(1024, 64, 192, ld_u=196, ld_dv=196, x_mod16=0, dv_mod16=4)
    assert (t.mf_reg_slabs, t.mf_block, t.mf_aln) == (0, 16, 4)
    assert t.lds_bytes == 16 * 3 * t.slab_rows * 16 + 4 * 3 * t.slab_rows * 16 * t.mf_col_waves
    # workload 4's shape with d_dv off the boundary: the 32-column 64 x 128 items, d_dv rows by 4-byte DMA
    r = g.sdm_gx_plan_for(512, 128, 128, x_mod16=0, dv_mod16=12)
    assert (r.mf_row_waves, r.mf_col_waves, r.mf_block, r.slab_rows, r.mf_aln) == (1, 4, 32, 32, 4)
    # a row stride that is not a multiple of 4: the register ring (hd <= 128), or the vector ALUs (hd > 128)
    s_ = g.sdm_gx_plan_for(256, 64, 128, ld_u=131, ld_dv=131)
    assert (s_.engine, s_.mf_reg_slabs, s_.mf_block, s_.mf_aln) == (g.SDM_GX_ENGINE_MFMA, 4, 32, 0)
    assert g.sdm_gx_plan_for(256, 64, 200, ld_u=203, ld_dv=203).engine == g.SDM_GX_ENGINE_VALU
    # d_u's stride alone never changes the instance, unless the 32-bit d_u offsets would overflow
    assert g.sdm_gx_plan_for(256, 64, 128, ld_u=131, ld_dv=128).mf_reg_slabs == 0
    assert g.sdm_gx_plan_for(2, 256, 64, ld_u=1 << 21, ld_dv=64).engine == g.SDM_GX_ENGINE_VALU


def test_plan_complete_resolves_the_layout():
    """A caller-made direct-to-LDS plan is completed for the layout: its unaligned-row twin, or the register-ring plan
    of the same work items where there is none; mf_aln on input is ignored."""
    p = g.make_mfma_plan(1, 4, 3, 0, 1, 0, 0, 16, 16)
    p.mf_aln = 3
    assert g.sdm_gx_plan_complete(p, 64, 64, 128).mf_aln == 0
    p = g.sdm_gx_plan_complete(g.make_mfma_plan(1, 4, 3, 0, 1, 0, 0, 16, 16), 64, 64, 128, dv_mod16=8)
    assert (p.mf_reg_slabs, p.mf_aln, p.mf_col_waves) == (0, 4, 4)
    # the 32-column 64 x 128 instance with 32-row stages has twins (d_dv rows, and x rows too, from the boundary below)
    p = g.sdm_gx_plan_complete(g.make_mfma_plan(1, 4, 3, 0, 1, 0, 0, 32, 32), 64, 64, 256, dv_mod16=8)
    assert (p.mf_reg_slabs, p.mf_block, p.mf_aln) == (0, 32, 2)
    p = g.sdm_gx_plan_complete(g.make_mfma_plan(1, 4, 3, 0, 1, 0, 0, 32, 32), 64, 64, 256, x_mod16=4)
    assert (p.mf_reg_slabs, p.mf_block, p.mf_aln) == (0, 32, 3)
    # the other 32-column direct-to-LDS instances have no twins: the register ring, same tile
    p = g.sdm_gx_plan_complete(g.make_mfma_plan(1, 2, 4, 0, 1, 0, 0, 32, 16), 64, 64, 128, x_mod16=4)
    assert (p.mf_reg_slabs, p.mf_stages, p.mf_loader_waves, p.mf_block, p.mf_col_waves, p.mf_aln) == \
        (2, 4, 4, 32, 2, 0)
    # 16-column plan, odd stride: the register ring with half the column wavefronts (32 columns each)
    p = g.sdm_gx_plan_complete(g.make_mfma_plan(1, 4, 3, 0, 1, 0, 0, 16, 32, 1), 64, 64, 128, ld_u=130, ld_dv=130)
    assert (p.mf_reg_slabs, p.mf_block, p.mf_col_waves, p.slab_rows, p.mf_stream_du) == (2, 32, 2, 16, 0)


@pytest.mark.parametrize("kw", [dict(x_mod16=2), dict(dv_mod16=16), dict(x_mod16=-4), dict(ld_u=63),
                                dict(ld_dv=1 << 31), dict(engine=2), dict(engine=-2)])
def test_planner_rejects_bad_layout_arguments(kw):
    with pytest.raises(ValueError):
        g.sdm_gx_plan_for(8, 64, 64, **kw)


def test_planner_engine_choice():
    assert g.sdm_gx_plan_for(128, 64, 64, engine=g.SDM_GX_ENGINE_VALU).engine == g.SDM_GX_ENGINE_VALU
    assert g.sdm_gx_plan_for(2, 16, 16).engine == g.SDM_GX_ENGINE_VALU
    p = g.sdm_gx_plan_for(2, 16, 16, engine=g.SDM_GX_ENGINE_MFMA)
    assert p.engine == g.SDM_GX_ENGINE_MFMA and p.mf_reg_slabs == 0
    with pytest.raises(RuntimeError):           # 32-bit d_u offsets: the matrix cores cannot take this stride
        g.sdm_gx_plan_for(2, 256, 64, ld_u=1 << 21, engine=g.SDM_GX_ENGINE_MFMA)


def test_plan_complete_rows_beyond_c():
    with pytest.raises(ValueError):
        g.sdm_gx_plan_complete(g.make_plan(16, 1, 1), 4, 8, 64)
    assert g.sdm_gx_plan_complete(g.make_plan(8, 1, 1), 4, 8, 64).grid == 4


def test_plan_complete_lds_limit():
    p = g.sdm_gx_plan_complete(g.make_plan(8, 2, 4, staging=1, slab_rows=256), 4, 256, 256, 160 * 1024)
    assert p.slab_rows == 256 and p.lds_bytes == 256 * 128 * 4
    with pytest.raises(RuntimeError):
        g.sdm_gx_plan_complete(g.make_plan(8, 2, 4, staging=1, slab_rows=256), 4, 256, 256, 64 * 1024)
    p = g.sdm_gx_plan_complete(g.make_plan(8, 4, 4, staging=1, slab_rows=300), 4, 100, 256, 160 * 1024)
    assert p.slab_rows == 100                       # clamped to C
    p = g.sdm_gx_plan_complete(g.make_plan(8, 4, 4, staging=1), 4, 256, 256)
    assert p.slab_rows == 32 and p.lds_bytes == 32 * 1024


def test_tensor_layout_rejects_bad_shapes():
    torch = pytest.importorskip("torch")
    from deterministic_fp32_gemm_amd import tensor_layout
    x = torch.zeros(4, 8, 8)
    du = torch.zeros(4, 8, 12)[:, :, :10]
    dv = torch.zeros(32, 10)
    assert tensor_layout(du, x, dv) == (4, 8, 10, 12, 10)
    with pytest.raises(ValueError):
        tensor_layout(du, x.transpose(1, 2), dv)
    with pytest.raises(ValueError):
        tensor_layout(du, x, torch.zeros(31, 10))


def test_graph_entry_points_reject_bad_handles_without_a_device():
    """Graph calls check their arguments before any HIP call."""
    lib = g.load()
    h = ctypes.c_void_p()
    bad = g.sdm_gx_launch_t()                                        # no magic: not a prepared launch
    assert lib.sdm_gx_graph_create(None, ctypes.byref(bad), 0, 1, 2) == g.SDM_GX_ERR_ARG
    assert lib.sdm_gx_graph_create(ctypes.byref(h), ctypes.byref(bad), 0, 1, 7) == g.SDM_GX_ERR_ARG
    assert lib.sdm_gx_graph_create(ctypes.byref(h), ctypes.byref(bad), 0, 1, 2) == g.SDM_GX_ERR_PLAN
    assert lib.sdm_gx_graph_create(ctypes.byref(h), None, 0, 1, 2) == g.SDM_GX_ERR_PLAN
    assert not h.value
    assert lib.sdm_gx_graph_launch(None, None) == g.SDM_GX_ERR_PLAN
    assert lib.sdm_gx_graph_nodes(None) == -1
    assert lib.sdm_gx_graph_destroy(None) == g.SDM_GX_OK
