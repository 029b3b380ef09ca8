// Host entry points of libsdm_gx_gemm: argument checks, the launch planner, single-step, multi-step and prepared
// launches. Everything that decides whether and how to launch runs here; every arithmetic step of the update runs
// in the kernels of gx_gemm_kernel.hip (vector-ALU engine) and gx_gemm_mfma.hip (matrix-core engine).
//
// The checks follow the page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_gemm_cuda.py": the host entry
// gx_gemm (shape, step range, overlap and alignment checks) and supported(); the prepared launch follows its
// per-backward plan (gx_gemm_plan / gx_gemm_plan_launch: validate once at ti_max, then patch only ti).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/sdm_gx_gemm.h"
#include "gx_gemm_kernel.h"
#include "gx_gemm_mfma.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = static_cast<int>(e);
    return SDM_GX_ERR_HIP;
}

constexpr uint64_t kLaunchMagic = 0x314843554E4C4753ull;   // prepared-launch tag

}  // namespace

namespace sdm_gx {
// The HIP error behind an SDM_GX_ERR_HIP status of any entry point of the library (Phase A's included).
int record_hip_error(hipError_t e) { return hip_fail(e); }
}  // namespace sdm_gx

namespace {

// ---- argument checks (no device access) ---------------------------------------------------------------------------
int64_t row_extent(int64_t N, int64_t C, int64_t ld, int64_t hd) {   // elements reachable in a [N][C] ld-strided array
    return (N * C - 1) * ld + hd;
}

bool overlaps(const void* a, int64_t a_elems, const void* b, int64_t b_elems) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    const uintptr_t a1 = a0 + static_cast<uintptr_t>(a_elems) * sizeof(float);
    const uintptr_t b1 = b0 + static_cast<uintptr_t>(b_elems) * sizeof(float);
    return a0 < b1 && b0 < a1;
}

int check_args(const float* du, int64_t ld_u, const float* x, const float* dv, int64_t ld_dv, int64_t N, int64_t ti,
               int64_t P, int64_t C, int64_t hd) {
    if (!du || !x || !dv) return SDM_GX_ERR_NULL;
    if (C < 1 || C > SDM_GX_MAX_C || hd < 1 || hd >= SDM_GX_HD_LIMIT) return SDM_GX_ERR_SHAPE;
    if (N < 1 || N >= SDM_GX_N_LIMIT || P < 1) return SDM_GX_ERR_SHAPE;
    if (ld_u < hd || ld_dv < hd || ld_u >= SDM_GX_LD_LIMIT || ld_dv >= SDM_GX_LD_LIMIT) return SDM_GX_ERR_STRIDE;
    // bounds by division before any product (no overflow for any int64 ti / P)
    if (P > N || ti < 0 || ti >= N / P) return SDM_GX_ERR_STEP;
    if ((reinterpret_cast<uintptr_t>(du) | reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(dv)) & 3u)
        return SDM_GX_ERR_ALIGN;
    const int64_t nu = row_extent(N, C, ld_u, hd), nv = row_extent(N, C, ld_dv, hd), nx = N * C * C;
    if (overlaps(du, nu, x, nx) || overlaps(du, nu, dv, nv)) return SDM_GX_ERR_OVERLAP;
    return SDM_GX_OK;
}

// ---- device facts -------------------------------------------------------------------------------------------------
struct DeviceInfo {
    bool known = false;
    bool gfx950 = false;
    int num_cus = 0;
    int lds_per_wg = 0;     // max dynamic + static LDS bytes per workgroup
    int lds_per_cu = 0;
};

std::mutex g_dev_mu;
std::vector<DeviceInfo> g_dev;

int device_info(int dev, DeviceInfo* out) {
    {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        if (dev >= 0 && dev < static_cast<int>(g_dev.size()) && g_dev[dev].known) {
            *out = g_dev[dev];
            return SDM_GX_OK;
        }
    }
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e);
    DeviceInfo d;
    d.known = true;
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.num_cus = prop.multiProcessorCount;
    d.lds_per_wg = static_cast<int>(prop.sharedMemPerBlock);
    d.lds_per_cu = static_cast<int>(prop.maxSharedMemoryPerMultiProcessor);
    if (d.lds_per_cu <= 0) d.lds_per_cu = d.lds_per_wg;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (static_cast<int>(g_dev.size()) <= dev) g_dev.resize(dev + 1);
    g_dev[dev] = d;
    *out = d;
    return SDM_GX_OK;
}

int current_device(int* dev, DeviceInfo* info) {
    hipError_t e = hipGetDevice(dev);
    if (e != hipSuccess) return hip_fail(e);
    int st = device_info(*dev, info);
    if (st) return st;
    return info->gfx950 ? SDM_GX_OK : SDM_GX_ERR_DEVICE;
}

// The pointer is device (or managed) memory of device `dev`.
int on_device(const void* p, int dev) {
    hipPointerAttribute_t a;
    hipError_t e = hipPointerGetAttributes(&a, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();     // an unknown (host) pointer: clear the sticky error, report a device error
        return SDM_GX_ERR_DEVICE;
    }
    if (a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged) return SDM_GX_ERR_DEVICE;
    if (a.device != dev) return SDM_GX_ERR_DEVICE;
    return SDM_GX_OK;
}

// ---- planner ------------------------------------------------------------------------------------------------------
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool valid_ri(int v) { return v == 1 || v == 2 || v == 4 || v == 8 || v == 16; }
bool valid_rc(int v) { return v == 1 || v == 2 || v == 4; }
bool valid_waves(int v) { return v == 1 || v == 2 || v == 4 || v == 8 || v == 16; }

constexpr int kDefaultSlabBytes = 32 * 1024;

constexpr int kDefaultCus = 256;                // MI355X

// The matrix-core kernel instance of a plan (mf_block 0 means 32, slab_rows 0 means 16), or nullptr.
const sdm_gx::MfmaEntry* find_mfma(const sdm_gx_plan_t& p) {
    return sdm_gx::find_mfma_kernel(p.mf_row_waves, p.mf_col_waves, p.mf_stages, p.mf_reg_slabs, p.mf_loader_waves,
                                    p.mf_du_at_end, p.mf_block > 0 ? p.mf_block : 32,
                                    p.slab_rows > 0 ? p.slab_rows : 16, p.mf_aln);
}

// Row strides and the placement of x and d_dv relative to a 16-byte boundary: what decides, besides the shape, which
// kernel instance a launch runs.
struct Layout {
    int64_t ld_u, ld_dv;
    int x_mod16, dv_mod16;      // base address mod 16, in bytes (0, 4, 8 or 12)
};

Layout layout_of(int64_t ld_u, int64_t ld_dv, const float* x, const float* dv) {
    return Layout{ld_u, ld_dv, static_cast<int>(reinterpret_cast<uintptr_t>(x) & 15u),
                  static_cast<int>(reinterpret_cast<uintptr_t>(dv) & 15u)};
}

// Geometry of the matrix-core engine for nchunks chunks: work items and the persistent grid.
struct MfmaGeom {
    int64_t nrg, ncg, items, per, grid;
};
MfmaGeom mfma_geom(const sdm_gx_plan_t& p, int64_t nchunks, int64_t C, int64_t hd) {
    MfmaGeom g;
    g.nrg = cdiv(cdiv(C, 64), p.mf_row_waves);
    g.ncg = cdiv(hd, static_cast<int64_t>(p.mf_block > 0 ? p.mf_block : 32) * p.mf_col_waves);
    g.items = nchunks * g.nrg * g.ncg;
    const int64_t wg = p.mf_workgroups > 0 ? p.mf_workgroups : kDefaultCus;
    const int64_t g0 = g.items < wg ? g.items : wg;
    g.per = g0 > 0 ? cdiv(g.items, g0) : 0;
    g.grid = g.per > 0 ? cdiv(g.items, g.per) : 0;
    return g;
}

// Fill the derived fields of a plan and check it against the shape; lds_limit: max LDS bytes per workgroup.
int complete_plan(sdm_gx_plan_t* p, int64_t nchunks, int64_t C, int64_t hd, int64_t lds_limit) {
    if (nchunks < 0) return SDM_GX_ERR_ARG;
    if (p->engine == SDM_GX_ENGINE_MFMA) {
        if (p->mf_workgroups < 0) return SDM_GX_ERR_PLAN;
        if (p->mf_block == 0) p->mf_block = 32;
        if (p->slab_rows == 0) p->slab_rows = 16;
        if (p->mf_reg_slabs != 0) p->mf_aln = 0;
        const sdm_gx::MfmaEntry* e = find_mfma(*p);
        if (!e) return SDM_GX_ERR_PLAN;
        p->lds_bytes = e->lds_bytes;
        if (lds_limit > 0 && p->lds_bytes > lds_limit) return SDM_GX_ERR_LIMIT;
        const MfmaGeom g = mfma_geom(*p, nchunks, C, hd);
        if (g.items >= (int64_t(1) << 31)) return SDM_GX_ERR_LIMIT;   // item indices are 32-bit in the kernel
        p->grid = g.grid;
        return SDM_GX_OK;
    }
    if (p->engine != SDM_GX_ENGINE_VALU) return SDM_GX_ERR_PLAN;
    p->mf_aln = 0;
    if (!valid_ri(p->rows_per_wave) || !valid_rc(p->cols_per_lane) || !valid_waves(p->waves_per_wg))
        return SDM_GX_ERR_PLAN;
    if (p->staging != 0 && p->staging != 1) return SDM_GX_ERR_PLAN;
    if (p->xcd_remap != 0 && p->xcd_remap != 1) return SDM_GX_ERR_PLAN;
    if (p->rows_per_wave > C || p->slab_rows < 0) return SDM_GX_ERR_PLAN;
    if (!sdm_gx::find_kernel(p->rows_per_wave, p->cols_per_lane, p->waves_per_wg, p->staging)) return SDM_GX_ERR_PLAN;
    const int64_t cw = 64 * p->cols_per_lane;
    if (p->staging == 1) {
        int64_t sj = p->slab_rows;
        if (sj == 0) sj = kDefaultSlabBytes / (cw * 4);
        if (sj > C) sj = C;
        p->slab_rows = static_cast<int32_t>(sj);
        p->lds_bytes = static_cast<int32_t>(sj * cw * 4);
        if (lds_limit > 0 && p->lds_bytes > lds_limit) return SDM_GX_ERR_LIMIT;
    } else {
        p->slab_rows = 0;
        p->lds_bytes = 0;
    }
    const int64_t nrb = cdiv(C, p->rows_per_wave);
    const int64_t nrg = cdiv(nrb, p->waves_per_wg);
    const int64_t ncb = cdiv(hd, cw);
    p->grid = nchunks * nrg * ncb;
    return SDM_GX_OK;
}

// The matrix-core engine addresses a chunk of d_u with 32-bit byte offsets.
bool mfma_strides_ok(int64_t C, int64_t ld_u) { return C * ld_u * 4 < (int64_t(1) << 31); }

// Direct-to-LDS slabs (mf_reg_slabs 0) move 16-byte groups, all rows of x and of d_dv at one offset from a 16-byte
// boundary (C and ld_dv multiples of 4), and address a chunk of d_dv, and the rows past C that pad its last slab,
// with 32-bit byte offsets.
bool dma_strides_ok(int64_t C, int64_t ld_dv) {
    return C % 4 == 0 && ld_dv % 4 == 0 && (C + 32) * ld_dv * 4 < (int64_t(1) << 31);
}

// The instance a matrix-core plan runs for a layout. Direct-to-LDS plans whose x or d_dv rows start off a 16-byte
// boundary take the unaligned-row twin of their instance (mf_aln 4: d_dv rows by 4-byte DMA, x aligned; 2: d_dv rows
// from the 16-byte boundary below; 3: x rows too). Where the strides rule out direct-to-LDS slabs, or no twin
// exists, the same work items run through the register ring: 32-column wavefronts (a 16-column tile of 2k column
// wavefronts is k of them), 2 register slabs, 4 stages, 4 loader wavefronts. The results are the same either way.
int resolve_layout(sdm_gx_plan_t* p, int64_t C, const Layout& lay) {
    p->mf_aln = 0;
    if (p->engine != SDM_GX_ENGINE_MFMA || p->mf_reg_slabs != 0) return SDM_GX_OK;
    const bool xa = lay.x_mod16 == 0, da = lay.dv_mod16 == 0;
    if (dma_strides_ok(C, lay.ld_dv)) {
        if (xa && da) return SDM_GX_OK;
        for (int aln : {xa ? 4 : 3, xa ? 2 : 3}) {
            sdm_gx_plan_t q = *p;
            q.mf_aln = aln;
            if (find_mfma(q)) {
                *p = q;
                return SDM_GX_OK;
            }
        }
    }
    if (p->mf_block == 16) p->mf_col_waves /= 2;
    p->mf_block = 32;
    p->slab_rows = 16;
    p->mf_stages = 4;
    p->mf_reg_slabs = 2;
    p->mf_loader_waves = 4;
    p->mf_stream_du = 0;        // the register-ring kernel has no streaming-store variant
    return find_mfma(*p) ? SDM_GX_OK : SDM_GX_ERR_PLAN;
}

// A plan made complete for a launch: output fields filled, the instance resolved for the layout (mf_aln is an
// output; its input value is ignored), and every limit the launch will check checked here.
int finish_plan(sdm_gx_plan_t* p, int64_t nchunks, int64_t C, int64_t hd, const Layout& lay, int64_t lds_limit) {
    p->mf_aln = 0;
    int st = complete_plan(p, nchunks, C, hd, lds_limit);
    if (st || p->engine != SDM_GX_ENGINE_MFMA) return st;
    if (!mfma_strides_ok(C, lay.ld_u)) return SDM_GX_ERR_LIMIT;
    if ((st = resolve_layout(p, C, lay))) return st;
    return complete_plan(p, nchunks, C, hd, lds_limit);
}

// The launch planner. It plays the part of the page's launch rules for gx_gemm (_rows: rows per CTA from the grid
// target; _cap: CTAs per SM; one_wave: the kernel only for single-wave grids), re-derived for MI355X from
// interleaved timing of every plan (launches replayed from HIP graphs). The choice never changes results.
// Engine (`engine` -1): the matrix cores for 32 <= C when the direct-to-LDS kernel can take the strides (C and
// ld_dv multiples of 4), or when hd <= 128 (register-ring kernel); the vector ALUs otherwise (narrow chunks, where
// 64-row MFMA tiles would be mostly padding, and wide rows of odd strides). engine 0 or 1 forces one engine; the
// matrix cores also need C * ld_u * 4 < 2^31 (32-bit d_u offsets), else SDM_GX_ERR_LIMIT when forced.
//  Matrix cores, direct-to-LDS slabs: 16-column wavefronts (v_mfma_f32_16x16x1_4b_f32: half the chain latency per
//  work item of the 32-column MFMA), 3 LDS stages, 1 loader wavefront (1-3% faster than 4 stages; 6 or 8 slower).
//  Where one workgroup per CU walks several items and hd is a multiple of 128: 64 x 128 items on four 32-column
//  wavefronts (v_mfma_f32_32x32x1_2b_f32), 3 stages of 32 rows and 2 loader wavefronts (1 when x rows are off a
//  16-byte boundary, whose twin needs the extra group per row): half as many d_u accesses per item, in 128-byte row
//  segments; up to 3% faster warm and cold than 16-column wavefronts on C = 64 and C = 128 chunks.
//  Work items of 64 or 128 rows (C <= 64 or not) by 64 columns; 32 columns when hd <= 32, or when 64-column items
//  would leave CUs idle; 64 rows by 128 columns when C > 64 and hd is a multiple of 128 with items enough for every
//  CU (2% faster than 128 x 64 at C = hd = 128). Two workgroups per CU when an item has fewer than 8 compute
//  wavefronts and there are fewer than 4 items per CU, else one. One workgroup per CU walking several items: stages
//  of 32 chain rows (half the barrier bubbles, which no other workgroup fills). One item per workgroup: stages of 16
//  rows (the chain starts on a smaller first slab). Two workgroups per CU: stages of 16 rows and d_u stores with the
//  non-temporal hint (6% faster on 64x128 chunks; 6% slower on 128x128 chunks with one workgroup per CU). Rows off a
//  16-byte boundary take the unaligned-row twins (resolve_layout).
//  Matrix cores, register ring (strides that rule out direct-to-LDS slabs, hd <= 128): 32-column wavefronts, 64 or
//  128 rows by up to 128 columns, 4 register slabs and 4 stages; 128 x 128 items with 2 register slabs, d_u read at
//  the item's end and two workgroups per CU.
//  Vector ALUs:
//  * Columns per lane RC: the widest RC whose 64*RC-column blocks waste no more lanes than a narrower one.
//  * Rows per wavefront RI: 8 (two batches of 4 rows of x in flight), halved to 4 while the grid would
//    hold fewer than 8 wavefronts per CU (small steps are latency-bound: more, shorter tiles overlap better);
//    never more than C.
//  * 8 wavefronts per workgroup (fewer when the chunk has fewer row blocks, or when fewer would spread the grid
//    over more CUs: at least one workgroup per CU).
//  * RC <= 2: the workgroup stages d_dv through a 32 KiB LDS slab, with the XCD-grouped workgroup order.
//    RC = 4: each wavefront reads d_dv straight from global memory (64 columns of 16 bytes per row: the LDS round
//    trip measured slower there).
int plan_for(int64_t nchunks, int64_t C, int64_t hd, const Layout& lay, int engine, int num_cus, int lds_limit,
             sdm_gx_plan_t* out) {
    if (!out) return SDM_GX_ERR_ARG;
    if (C < 1 || C > SDM_GX_MAX_C || hd < 1 || hd >= SDM_GX_HD_LIMIT || nchunks < 0) return SDM_GX_ERR_SHAPE;
    if (engine != -1 && engine != SDM_GX_ENGINE_VALU && engine != SDM_GX_ENGINE_MFMA) return SDM_GX_ERR_ARG;
    if (num_cus < 1) num_cus = kDefaultCus;
    const bool allow_mfma = engine != SDM_GX_ENGINE_VALU && mfma_strides_ok(C, lay.ld_u);
    if (engine == SDM_GX_ENGINE_MFMA && !allow_mfma) return SDM_GX_ERR_LIMIT;
    const bool dma_ok = dma_strides_ok(C, lay.ld_dv);
    if (allow_mfma && (engine == SDM_GX_ENGINE_MFMA || (C >= 32 && (dma_ok || hd <= 128)))) {
        sdm_gx_plan_t p{};
        p.engine = SDM_GX_ENGINE_MFMA;
        int st;
        if (dma_ok) {                                   // direct-to-LDS slabs, 16-column wavefronts
            p.mf_block = 16;
            p.mf_row_waves = C > 64 ? 2 : 1;
            p.mf_col_waves = hd > 32 ? 4 : 2;
            if (nchunks * cdiv(C, 64 * p.mf_row_waves) * cdiv(hd, 64) < num_cus) p.mf_col_waves = 2;
            else if (C > 64 && hd % 128 == 0 && nchunks * cdiv(C, 64) * (hd / 128) >= num_cus) {
                p.mf_row_waves = 1;                     // 64 x 128 items
                p.mf_col_waves = 8;
            }
            p.mf_stages = 3;
            p.mf_reg_slabs = 0;
            p.mf_loader_waves = 1;
            const int64_t items = nchunks * cdiv(C, 64 * p.mf_row_waves) * cdiv(hd, 16 * p.mf_col_waves);
            p.mf_workgroups = (p.mf_row_waves * p.mf_col_waves < 8 && items < 4 * num_cus ? 2 : 1) * num_cus;
            p.slab_rows = 16;
            st = complete_plan(&p, nchunks, C, hd, lds_limit);
            if (st == SDM_GX_OK && p.grid <= num_cus) {         // one workgroup per CU
                if (items > p.grid) p.slab_rows = 32;           // walking several items: 32-row stages
                if (items > p.grid && hd % 128 == 0) {          // streaming 64 x 128 items: 32-column wavefronts
                    sdm_gx_plan_t q = p;
                    q.mf_block = 32;
                    q.mf_row_waves = 1;
                    q.mf_col_waves = 4;
                    q.mf_workgroups = num_cus;
                    q.mf_loader_waves = lay.x_mod16 == 0 ? 2 : 1;   // 2: d_dv rows by 4-byte DMA when unaligned
                    const int64_t items32 = nchunks * cdiv(C, 64) * (hd / 128);
                    if (items32 > num_cus && complete_plan(&q, nchunks, C, hd, lds_limit) == SDM_GX_OK) p = q;
                }
            } else {                                            // two per CU: streaming d_u stores
                p.mf_stream_du = 1;
            }
        } else {                                        // register ring, 32-column wavefronts
            p.mf_block = 32;
            p.mf_row_waves = C > 64 ? 2 : 1;
            p.mf_col_waves = static_cast<int32_t>(cdiv(hd, 32) > 2 ? 4 : cdiv(hd, 32));
            p.mf_stages = 4;
            p.mf_reg_slabs = 4;
            p.mf_loader_waves = p.mf_row_waves * p.mf_col_waves <= 2 ? 2 : 4;
            p.mf_workgroups = num_cus;
            if (p.mf_row_waves == 2 && p.mf_col_waves == 4) {   // 128 x 128 items: two workgroups per CU
                p.mf_reg_slabs = 2;
                p.mf_du_at_end = 1;
                p.mf_workgroups = 2 * num_cus;
            }
        }
        st = finish_plan(&p, nchunks, C, hd, lay, lds_limit);
        if (st == SDM_GX_OK) {
            *out = p;
            return SDM_GX_OK;
        }
        if (st != SDM_GX_ERR_LIMIT || engine == SDM_GX_ENGINE_MFMA) return st;
    }
    int rc = 1;
    int64_t best_waste = cdiv(hd, 64) * 64 - hd;
    for (int cand : {2, 4}) {
        const int64_t w = cdiv(hd, 64 * cand) * 64 * cand - hd;
        if (w <= best_waste) {
            best_waste = w;
            rc = cand;
        }
    }
    int ri = 1;
    while (ri * 2 <= 8 && ri * 2 <= C) ri *= 2;
    const int64_t ncb = cdiv(hd, 64 * rc);
    while (ri > 4 && nchunks * cdiv(C, ri) * ncb < 8LL * num_cus) ri /= 2;
    const int64_t nrb = cdiv(C, ri);
    int waves = 1;
    while (waves * 2 <= 8 && waves * 2 <= nrb) waves *= 2;
    while (waves > 1 && nchunks * cdiv(nrb, waves) * ncb < num_cus) waves /= 2;   // at least one workgroup per CU
    sdm_gx_plan_t p{};
    p.engine = SDM_GX_ENGINE_VALU;
    p.rows_per_wave = ri;
    p.cols_per_lane = rc;
    p.waves_per_wg = waves;
    p.staging = rc <= 2 ? 1 : 0;
    p.xcd_remap = rc <= 2 ? 1 : 0;
    p.slab_rows = 0;
    int st = finish_plan(&p, nchunks, C, hd, lay, lds_limit);
    if (st == SDM_GX_ERR_LIMIT) {               // a device with less LDS per workgroup: read d_dv directly
        p.staging = 0;
        st = finish_plan(&p, nchunks, C, hd, lay, lds_limit);
    }
    if (st) return st;
    *out = p;
    return SDM_GX_OK;
}

// The placement arguments of the planner entry points: byte offsets from a 16-byte boundary.
bool valid_mod16(int32_t v) { return v >= 0 && v < 16 && v % 4 == 0; }

// ---- launching ----------------------------------------------------------------------------------------------------
// Chunks n_begin .. n_begin + nchunks - 1 with a completed, validated plan. Splits very large grids so that one
// launch stays below 2^31 work-items.
// One kernel launch: function, shape and the argument block it takes by value.
struct LaunchRec {
    const void* fn = nullptr;
    unsigned grid = 0, block = 0, lds = 0;
    bool mfma = false;
    sdm_gx::KernelArgs va{};
    sdm_gx::MfmaArgs ma{};
    void* args() const { return mfma ? const_cast<sdm_gx::MfmaArgs*>(&ma) : static_cast<void*>(const_cast<sdm_gx::KernelArgs*>(&va)); }
};

// The kernel launches that update chunks n_begin .. n_begin + nchunks - 1 with a completed, validated plan, in
// order, each handed to sink(const LaunchRec&) -> hipError_t. The vector-ALU engine splits very large grids so that
// one launch stays below 2^31 work-items; the matrix-core engine is one launch.
template <class Sink>
int for_each_launch(const sdm_gx_plan_t& p, float* du, int64_t ld_u, const float* x, const float* dv, int64_t ld_dv,
                    int64_t n_begin, int64_t nchunks, int64_t C, int64_t hd, Sink&& sink) {
    if (nchunks <= 0) return SDM_GX_OK;
    LaunchRec r;
    if (p.engine == SDM_GX_ENGINE_MFMA) {
        const sdm_gx::MfmaEntry* e = find_mfma(p);
        if (!e) return SDM_GX_ERR_PLAN;
        if (!mfma_strides_ok(C, ld_u)) return SDM_GX_ERR_LIMIT;
        if (e->reg_slabs == 0) {
            // the plan was resolved for this layout (finish_plan); a direct-to-LDS instance needs its strides, and
            // rows on 16-byte boundaries wherever it has no unaligned-row path for them
            const Layout lay = layout_of(ld_u, ld_dv, x, dv);
            if (!dma_strides_ok(C, ld_dv) || (!(e->aln & 1) && lay.x_mod16 != 0) ||
                (!(e->aln & 6) && lay.dv_mod16 != 0))
                return SDM_GX_ERR_PLAN;
        }
        const MfmaGeom g = mfma_geom(p, nchunks, C, hd);
        if (g.items >= (int64_t(1) << 31)) return SDM_GX_ERR_LIMIT;     // item indices are 32-bit in the kernel
        r.mfma = true;
        r.fn = e->fn;
        r.grid = static_cast<unsigned>(g.grid);
        r.block = 64u * static_cast<unsigned>(e->row_waves * e->col_waves + e->loader_waves);
        r.lds = 0;
        sdm_gx::MfmaArgs& a = r.ma;
        a.du = du;
        a.x = x;
        a.dv = dv;
        a.ld_u = ld_u;
        a.ld_dv = ld_dv;
        a.n_begin = n_begin;
        a.n_items = static_cast<int32_t>(g.items);
        a.per = static_cast<int32_t>(g.per);
        a.C = static_cast<int32_t>(C);
        a.hd = static_cast<int32_t>(hd);
        a.nrg = static_cast<int32_t>(g.nrg);
        a.ncg = static_cast<int32_t>(g.ncg);
        a.stream_du = p.mf_stream_du != 0;
        const hipError_t err = sink(static_cast<const LaunchRec&>(r));
        return err == hipSuccess ? SDM_GX_OK : hip_fail(err);
    }
    const void* fn = sdm_gx::find_kernel(p.rows_per_wave, p.cols_per_lane, p.waves_per_wg, p.staging);
    if (!fn) return SDM_GX_ERR_PLAN;
    const int64_t nrb = cdiv(C, p.rows_per_wave);
    const int64_t nrg = cdiv(nrb, p.waves_per_wg);
    const int64_t ncb = cdiv(hd, 64 * p.cols_per_lane);
    const int64_t per_chunk = nrg * ncb;
    const int64_t max_blocks = (int64_t(1) << 31) / (64 * p.waves_per_wg);
    int64_t step = max_blocks / per_chunk;
    if (step < 1) return SDM_GX_ERR_LIMIT;
    r.fn = fn;
    r.block = 64u * static_cast<unsigned>(p.waves_per_wg);
    r.lds = static_cast<unsigned>(p.lds_bytes);
    sdm_gx::KernelArgs& a = r.va;
    a.du = du;
    a.x = x;
    a.dv = dv;
    a.ld_u = ld_u;
    a.ld_dv = ld_dv;
    a.C = static_cast<int32_t>(C);
    a.hd = static_cast<int32_t>(hd);
    a.nrg = static_cast<int32_t>(nrg);
    a.ncb = static_cast<int32_t>(ncb);
    a.xcd_remap = p.xcd_remap;
    a.slab_rows = p.slab_rows;
    for (int64_t s = 0; s < nchunks; s += step) {
        const int64_t cnt = nchunks - s < step ? nchunks - s : step;
        a.n_begin = n_begin + s;
        r.grid = static_cast<unsigned>(cnt * per_chunk);
        const hipError_t e = sink(static_cast<const LaunchRec&>(r));
        if (e != hipSuccess) return hip_fail(e);
    }
    return SDM_GX_OK;
}

int launch_chunks(const sdm_gx_plan_t& p, float* du, int64_t ld_u, const float* x, const float* dv, int64_t ld_dv,
                  int64_t n_begin, int64_t nchunks, int64_t C, int64_t hd, hipStream_t stream) {
    return for_each_launch(p, du, ld_u, x, dv, ld_dv, n_begin, nchunks, C, hd, [stream](const LaunchRec& r) {
        void* args[] = {r.args()};
        return hipLaunchKernel(r.fn, dim3(r.grid), dim3(r.block), args, r.lds, stream);
    });
}

// Plan (given or planned) for nchunks chunks on a device with `info`, resolved for the launch's layout.
int resolve_plan(const sdm_gx_plan_t* given, int64_t nchunks, int64_t C, int64_t hd, const Layout& lay,
                 const DeviceInfo& info, sdm_gx_plan_t* out) {
    if (given) {
        *out = *given;
        if (out->engine == SDM_GX_ENGINE_MFMA && out->mf_workgroups == 0) out->mf_workgroups = info.num_cus;
        return finish_plan(out, nchunks, C, hd, lay, info.lds_per_wg);
    }
    return plan_for(nchunks, C, hd, lay, -1, info.num_cus, info.lds_per_wg, out);
}

int check_device_pointers(const float* du, const float* x, const float* dv, int dev) {
    int st = on_device(du, dev);
    if (!st) st = on_device(x, dev);
    if (!st) st = on_device(dv, dev);
    return st;
}

}  // namespace

extern "C" {

int sdm_gx_check(const float* d_u, int64_t ld_u, const float* x, const float* d_dv, int64_t ld_dv, int64_t N,
                 int64_t ti, int64_t P, int64_t C, int64_t hd) {
    return check_args(d_u, ld_u, x, d_dv, ld_dv, N, ti, P, C, hd);
}

int sdm_gx_gemm_ex(float* d_u, int64_t ld_u, const float* x, const float* d_dv, int64_t ld_dv, int64_t N, int64_t ti,
                   int64_t P, int64_t C, int64_t hd, const sdm_gx_plan_t* plan, void* stream) {
    int st = check_args(d_u, ld_u, x, d_dv, ld_dv, N, ti, P, C, hd);
    if (st) return st;
    int dev = 0;
    DeviceInfo info;
    if ((st = current_device(&dev, &info))) return st;
    if ((st = check_device_pointers(d_u, x, d_dv, dev))) return st;
    sdm_gx_plan_t p;
    if ((st = resolve_plan(plan, P, C, hd, layout_of(ld_u, ld_dv, x, d_dv), info, &p))) return st;
    return launch_chunks(p, d_u, ld_u, x, d_dv, ld_dv, ti * P, P, C, hd, static_cast<hipStream_t>(stream));
}

int sdm_gx_gemm(float* d_u, const float* x, const float* d_dv, int64_t ti, int64_t P, int64_t C, int64_t hd,
                void* stream) {
    if (P < 1) return SDM_GX_ERR_SHAPE;
    if (ti < 0 || ti >= (SDM_GX_N_LIMIT - 1) / P) return SDM_GX_ERR_STEP;    // (ti + 1) * P < 2^31
    const int64_t N = (ti + 1) * P;
    return sdm_gx_gemm_ex(d_u, hd, x, d_dv, hd, N, ti, P, C, hd, nullptr, stream);
}

int sdm_gx_gemm_steps(float* d_u, int64_t ld_u, const float* x, const float* d_dv, int64_t ld_dv, int64_t N,
                      int64_t P, int64_t C, int64_t hd, int64_t ti_begin, int64_t ti_end, int32_t mode,
                      const sdm_gx_plan_t* plan, void* stream) {
    if (mode != SDM_GX_STEPS_FORWARD && mode != SDM_GX_STEPS_REVERSE && mode != SDM_GX_STEPS_FUSED)
        return SDM_GX_ERR_ARG;
    if (ti_begin < 0 || ti_end < ti_begin) return SDM_GX_ERR_STEP;
    // validate once, at the last step of the range (its bound covers every earlier step)
    int st = check_args(d_u, ld_u, x, d_dv, ld_dv, N, ti_end > ti_begin ? ti_end - 1 : ti_begin, P, C, hd);
    if (st) return st;
    if (ti_end == ti_begin) return SDM_GX_OK;
    int dev = 0;
    DeviceInfo info;
    if ((st = current_device(&dev, &info))) return st;
    if ((st = check_device_pointers(d_u, x, d_dv, dev))) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    sdm_gx_plan_t p;
    if (mode == SDM_GX_STEPS_FUSED) {
        const int64_t nchunks = (ti_end - ti_begin) * P;
        if ((st = resolve_plan(plan, nchunks, C, hd, layout_of(ld_u, ld_dv, x, d_dv), info, &p))) return st;
        return launch_chunks(p, d_u, ld_u, x, d_dv, ld_dv, ti_begin * P, nchunks, C, hd, s);
    }
    if ((st = resolve_plan(plan, P, C, hd, layout_of(ld_u, ld_dv, x, d_dv), info, &p))) return st;
    for (int64_t k = 0; k < ti_end - ti_begin; ++k) {
        const int64_t ti = mode == SDM_GX_STEPS_FORWARD ? ti_begin + k : ti_end - 1 - k;
        if ((st = launch_chunks(p, d_u, ld_u, x, d_dv, ld_dv, ti * P, P, C, hd, s))) return st;
    }
    return SDM_GX_OK;
}

int sdm_gx_plan(int64_t nchunks, int64_t C, int64_t hd, int64_t ld_u, int64_t ld_dv, int32_t x_mod16,
                int32_t dv_mod16, int32_t engine, int32_t device, sdm_gx_plan_t* out) {
    if (!out) return SDM_GX_ERR_ARG;
    if (ld_u < hd || ld_dv < hd || ld_u >= SDM_GX_LD_LIMIT || ld_dv >= SDM_GX_LD_LIMIT) return SDM_GX_ERR_STRIDE;
    if (!valid_mod16(x_mod16) || !valid_mod16(dv_mod16)) return SDM_GX_ERR_ALIGN;
    int dev = device;
    if (dev < 0) {
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_fail(e);
    }
    DeviceInfo info;
    int st = device_info(dev, &info);
    if (st) return st;
    if (!info.gfx950) return SDM_GX_ERR_DEVICE;
    const Layout lay{ld_u, ld_dv, x_mod16, dv_mod16};
    if ((st = plan_for(nchunks, C, hd, lay, engine, info.num_cus, info.lds_per_wg, out))) return st;
    const void* fn;
    int threads, dyn_lds;
    if (out->engine == SDM_GX_ENGINE_MFMA) {
        const sdm_gx::MfmaEntry* e = find_mfma(*out);
        fn = e->fn;
        threads = 64 * (out->mf_row_waves * out->mf_col_waves + out->mf_loader_waves);
        dyn_lds = 0;
    } else {
        fn = sdm_gx::find_kernel(out->rows_per_wave, out->cols_per_lane, out->waves_per_wg, out->staging);
        threads = 64 * out->waves_per_wg;
        dyn_lds = out->lds_bytes;
    }
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, threads, dyn_lds) == hipSuccess)
        out->wgs_per_cu = blocks;
    else
        (void)hipGetLastError();
    return SDM_GX_OK;
}

int sdm_gx_plan_for(int64_t nchunks, int64_t C, int64_t hd, int64_t ld_u, int64_t ld_dv, int32_t x_mod16,
                    int32_t dv_mod16, int32_t engine, int32_t num_cus, int32_t lds_per_cu, sdm_gx_plan_t* out) {
    if (!out) return SDM_GX_ERR_ARG;
    if (ld_u < hd || ld_dv < hd || ld_u >= SDM_GX_LD_LIMIT || ld_dv >= SDM_GX_LD_LIMIT) return SDM_GX_ERR_STRIDE;
    if (!valid_mod16(x_mod16) || !valid_mod16(dv_mod16)) return SDM_GX_ERR_ALIGN;
    return plan_for(nchunks, C, hd, Layout{ld_u, ld_dv, x_mod16, dv_mod16}, engine, num_cus, lds_per_cu, out);
}

int sdm_gx_plan_complete(sdm_gx_plan_t* plan, int64_t nchunks, int64_t C, int64_t hd, int64_t ld_u, int64_t ld_dv,
                         int32_t x_mod16, int32_t dv_mod16, int32_t lds_per_cu) {
    if (!plan) return SDM_GX_ERR_ARG;
    if (C < 1 || C > SDM_GX_MAX_C || hd < 1 || hd >= SDM_GX_HD_LIMIT) return SDM_GX_ERR_SHAPE;
    if (ld_u < hd || ld_dv < hd || ld_u >= SDM_GX_LD_LIMIT || ld_dv >= SDM_GX_LD_LIMIT) return SDM_GX_ERR_STRIDE;
    if (!valid_mod16(x_mod16) || !valid_mod16(dv_mod16)) return SDM_GX_ERR_ALIGN;
    return finish_plan(plan, nchunks, C, hd, Layout{ld_u, ld_dv, x_mod16, dv_mod16}, lds_per_cu);
}

int sdm_gx_prepare(sdm_gx_launch_t* out, float* d_u, int64_t ld_u, const float* x, const float* d_dv, int64_t ld_dv,
                   int64_t N, int64_t P, int64_t C, int64_t hd, int64_t ti_max, const sdm_gx_plan_t* plan) {
    if (!out) return SDM_GX_ERR_ARG;
    std::memset(out, 0, sizeof(*out));
    int st = check_args(d_u, ld_u, x, d_dv, ld_dv, N, ti_max, P, C, hd);
    if (st) return st;
    int dev = 0;
    DeviceInfo info;
    if ((st = current_device(&dev, &info))) return st;
    if ((st = check_device_pointers(d_u, x, d_dv, dev))) return st;
    sdm_gx_launch_t l;
    std::memset(&l, 0, sizeof(l));
    const Layout lay = layout_of(ld_u, ld_dv, x, d_dv);
    if ((st = resolve_plan(plan, P, C, hd, lay, info, &l.plan_step))) return st;
    if ((st = resolve_plan(plan, (ti_max + 1) * P, C, hd, lay, info, &l.plan_fused))) return st;
    l.device = dev;
    l.d_u = d_u;
    l.x = x;
    l.d_dv = d_dv;
    l.ld_u = ld_u;
    l.ld_dv = ld_dv;
    l.N = N;
    l.P = P;
    l.C = C;
    l.hd = hd;
    l.ti_max = ti_max;
    l.magic = kLaunchMagic;
    *out = l;
    return SDM_GX_OK;
}

static int prepared_ok(const sdm_gx_launch_t* l) {
    if (!l || l->magic != kLaunchMagic) return SDM_GX_ERR_PLAN;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev != l->device) return SDM_GX_ERR_DEVICE;
    return SDM_GX_OK;
}

int sdm_gx_launch(const sdm_gx_launch_t* prepared, int64_t ti, void* stream) {
    int st = prepared_ok(prepared);
    if (st) return st;
    const sdm_gx_launch_t& l = *prepared;
    if (ti < 0 || ti > l.ti_max) return SDM_GX_ERR_STEP;
    return launch_chunks(l.plan_step, l.d_u, l.ld_u, l.x, l.d_dv, l.ld_dv, ti * l.P, l.P, l.C, l.hd,
                         static_cast<hipStream_t>(stream));
}

int sdm_gx_launch_fused(const sdm_gx_launch_t* prepared, int64_t ti_begin, int64_t ti_end, void* stream) {
    int st = prepared_ok(prepared);
    if (st) return st;
    const sdm_gx_launch_t& l = *prepared;
    if (ti_begin < 0 || ti_end < ti_begin || ti_end > l.ti_max + 1) return SDM_GX_ERR_STEP;
    return launch_chunks(l.plan_fused, l.d_u, l.ld_u, l.x, l.d_dv, l.ld_dv, ti_begin * l.P, (ti_end - ti_begin) * l.P,
                         l.C, l.hd, static_cast<hipStream_t>(stream));
}

// ---- HIP graphs of a prepared step range --------------------------------------------------------------------------
struct sdm_gx_graph {
    uint64_t magic;
    int32_t device;
    int64_t nodes;
    hipGraph_t graph;
    hipGraphExec_t exec;
};

constexpr uint64_t kGraphMagic = 0x4850415247584753ull;   // graph tag

int sdm_gx_graph_create(sdm_gx_graph_t** out, const sdm_gx_launch_t* prepared, int64_t ti_begin, int64_t ti_end,
                        int32_t mode) {
    if (!out) return SDM_GX_ERR_ARG;
    *out = nullptr;
    if (mode != SDM_GX_STEPS_FORWARD && mode != SDM_GX_STEPS_REVERSE && mode != SDM_GX_STEPS_FUSED)
        return SDM_GX_ERR_ARG;
    int st = prepared_ok(prepared);
    if (st) return st;
    const sdm_gx_launch_t& l = *prepared;
    if (ti_begin < 0 || ti_end < ti_begin || ti_end > l.ti_max + 1) return SDM_GX_ERR_STEP;
    hipGraph_t graph = nullptr;
    hipError_t e = hipGraphCreate(&graph, 0);
    if (e != hipSuccess) return hip_fail(e);
    hipGraphNode_t prev = nullptr;
    int64_t nodes = 0;
    auto add = [&](const LaunchRec& r) {               // kernel nodes in issue order, each after the previous one
        hipKernelNodeParams np{};
        void* args[] = {r.args()};
        np.func = const_cast<void*>(r.fn);
        np.gridDim = dim3(r.grid);
        np.blockDim = dim3(r.block);
        np.sharedMemBytes = r.lds;
        np.kernelParams = args;
        np.extra = nullptr;
        hipGraphNode_t node = nullptr;
        const hipError_t err = hipGraphAddKernelNode(&node, graph, prev ? &prev : nullptr, prev ? 1 : 0, &np);
        if (err == hipSuccess) {
            prev = node;
            ++nodes;
        }
        return err;
    };
    if (mode == SDM_GX_STEPS_FUSED) {
        st = for_each_launch(l.plan_fused, l.d_u, l.ld_u, l.x, l.d_dv, l.ld_dv, ti_begin * l.P,
                             (ti_end - ti_begin) * l.P, l.C, l.hd, add);
    } else {
        for (int64_t k = 0; k < ti_end - ti_begin && !st; ++k) {
            const int64_t ti = mode == SDM_GX_STEPS_FORWARD ? ti_begin + k : ti_end - 1 - k;
            st = for_each_launch(l.plan_step, l.d_u, l.ld_u, l.x, l.d_dv, l.ld_dv, ti * l.P, l.P, l.C, l.hd, add);
        }
    }
    hipGraphExec_t exec = nullptr;
    if (!st) {
        e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
        if (e != hipSuccess) st = hip_fail(e);
    }
    sdm_gx_graph* g = nullptr;
    if (!st) {
        g = new (std::nothrow) sdm_gx_graph;
        if (!g) st = SDM_GX_ERR_HIP;
    }
    if (st) {
        if (exec) (void)hipGraphExecDestroy(exec);
        (void)hipGraphDestroy(graph);
        return st;
    }
    g->magic = kGraphMagic;
    g->device = l.device;
    g->nodes = nodes;
    g->graph = graph;
    g->exec = exec;
    *out = g;
    return SDM_GX_OK;
}

int sdm_gx_graph_launch(const sdm_gx_graph_t* graph, void* stream) {
    if (!graph || graph->magic != kGraphMagic) return SDM_GX_ERR_PLAN;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev != graph->device) return SDM_GX_ERR_DEVICE;
    e = hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SDM_GX_OK : hip_fail(e);
}

int64_t sdm_gx_graph_nodes(const sdm_gx_graph_t* graph) {
    return graph && graph->magic == kGraphMagic ? graph->nodes : -1;
}

int sdm_gx_graph_destroy(sdm_gx_graph_t* graph) {
    if (!graph) return SDM_GX_OK;
    if (graph->magic != kGraphMagic) return SDM_GX_ERR_PLAN;
    hipError_t e1 = hipGraphExecDestroy(graph->exec);
    hipError_t e2 = hipGraphDestroy(graph->graph);
    graph->magic = 0;
    delete graph;
    if (e1 != hipSuccess) return hip_fail(e1);
    if (e2 != hipSuccess) return hip_fail(e2);
    return SDM_GX_OK;
}

int sdm_gx_kernel_attrs(const sdm_gx_plan_t* plan, int64_t out[5]) {
    if (!plan || !out) return SDM_GX_ERR_ARG;
    const void* fn = nullptr;
    if (plan->engine == SDM_GX_ENGINE_MFMA) {
        const sdm_gx::MfmaEntry* e = find_mfma(*plan);
        if (e) fn = e->fn;
    } else if (plan->engine == SDM_GX_ENGINE_VALU) {
        fn = sdm_gx::find_kernel(plan->rows_per_wave, plan->cols_per_lane, plan->waves_per_wg, plan->staging);
    }
    if (!fn) return SDM_GX_ERR_PLAN;
    hipFuncAttributes a;
    hipError_t e = hipFuncGetAttributes(&a, fn);
    if (e != hipSuccess) return hip_fail(e);
    out[0] = a.numRegs;
    out[1] = static_cast<int64_t>(a.localSizeBytes);
    out[2] = static_cast<int64_t>(a.sharedSizeBytes);
    out[3] = a.maxThreadsPerBlock;
    out[4] = plan->engine == SDM_GX_ENGINE_MFMA ? 0 : plan->lds_bytes;
    return SDM_GX_OK;
}

const char* sdm_gx_strerror(int code) {
    switch (code) {
        case SDM_GX_OK: return "ok";
        case SDM_GX_ERR_NULL: return "a required pointer is NULL";
        case SDM_GX_ERR_SHAPE: return "shape out of range (need 1 <= C <= 256, 1 <= hd < 2^20, 1 <= P, 1 <= N < 2^31)";
        case SDM_GX_ERR_STEP: return "step out of range (need 1 <= P <= N and 0 <= ti < N / P)";
        case SDM_GX_ERR_ALIGN: return "pointer not 4-byte aligned";
        case SDM_GX_ERR_OVERLAP: return "d_u overlaps x or d_dv (the in-place update needs disjoint operands)";
        case SDM_GX_ERR_STRIDE: return "row stride out of range (need hd <= ld < 2^31)";
        case SDM_GX_ERR_LIMIT: return "launch exceeds a device or engine limit";
        case SDM_GX_ERR_HIP: return "HIP runtime error (see sdm_gx_last_hip_error)";
        case SDM_GX_ERR_PLAN: return "invalid plan or prepared launch";
        case SDM_GX_ERR_DEVICE: return "no gfx950 device, or a pointer / prepared launch is not on the current device";
        case SDM_GX_ERR_ARG: return "invalid argument";
        default: return "unknown status";
    }
}

int sdm_gx_last_hip_error(void) { return g_last_hip_error; }

int sdm_gx_abi_version(void) { return SDM_GX_ABI_VERSION; }

}  // extern "C"
