// Host entry points of Phase A (sdm_gx_pa2.h): argument checks, the planner, per-step launches. Every arithmetic
// step runs in gx_pa2_kernel.hip.
//
// The checks follow the page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_pa2_cuda.py", host entry
// gx_pa2_run (shapes, step range, row counts, alignment, operands on one device); the planner takes the part of its
// plan() and tile_len() (warps per CTA, ring depth, a tile length that fills one wave of CTAs).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/sdm_gx_pa2.h"
#include "gx_pa2.h"

namespace sdm_gx {
int record_hip_error(hipError_t e);     // gx_gemm_api.cpp: keeps e for sdm_gx_last_hip_error, returns SDM_GX_ERR_HIP
}

namespace {

constexpr int kTargetWavesPerCu = 32;    // 8 per SIMD: gathers at group starts are latency-bound
constexpr int kMinTile = 4;     // records per tile at least (4 measured 8% faster than 8 on 64 x 8-record chunks)

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// LDS of a workgroup: token rows of its slices and beta, then, with staged outputs, a count and the outputs
int64_t lds_base(const sdm_pa2_args_t* a, int32_t slices_per_wave) {
    return a->C * 16 * 32 * slices_per_wave + a->C * 4;
}
int64_t lds_staged(const sdm_pa2_args_t* a, int32_t slices_per_wave) {
    const int64_t planes = (1 + (a->hd - 1) / 128 >= 2 && slices_per_wave == 2) ? 4 : 2;
    return 4 + planes * a->C * a->W * 4;
}

// Outputs go through LDS when one workgroup holds a whole chunk (ctas == 1) and they add at most a quarter to its
// LDS: each output plane of the chunk is then written in one contiguous run instead of one scattered 4-byte store per
// record and plane (with the 80-SGPR instance, 3.7% off a5's step).
bool stage_outputs(const sdm_pa2_args_t* a, const sdm_pa2_plan_t& p) {
    const int64_t base = lds_base(a, p.slices_per_wave), staged = lds_staged(a, p.slices_per_wave);
    return p.stage_out == 1 && p.ctas == 1 && 4 * staged <= base && p.lds_bytes == base + staged;
}

struct Extent {
    uintptr_t lo, hi;
};

Extent extent(const void* p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Extent{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlap(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

int64_t slices(int64_t hd) { return 1 + (hd - 1) / 128; }
int64_t slice_width(int64_t hd) {
    const int64_t nsl = slices(hd);
    return 4 * ((cdiv(hd, 4) + nsl - 1) / nsl);
}

int check(const sdm_pa2_args_t* a, int64_t ti) {
    if (!a) return SDM_GX_ERR_ARG;
    if (!a->grad || !a->bank || !a->snap || !a->d_u || !a->beta || !a->kpay || !a->rec || !a->out_eff || !a->out_g)
        return SDM_GX_ERR_NULL;
    if (a->ssr < 0 && !a->bpre) return SDM_GX_ERR_NULL;
    if (a->C < 1 || a->C > 256 || a->W < 1 || a->W > 256 || a->hd < 1 || a->hd >= SDM_GX_HD_LIMIT)
        return SDM_GX_ERR_SHAPE;
    if (a->N < 1 || a->N >= SDM_GX_N_LIMIT || a->P < 1) return SDM_GX_ERR_SHAPE;
    if (a->slots < 1 || a->slots >= (int64_t(1) << 31) || a->snap_rows < 0) return SDM_GX_ERR_SHAPE;
    if (a->ld_u < a->hd || a->ld_u >= SDM_GX_LD_LIMIT) return SDM_GX_ERR_STRIDE;
    if (a->P > a->N || ti < 0 || ti >= a->N / a->P) return SDM_GX_ERR_STEP;
    const int64_t n = a->C * a->W, nsl = slices(a->hd);
    if (a->planes != (nsl == 1 ? 1 : nsl) || a->plane < a->N * n) return SDM_GX_ERR_SHAPE;
    // the snapshot covers step ti (the page's need_rows for each reader)
    const int64_t need = a->ssr < 0 ? (ti + 1) * a->P * n : ti * a->ssr + a->P * n;
    if (need > a->snap_rows) return SDM_GX_ERR_SHAPE;
    const uintptr_t f4 = reinterpret_cast<uintptr_t>(a->grad) | reinterpret_cast<uintptr_t>(a->bank) |
                         reinterpret_cast<uintptr_t>(a->snap) | reinterpret_cast<uintptr_t>(a->d_u) |
                         reinterpret_cast<uintptr_t>(a->beta) | reinterpret_cast<uintptr_t>(a->kpay) |
                         reinterpret_cast<uintptr_t>(a->bpre) | reinterpret_cast<uintptr_t>(a->out_eff) |
                         reinterpret_cast<uintptr_t>(a->out_g);
    if ((f4 & 3u) || (reinterpret_cast<uintptr_t>(a->rec) & 15u)) return SDM_GX_ERR_ALIGN;
    const int64_t hd = a->hd;
    const Extent w[] = {extent(a->grad, a->slots * hd * 4), extent(a->bank, a->slots * hd * 4),
                        extent(a->out_eff, a->planes * a->plane * 4), extent(a->out_g, a->planes * a->plane * 4)};
    const int64_t nb = cdiv(n, 32) + 1;
    const Extent r[] = {extent(a->snap, a->snap_rows * hd * 4), extent(a->d_u, ((a->N * a->C - 1) * a->ld_u + hd) * 4),
                        extent(a->beta, a->N * a->C * 4), extent(a->kpay, a->N * n * 4),
                        extent(a->rec, a->N * n * 16), extent(a->bpre, a->bpre ? a->N * nb * 4 : 0)};
    for (int i = 0; i < 4; ++i) {
        for (int j = i + 1; j < 4; ++j)
            if (overlap(w[i], w[j])) return SDM_GX_ERR_OVERLAP;
        for (const Extent& e : r)
            if (overlap(w[i], e)) return SDM_GX_ERR_OVERLAP;
    }
    return SDM_GX_OK;
}

int complete(const sdm_pa2_args_t* a, int lds_limit, sdm_pa2_plan_t* p) {
    const int64_t n = a->C * a->W, nsl = slices(a->hd);
    if (p->slices_per_wave != 1 && p->slices_per_wave != 2) return SDM_GX_ERR_PLAN;
    if (p->waves_per_wg != 4 && p->waves_per_wg != 8 && p->waves_per_wg != 16) return SDM_GX_ERR_PLAN;
    if (p->tile_len < 1) return SDM_GX_ERR_PLAN;
    const int64_t tiles = cdiv(n, p->tile_len);
    p->ctas = static_cast<int32_t>(cdiv(tiles, p->waves_per_wg));
    p->npair = static_cast<int32_t>(p->slices_per_wave == 2 ? cdiv(nsl, 2) : nsl);
    const int64_t base = lds_base(a, p->slices_per_wave), staged = lds_staged(a, p->slices_per_wave);
    if (lds_limit > 0 && base > lds_limit) {
        p->lds_bytes = static_cast<int32_t>(base);
        p->stage_out = 0;
        return SDM_GX_ERR_LIMIT;
    }
    const bool stage = p->ctas == 1 && 4 * staged <= base && (lds_limit <= 0 || base + staged <= lds_limit);
    p->lds_bytes = static_cast<int32_t>(stage ? base + staged : base);
    p->stage_out = stage ? 1 : 0;
    const int64_t grid = a->P * p->npair * p->ctas;
    if (grid >= (int64_t(1) << 31)) return SDM_GX_ERR_LIMIT;
    p->grid = grid;
    return SDM_GX_OK;
}

int plan_for(const sdm_pa2_args_t* a, int num_cus, int lds_limit, sdm_pa2_plan_t* out) {
    if (!out) return SDM_GX_ERR_ARG;
    if (num_cus < 1) num_cus = 256;
    const int64_t n = a->C * a->W, nsl = slices(a->hd);
    sdm_pa2_plan_t p{};
    p.slices_per_wave = nsl >= 2 && a->C <= 128 ? 2 : 1;
    const int64_t npair = p.slices_per_wave == 2 ? cdiv(nsl, 2) : nsl;
    const int64_t want = cdiv(static_cast<int64_t>(kTargetWavesPerCu) * num_cus, a->P * npair);   // tiles a chunk
    int64_t L = cdiv(n, want);
    if (L < kMinTile) L = kMinTile;
    if (L > n) L = n;
    p.tile_len = static_cast<int32_t>(L);
    const int64_t tiles = cdiv(n, L);
    p.waves_per_wg = tiles >= 16 ? 16 : tiles >= 8 ? 8 : 4;
    int st = complete(a, lds_limit, &p);
    if (st == SDM_GX_ERR_LIMIT && p.slices_per_wave == 2) {       // token rows of two slices too large: one slice
        p.slices_per_wave = 1;
        st = complete(a, lds_limit, &p);
    }
    if (st) return st;
    *out = p;
    return SDM_GX_OK;
}

struct Dev {
    bool known = false, gfx950 = false;
    int num_cus = 0, lds_per_wg = 0;
};
std::mutex g_mu;
std::vector<Dev> g_devs;
struct LdsAllowed {
    const void* fn;
    int bytes;
};
std::vector<LdsAllowed> g_lds_set;   // dynamic LDS bytes allowed per kernel in this process

int device(int* dev, Dev* d) {
    hipError_t e = hipGetDevice(dev);
    if (e != hipSuccess) return sdm_gx::record_hip_error(e);
    std::lock_guard<std::mutex> lk(g_mu);
    if (*dev >= static_cast<int>(g_devs.size())) g_devs.resize(*dev + 1);
    Dev& c = g_devs[*dev];
    if (!c.known) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, *dev);
        if (e != hipSuccess) return sdm_gx::record_hip_error(e);
        c.known = true;
        c.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        c.num_cus = prop.multiProcessorCount;
        c.lds_per_wg = static_cast<int>(prop.maxSharedMemoryPerMultiProcessor > 0
                                             ? prop.maxSharedMemoryPerMultiProcessor
                                             : prop.sharedMemPerBlock);
    }
    *d = c;
    return d->gfx950 ? SDM_GX_OK : SDM_GX_ERR_DEVICE;
}

int on_device(const void* p, int dev) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();
        return SDM_GX_ERR_DEVICE;
    }
    if ((at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeManaged) || at.device != dev)
        return SDM_GX_ERR_DEVICE;
    return SDM_GX_OK;
}

int pointers_on(const sdm_pa2_args_t* a, int dev) {
    const void* ps[] = {a->grad, a->bank, a->snap, a->d_u, a->beta, a->kpay, a->rec, a->out_eff, a->out_g};
    for (const void* p : ps)
        if (int st = on_device(p, dev)) return st;
    if (a->bpre)
        if (int st = on_device(a->bpre, dev)) return st;
    return SDM_GX_OK;
}

// The page's set_smem: allow the kernel its dynamic LDS (once per kernel and size).
int allow_lds(const void* fn, int bytes) {
    std::lock_guard<std::mutex> lk(g_mu);
    for (const LdsAllowed& e : g_lds_set)
        if (e.fn == fn && e.bytes >= bytes) return SDM_GX_OK;
    const hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (err != hipSuccess) return sdm_gx::record_hip_error(err);
    g_lds_set.push_back(LdsAllowed{fn, bytes});
    return SDM_GX_OK;
}

int launch(const sdm_pa2_args_t* a, int64_t ti, const sdm_pa2_plan_t& p, hipStream_t stream) {
    if (p.grid == 0) return SDM_GX_OK;
    const bool staged = stage_outputs(a, p);
    const void* fn = sdm_gx::find_pa2_kernel(p.slices_per_wave, p.waves_per_wg, staged);
    if (!fn) return SDM_GX_ERR_PLAN;
    if (int st = allow_lds(fn, p.lds_bytes)) return st;
    sdm_gx::Pa2Args k{};
    k.grad = a->grad;
    k.bank = a->bank;
    k.snap = a->snap;
    k.du = a->d_u;
    k.beta = a->beta;
    k.kpay = a->kpay;
    k.rec = a->rec;
    k.bpre = a->bpre;
    k.out_eff = a->out_eff;
    k.out_g = a->out_g;
    k.slots = a->slots;
    k.snap_rows = a->snap_rows;
    k.ssr = a->ssr;
    k.ld_u = a->ld_u;
    k.plane = a->plane;
    k.ti = static_cast<int32_t>(ti);
    k.P = static_cast<int32_t>(a->P);
    k.C = static_cast<int32_t>(a->C);
    k.W = static_cast<int32_t>(a->W);
    k.n = static_cast<int32_t>(a->C * a->W);
    k.hd = static_cast<int32_t>(a->hd);
    k.nsl = static_cast<int32_t>(slices(a->hd));
    k.slw = static_cast<int32_t>(slice_width(a->hd));
    k.npair = p.npair;
    k.ctas = p.ctas;
    k.L = p.tile_len;
    k.stage_out = staged ? 1 : 0;
    void* args[] = {&k};
    const hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(p.grid)), dim3(64u * p.waves_per_wg), args,
                                         static_cast<unsigned>(p.lds_bytes), stream);
    return e == hipSuccess ? SDM_GX_OK : sdm_gx::record_hip_error(e);
}

int resolve(const sdm_pa2_args_t* a, const sdm_pa2_plan_t* given, const Dev& d, sdm_pa2_plan_t* out) {
    if (given) {
        *out = *given;
        return complete(a, d.lds_per_wg, out);
    }
    return plan_for(a, d.num_cus, d.lds_per_wg, out);
}

}  // namespace

extern "C" {

int sdm_pa2_check(const sdm_pa2_args_t* args, int64_t ti) { return check(args, ti); }

int sdm_pa2_plan_for(const sdm_pa2_args_t* args, int32_t num_cus, int32_t lds_limit, sdm_pa2_plan_t* out) {
    if (!args || !out) return SDM_GX_ERR_ARG;
    if (args->C < 1 || args->C > 256 || args->W < 1 || args->W > 256 || args->hd < 1 || args->hd >= SDM_GX_HD_LIMIT ||
        args->P < 1)
        return SDM_GX_ERR_SHAPE;
    return plan_for(args, num_cus, lds_limit, out);
}

int sdm_pa2_step(const sdm_pa2_args_t* args, int64_t ti, const sdm_pa2_plan_t* plan, void* stream) {
    int st = check(args, ti);
    if (st) return st;
    int dev = 0;
    Dev d;
    if ((st = device(&dev, &d))) return st;
    if ((st = pointers_on(args, dev))) return st;
    sdm_pa2_plan_t p;
    if ((st = resolve(args, plan, d, &p))) return st;
    return launch(args, ti, p, static_cast<hipStream_t>(stream));
}

int sdm_pa2_steps(const sdm_pa2_args_t* args, int64_t ti_begin, int64_t ti_end, int32_t mode,
                  const sdm_pa2_plan_t* plan, void* stream) {
    if (mode != SDM_GX_STEPS_FORWARD && mode != SDM_GX_STEPS_REVERSE) return SDM_GX_ERR_ARG;
    if (ti_begin < 0 || ti_end < ti_begin) return SDM_GX_ERR_STEP;
    int st = check(args, ti_end > ti_begin ? ti_end - 1 : ti_begin);
    if (st) return st;
    if (ti_end == ti_begin) return SDM_GX_OK;
    int dev = 0;
    Dev d;
    if ((st = device(&dev, &d))) return st;
    if ((st = pointers_on(args, dev))) return st;
    sdm_pa2_plan_t p;
    if ((st = resolve(args, plan, d, &p))) return st;
    for (int64_t k = 0; k < ti_end - ti_begin; ++k) {
        const int64_t ti = mode == SDM_GX_STEPS_FORWARD ? ti_begin + k : ti_end - 1 - k;
        if ((st = launch(args, ti, p, static_cast<hipStream_t>(stream)))) return st;
    }
    return SDM_GX_OK;
}

}  // extern "C"
