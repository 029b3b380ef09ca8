/*
 * sdm_gx_pa2 -- Phase A of the deterministic backward step on MI355X (gfx950), C ABI: the consumer of the updated
 * d_u. Part of libsdm_gx_gemm; status codes are sdm_gx_status (sdm_gx_gemm.h).
 *
 * The operation (page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_pa2_cuda.py", gx_pa2_kernel, for
 * float32 grad, bank and snapshot rows): step ti covers chunks k = ti*P + p (0 <= p < P). A chunk has n = C*W records,
 * each four int32 {payload, slot, sck bits, cpe bits}; payload bit 31 FIRST (a group's first record), bit 30 LAST
 * (its last), bit 17 INVALID, bits 18-29 the distance back to the group's FIRST (4095: that far or farther), bits 9-16
 * the token t, bits 0-7 the write w. The head's hd columns form nsl = 1 + (hd-1)/128 slices of
 * slw = 4*ceil(ceil(hd/4)/nsl) columns; a slice is 32 lanes of 4 columns, columns past the slice or hd read as +0.
 * For each chunk and slice the records are walked in order:
 *   FIRST:          acc = +0; valid: gdw = grad row `slot`, sn = the group's snapshot row; invalid: both +0;
 *                   per lane gp = fmaf(gdw3, sn3, fmaf(gdw2, sn2, fmaf(gdw1, sn1, gdw0 * sn0))), g = tree(gp)
 *   every record:   acc = fmaf(sck, x, acc) per column (x: row t of chunk k of d_u);
 *                   dot = tree(fmaf(x3, sn3, fmaf(x2, sn2, fmaf(x1, sn1, x0 * sn0)))) over the lanes
 *   valid LAST:     grad row `slot` = fmaf(gdw, cpe, acc), bank row `slot` = sn (the slice's columns < hd)
 *   output o = k*n + t*W + w: one slice: out_eff[o] = -beta[k*C + t] * dot, out_g[o] = cpe * g;
 *                             nsl slices: out_eff[s*plane + o] = dot, out_g[s*plane + o] = g of slice s;
 *                             +0 for INVALID records
 * tree: the balanced pairwise sum over the 32 lanes in lane order (the page's xor butterfly). Every multiply, fma
 * and add rounds to nearest even with subnormals kept. Snapshot rows: ssr < 0, dense rows: k*n + the number of valid
 * FIRST records before the group's FIRST in chunk k (bpre gives those counts at 32-record block starts: bpre[k][b] =
 * valid FIRST records among 0 .. 32b-1); ssr >= 0, per-entry rows: ti*ssr + p*C*W + t*W + w of the FIRST record.
 *
 * Contract on the records (device data the library does not read on the host): each chunk's n records name every
 * (t < C, w < W) pair once; kpay[k][j] equals record j's payload and bpre the counts above; a group's FIRST and LAST
 * name the same slot and no two groups of one step read or write the same grad or bank row (steps are sequential:
 * a step may read rows an earlier step wrote). Records outside the contract give unspecified values in the rows they
 * name and in their chunk's outputs, never an access outside the buffers: the kernel checks every token, write, slot
 * and snapshot row before the access it steers.
 *
 * Memory (caller-owned device memory of the current device; float32 unless marked):
 *   grad, bank   [slots][hd]                 read (grad, at FIRST) and written (both, at LAST) in place
 *   snap         [snap_rows][hd]
 *   d_u          [N*C] rows of ld_u           token rows, columns < hd read (d_u as the update leaves it)
 *   beta         [N*C]
 *   kpay         int32 [N][n]                 rec int32 [N][n][4] (16-byte aligned)
 *   bpre         int32 [N][ceil(n/32) + 1]    (dense rows only; may be NULL when ssr >= 0)
 *   out_eff, out_g  planes x plane floats     (planes = 1 when nsl == 1, else nsl; plane >= N*n)
 * Written arrays must not overlap each other or any read array. Execution is asynchronous on `stream`.
 */
#ifndef SDM_GX_PA2_H
#define SDM_GX_PA2_H

#include <stdint.h>

#include "sdm_gx_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sdm_pa2_args {
    float* grad;
    float* bank;
    int64_t slots;
    const float* snap;
    int64_t snap_rows;
    int64_t ssr;            /* < 0: dense snapshot rows; >= 0: per-entry rows, step stride */
    const float* d_u;
    int64_t ld_u;
    const float* beta;
    const int32_t* kpay;
    const int32_t* rec;
    const int32_t* bpre;
    float* out_eff;
    float* out_g;
    int64_t plane;
    int64_t planes;
    int64_t N, P, C, W, hd;
} sdm_pa2_args_t;

/* How a step is launched (never changes results): slices_per_wave 2 puts two slices in one wavefront (lanes 0-31 and
 * 32-63; the planner's choice when nsl >= 2 and C <= 128), 1 one slice; waves_per_wg 4, 8 or 16 wavefronts per
 * workgroup, which stages a chunk's token rows once; tile_len records per wavefront tile (tiles move back to group
 * starts). Outputs: ctas, npair (slice groups), grid, lds_bytes, stage_out. When one workgroup covers a chunk (ctas
 * == 1) and the chunk's outputs add at most a quarter to its LDS, it gathers them in LDS and writes each output plane
 * of the chunk in one contiguous run (stage_out 1, the kernel gx_pa2_staged_kernel); lds_bytes then includes them. */
typedef struct sdm_pa2_plan {
    int32_t slices_per_wave;
    int32_t waves_per_wg;
    int32_t tile_len;
    int32_t ctas;
    int32_t npair;
    int32_t lds_bytes;
    int32_t stage_out;
    int64_t grid;
} sdm_pa2_plan_t;

/* Argument checks for step ti (shapes, step range, strides, alignment, overlap, row counts), no device call.
 * The page's host entry gx_pa2 checks the same properties of its tensors. */
SDM_GX_API int sdm_pa2_check(const sdm_pa2_args_t* args, int64_t ti);

/* The planner (no device call): num_cus compute units, lds_limit LDS bytes per workgroup. The page's plan() and
 * tile_len(), re-derived for MI355X: wavefronts enough for 8 per SIMD where the step has records for them. */
SDM_GX_API int sdm_pa2_plan_for(const sdm_pa2_args_t* args, int32_t num_cus, int32_t lds_limit, sdm_pa2_plan_t* out);

/* Step ti (plan NULL: the planner's for the current device). */
SDM_GX_API int sdm_pa2_step(const sdm_pa2_args_t* args, int64_t ti, const sdm_pa2_plan_t* plan, void* stream);

/* Steps ti_begin .. ti_end - 1, one launch each, in order (SDM_GX_STEPS_FORWARD) or descending
 * (SDM_GX_STEPS_REVERSE, the backward's order); there is no fused mode: a step may read grad rows an earlier step
 * wrote. Validated once. */
SDM_GX_API int sdm_pa2_steps(const sdm_pa2_args_t* args, int64_t ti_begin, int64_t ti_end, int32_t mode,
                             const sdm_pa2_plan_t* plan, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SDM_GX_PA2_H */
