/*
 * sdm_gx_gemm -- deterministic FP32 per-step d_u update for MI355X (gfx950), C ABI.
 *
 * The operation (page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_gemm_cuda.py", module docstring;
 * gx_gemm_kernel's j-chain and epilogue on the same page):
 *
 *   for every chunk n = ti*P + p (0 <= p < P) of step ti, row i < C and column c < hd:
 *       acc = +0
 *       for j = 0, 1, ..., C-1 in this order:   acc = fmaf(x[n, j, i], d_dv[n, j, c], acc)
 *       d_u[n, i, c] = d_u[n, i, c] + acc        (one separately rounded IEEE binary32 add, in place)
 *
 * Every fused multiply-add and the final add round to nearest even and keep subnormals. Each output element is
 * computed by exactly that chain, either by one GPU lane on the vector ALUs (engine SDM_GX_ENGINE_VALU) or on the
 * FP32 matrix cores as one K=1 MFMA per chain step (engine SDM_GX_ENGINE_MFMA: d = c + a*b, a single rounding, no
 * reduction inside the instruction). Results are bit-identical for every engine, launch plan, step order and run,
 * and equal to the CPU definition wherever the result is not NaN (NaN results are NaN on both sides; their payload
 * is not specified).
 *
 * Memory layout (FP32, row-major; element offsets):
 *   x     [N][C][C]               x[n, j, i]    at (n*C + j)*C + i        (contiguous; used transposed)
 *   d_dv  [N][C] rows of ld_dv    d_dv[n, j, c] at (n*C + j)*ld_dv + c    (c < hd <= ld_dv)
 *   d_u   [N][C] rows of ld_u     d_u[n, i, c]  at (n*C + i)*ld_u + c     (c < hd <= ld_u), updated in place
 * Writes: only d_u[n, i, c] with c < hd, for the chunks n of the requested steps; padding columns hd..ld_u-1 and
 * every other chunk keep their bytes.
 * Reads: d_u only where it is written. x and d_dv only inside the chunks of the requested steps, where the
 * matrix-core engine's direct-to-LDS kernel moves whole 16-byte groups: it may read any element of such a chunk of
 * x, and the elements of such a chunk of d_dv from its first row start through element (C-1)*ld_dv + hd - 1 (so the
 * padding columns of every row but the chunk's last); when x or d_dv starts off a 16-byte boundary it may also read
 * the bytes from the 16-byte boundary at or below each row start (the same 16-byte block, hence the same page, as the
 * row's first element; for the first row of chunk 0 that is up to 12 bytes below the pointer passed in). No value
 * read outside columns c < hd reaches a result. The other kernels read only columns c < hd. Chunks
 * n >= (N / P) * P belong to no step and are never touched.
 *
 * Ownership and execution: every pointer is caller-owned device memory of the current HIP device (for example a
 * torch tensor's data_ptr()). The library allocates nothing on the caller's behalf, keeps no pointer after a call
 * returns (except inside a caller-owned sdm_gx_launch_t), and runs its kernels asynchronously on the caller's
 * stream (`stream` is a hipStream_t; NULL means the null stream). Calls on the same stream run in order. d_u must
 * not overlap x or d_dv.
 *
 * Errors: every entry point returns an int status (sdm_gx_status); no exception crosses the ABI. Argument checks
 * run on the host before anything is launched; on an error nothing is launched and no memory is touched.
 * SDM_GX_ERR_HIP carries the HIP runtime error of the failing call in sdm_gx_last_hip_error() (per host thread).
 * All entry points are thread-safe.
 */
#ifndef SDM_GX_GEMM_H
#define SDM_GX_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDM_GX_ABI_VERSION 4

#if defined(__GNUC__)
#define SDM_GX_API __attribute__((visibility("default")))
#else
#define SDM_GX_API
#endif

/* Shape limits (the page's host entry gx_gemm and its supported(): 1 <= C <= 256, 1 <= hd < 2^20,
 * 1 <= P <= N < 2^31). */
#define SDM_GX_MAX_C 256
#define SDM_GX_HD_LIMIT (1 << 20)          /* hd < SDM_GX_HD_LIMIT */
#define SDM_GX_N_LIMIT (INT64_C(1) << 31)  /* N < SDM_GX_N_LIMIT */
#define SDM_GX_LD_LIMIT (INT64_C(1) << 31) /* ld_u, ld_dv < SDM_GX_LD_LIMIT */

typedef enum sdm_gx_status {
    SDM_GX_OK = 0,             /* done (also: nothing to do) */
    SDM_GX_ERR_NULL = -1,      /* a required pointer is NULL */
    SDM_GX_ERR_SHAPE = -2,     /* C not in [1, 256], hd not in [1, 2^20), P < 1, N not in [1, 2^31) */
    SDM_GX_ERR_STEP = -3,      /* ti < 0, ti >= N / P, P > N, or an empty / out-of-range step range */
    SDM_GX_ERR_ALIGN = -4,     /* a pointer is not 4-byte aligned */
    SDM_GX_ERR_OVERLAP = -5,   /* d_u overlaps x or d_dv */
    SDM_GX_ERR_STRIDE = -6,    /* ld_u or ld_dv < hd, or >= 2^31 */
    SDM_GX_ERR_LIMIT = -7,     /* the launch exceeds a device or engine limit (LDS per workgroup; for the MFMA
                                  engine C * ld_u * 4 must stay below 2^31 bytes) */
    SDM_GX_ERR_HIP = -8,       /* a HIP runtime call failed: see sdm_gx_last_hip_error() */
    SDM_GX_ERR_PLAN = -9,      /* a plan / prepared launch is malformed or does not fit this shape */
    SDM_GX_ERR_DEVICE = -10,   /* no usable gfx950 device, pointers not on the current device, or a prepared
                                  launch used on another device */
    SDM_GX_ERR_ARG = -11       /* any other invalid argument (unknown mode, NULL output struct, ...) */
} sdm_gx_status;

/* Engines (sdm_gx_plan_t.engine). */
#define SDM_GX_ENGINE_VALU 0   /* one lane per output element, v_fma_f32 chains on the vector ALUs */
#define SDM_GX_ENGINE_MFMA 1   /* the same chains on the FP32 matrix cores, one K=1 MFMA per chain step */

/* A launch plan: which engine runs the update and how output tiles map onto wavefronts and workgroups. Results
 * never depend on it.
 *   engine         SDM_GX_ENGINE_VALU or SDM_GX_ENGINE_MFMA
 * SDM_GX_ENGINE_VALU (the other engine ignores these fields, except slab_rows):
 *   rows_per_wave  RI: output rows one wavefront owns (1, 2, 4, 8 or 16; RI <= C)
 *   cols_per_lane  RC: adjacent output columns one lane owns (1, 2 or 4); a wavefront covers 64*RC columns
 *   waves_per_wg   wavefronts per workgroup (1, 2, 4, 8, or 16 for some tiles); they take consecutive row blocks of
 *                  one chunk and column block
 *   staging        0: each wavefront reads its d_dv columns straight from global memory;
 *                  1: the workgroup stages its d_dv column block in LDS once and every wavefront reads it there
 *   xcd_remap      1: workgroup ids are permuted so that the workgroups of one chunk run on one XCD (one L2)
 *   slab_rows      staging 1: d_dv rows per LDS slab (0: the planner's choice; clamped to C). The MFMA engine reads
 *                  it too: chain rows per LDS stage, 16 (0 means 16) or 32 (direct-to-LDS 16-column tiles with
 *                  3 stages and 1 loader wavefront)
 * SDM_GX_ENGINE_MFMA (persistent workgroups walking (chunk, row group, column group) work items; the other engine
 * ignores these fields):
 *   mf_row_waves     compute wavefronts along the rows of a work item, 64 rows each (1 or 2)
 *   mf_col_waves     compute wavefronts along its columns, mf_block columns each (1, 2, 4, or 8 with mf_row_waves 1)
 *   mf_stages        LDS ring stages of slab_rows chain rows of x and d_dv (4 with register slabs; with
 *                    mf_reg_slabs 0: 4 or 8 for mf_block 32, 3 or 8 for mf_block 16)
 *   mf_reg_slabs     slabs of 16 chain rows the loader wavefronts keep in flight in registers (2 or 4), or 0: the
 *                    loader wavefronts move slabs straight from memory into the LDS ring (buffer loads to LDS), up
 *                    to mf_stages - 1 slabs in flight. That needs C and ld_dv multiples of 4 and
 *                    (C + 32) * ld_dv * 4 < 2^31; rows off a 16-byte boundary run an unaligned-row instance
 *                    (mf_aln). Completing a plan for a layout that rules it out gives the register-ring plan of the
 *                    same work items (32-column wavefronts, 2 register slabs, 4 stages, 4 loader wavefronts), with
 *                    the same results
 *   mf_loader_waves  loader wavefronts per workgroup (2 or 4 with register slabs, 4 with 4 register slabs for 64x256
 *                    and 128x128 items; with mf_reg_slabs 0: 1 with 4 stages, 2 with 8 stages)
 *   mf_workgroups    workgroups to launch (0: one per compute unit); each takes a contiguous range of work items
 *   mf_du_at_end     0: d_u prefetched when a work item starts; 1: read at its end (fewer registers: two workgroups
 *                    fit one compute unit; instances for 128x128 and 64x128 items with 2 register slabs and 4
 *                    loader wavefronts, and for 128x128 items with mf_reg_slabs 0, mf_block 32, 4 stages,
 *                    1 loader wavefront)
 *   mf_block         the MFMA that runs the chain, by output columns per compute wavefront (0 means 32):
 *                    32: v_mfma_f32_32x32x1_2b_f32, a 64x32 tile per wavefront, 64 cycles per chain step;
 *                    16: v_mfma_f32_16x16x1_4b_f32, a 64x16 tile, 32 cycles per step (half the chain latency of a
 *                    work item, twice the wavefronts; mf_reg_slabs 0 only, tiles 64x32 .. 128x64 of mf_col_waves 2,
 *                    4 or 8). Both are exact fma steps; the results do not depend on the choice. Where the layout
 *                    rules out direct-to-LDS slabs, a mf_block 16 plan runs as mf_block 32 with half the column
 *                    wavefronts (mf_col_waves 2 -> 1 ..), register slabs as above
 *   mf_stream_du     mf_reg_slabs 0: 1 = d_u stores carry the non-temporal (streaming) cache hint; 0 = plain stores.
 *                    No effect on results.
 * Outputs of the planner / sdm_gx_plan_complete (also filled in the plans of a prepared launch, for the layout of
 * its pointers and strides; input values are ignored):
 *   lds_bytes      LDS bytes per workgroup (dynamic for the VALU engine, static for the MFMA engine)
 *   wgs_per_cu     workgroups per CU that can be resident (0 if not known)
 *   mf_aln         which instance a direct-to-LDS plan (mf_reg_slabs 0) runs for rows that start off a 16-byte
 *                  boundary: 0 rows on 16-byte boundaries; 4 d_dv rows moved by 4-byte DMA (x aligned); 2 d_dv rows
 *                  loaded from the 16-byte boundary below each row start (x aligned); 3 x and d_dv rows both so.
 *                  A direct-to-LDS plan whose layout has no such instance (or whose strides rule out direct-to-LDS
 *                  slabs) is completed as the register-ring plan that runs the same work items, as described under
 *                  mf_reg_slabs; the plan reported is the kernel that runs
 *   grid           workgroups for the chunk count it was planned for */
typedef struct sdm_gx_plan {
    int32_t engine;
    int32_t rows_per_wave;
    int32_t cols_per_lane;
    int32_t waves_per_wg;
    int32_t staging;
    int32_t xcd_remap;
    int32_t slab_rows;
    int32_t mf_row_waves;
    int32_t mf_col_waves;
    int32_t mf_stages;
    int32_t mf_reg_slabs;
    int32_t mf_loader_waves;
    int32_t mf_workgroups;
    int32_t lds_bytes;
    int32_t wgs_per_cu;
    int32_t mf_du_at_end;
    int32_t mf_block;
    int32_t mf_stream_du;
    int32_t mf_aln;
    int64_t grid;
} sdm_gx_plan_t;

/* One step ti of the update with contiguous rows (ld_u = ld_dv = hd), planned automatically. There is no N: the
 * caller vouches that chunks 0 .. (ti+1)*P - 1 exist in all three arrays, and the checks of sdm_gx_gemm_ex run with
 * N = (ti+1)*P (so P >= 1, ti >= 0, (ti+1)*P < 2^31, and no overlap among those chunks).
 * Same operation as the page's host entry gx_gemm (its plain, non-PDL launch). */
SDM_GX_API int sdm_gx_gemm(float* d_u, const float* x, const float* d_dv, int64_t ti, int64_t P, int64_t C,
                           int64_t hd, void* stream);

/* One step ti with row strides and the full chunk count N (checks 0 <= ti < N / P and whole-array overlap, as the
 * page's gx_gemm does). plan == NULL: the planner chooses; otherwise the given plan is validated and used. */
SDM_GX_API int sdm_gx_gemm_ex(float* d_u, int64_t ld_u, const float* x, const float* d_dv, int64_t ld_dv,
                              int64_t N, int64_t ti, int64_t P, int64_t C, int64_t hd, const sdm_gx_plan_t* plan,
                              void* stream);

/* Multi-step driver (the page's per-backward plan gx_gemm_plan / gx_gemm_plan_launch and make_step's step loop):
 * validates once for steps ti_begin .. ti_end - 1, then
 *   SDM_GX_STEPS_FORWARD  one launch per step, ti ascending
 *   SDM_GX_STEPS_REVERSE  one launch per step, ti descending (the backward's order)
 *   SDM_GX_STEPS_FUSED    one launch covering every chunk of those steps
 * All three give identical bits: steps update disjoint chunks and each element is still one fixed chain.
 * ti_begin == ti_end is a no-op. */
#define SDM_GX_STEPS_FORWARD 0
#define SDM_GX_STEPS_REVERSE 1
#define SDM_GX_STEPS_FUSED 2
SDM_GX_API int sdm_gx_gemm_steps(float* d_u, int64_t ld_u, const float* x, const float* d_dv, int64_t ld_dv,
                                 int64_t N, int64_t P, int64_t C, int64_t hd, int64_t ti_begin, int64_t ti_end,
                                 int32_t mode, const sdm_gx_plan_t* plan, void* stream);

/* Argument checks of sdm_gx_gemm_ex without touching any device (no HIP call): the status the launch would return
 * before reaching the GPU, except for device-membership checks. Mirrors the page's gx_gemm checks. */
SDM_GX_API int sdm_gx_check(const float* d_u, int64_t ld_u, const float* x, const float* d_dv, int64_t ld_dv,
                            int64_t N, int64_t ti, int64_t P, int64_t C, int64_t hd);

/* The launch planner: the plan a launch over `nchunks` chunks of shape (C, hd) runs, on HIP device `device` (-1: the
 * current device). It takes the part of the page's launch rules for gx_gemm (_rows: rows per CTA from a grid target;
 * _cap: CTAs per SM, forced by padding shared memory; one_wave: the kernel only when its grid fits one wave),
 * re-derived for MI355X: engine, work-item tile, LDS stages and workgroups per CU, for single- and multi-wave grids
 * alike. The result never changes the output bits.
 *   ld_u, ld_dv        the row strides the launch will use (hd <= ld < 2^31; else SDM_GX_ERR_STRIDE)
 *   x_mod16, dv_mod16  the byte offsets of x and d_dv from a 16-byte boundary (address mod 16: 0, 4, 8 or 12; else
 *                      SDM_GX_ERR_ALIGN); with the strides they decide which kernel instance runs (mf_aln)
 *   engine             -1: the planner's choice; SDM_GX_ENGINE_VALU or SDM_GX_ENGINE_MFMA: that engine
 *                      (SDM_GX_ERR_LIMIT when the matrix-core engine cannot take the strides)
 * The plan filled in is exactly what sdm_gx_gemm_ex / sdm_gx_gemm_steps / sdm_gx_prepare run for those arguments
 * when given no plan (engine -1). */
SDM_GX_API int sdm_gx_plan(int64_t nchunks, int64_t C, int64_t hd, int64_t ld_u, int64_t ld_dv, int32_t x_mod16,
                           int32_t dv_mod16, int32_t engine, int32_t device, sdm_gx_plan_t* out);

/* The same planner with the device facts given explicitly (no HIP call): compute units and LDS bytes per
 * workgroup. */
SDM_GX_API int sdm_gx_plan_for(int64_t nchunks, int64_t C, int64_t hd, int64_t ld_u, int64_t ld_dv,
                               int32_t x_mod16, int32_t dv_mod16, int32_t engine, int32_t num_cus,
                               int32_t lds_per_cu, sdm_gx_plan_t* out);

/* Validate a caller-made plan for shape (C, hd), strides and placement as for sdm_gx_plan, and fill its output
 * fields for `nchunks` chunks (the page's gx_gemm checks its ti_rows argument the same way: a plan that does not fit
 * is an error, never silently replaced). */
SDM_GX_API int sdm_gx_plan_complete(sdm_gx_plan_t* plan, int64_t nchunks, int64_t C, int64_t hd, int64_t ld_u,
                                    int64_t ld_dv, int32_t x_mod16, int32_t dv_mod16, int32_t lds_per_cu);

/* A prepared step launch (the page's GemmPlan): everything is validated once for every ti <= ti_max, then
 * sdm_gx_launch issues step ti with only ti changed. The struct is caller-owned plain data; it holds the three
 * device pointers, so it is valid while those buffers are. */
typedef struct sdm_gx_launch {
    uint64_t magic;
    int32_t device;
    int32_t reserved0;
    float* d_u;
    const float* x;
    const float* d_dv;
    int64_t ld_u, ld_dv, N, P, C, hd, ti_max;
    sdm_gx_plan_t plan_step;   /* used by sdm_gx_launch (P chunks) */
    sdm_gx_plan_t plan_fused;  /* used by sdm_gx_launch_fused (planned for (ti_max+1)*P chunks) */
} sdm_gx_launch_t;

/* plan == NULL: the planner chooses both plans; otherwise the given plan is validated and used for both. */
SDM_GX_API int sdm_gx_prepare(sdm_gx_launch_t* out, float* d_u, int64_t ld_u, const float* x, const float* d_dv,
                              int64_t ld_dv, int64_t N, int64_t P, int64_t C, int64_t hd, int64_t ti_max,
                              const sdm_gx_plan_t* plan);
/* Issue step ti (0 <= ti <= ti_max) of a prepared launch on `stream`; the current device must be the prepared one. */
SDM_GX_API int sdm_gx_launch(const sdm_gx_launch_t* prepared, int64_t ti, void* stream);
/* Issue steps ti_begin .. ti_end - 1 of a prepared launch as ONE launch (every ti <= ti_max). */
SDM_GX_API int sdm_gx_launch_fused(const sdm_gx_launch_t* prepared, int64_t ti_begin, int64_t ti_end, void* stream);

/* A HIP graph of a prepared step range (the page's plan replay: the whole multi-step sequence captured once, then
 * issued with one call). Kernel nodes are added explicitly, in issue order, each depending on the previous one:
 *   SDM_GX_STEPS_FORWARD / SDM_GX_STEPS_REVERSE  one node per step launch (plan_step), ti ascending / descending
 *   SDM_GX_STEPS_FUSED                           the fused launch of the range (plan_fused)
 * The graph holds no memory of its own beyond the runtime's graph objects; it refers to the prepared launch's three
 * buffers, which must outlive it. Replays are in-place updates like any launch (each replay adds the update again).
 * ti_begin == ti_end gives an empty graph; launching it does nothing. The caller owns the graph and releases it with
 * sdm_gx_graph_destroy (NULL is accepted). */
typedef struct sdm_gx_graph sdm_gx_graph_t;
SDM_GX_API int sdm_gx_graph_create(sdm_gx_graph_t** out, const sdm_gx_launch_t* prepared, int64_t ti_begin,
                                   int64_t ti_end, int32_t mode);
/* Replay the graph on `stream` (the current device must be the prepared one). */
SDM_GX_API int sdm_gx_graph_launch(const sdm_gx_graph_t* graph, void* stream);
/* Kernel nodes in the graph; -1 for an invalid handle. */
SDM_GX_API int64_t sdm_gx_graph_nodes(const sdm_gx_graph_t* graph);
SDM_GX_API int sdm_gx_graph_destroy(sdm_gx_graph_t* graph);

/* Resource usage of the kernel instance a plan selects (the page's gx_gemm_attrs): out[0] VGPRs per lane,
 * out[1] private (scratch) bytes per lane, out[2] static LDS bytes, out[3] max threads per workgroup,
 * out[4] the plan's dynamic LDS bytes. Needs a device. */
SDM_GX_API int sdm_gx_kernel_attrs(const sdm_gx_plan_t* plan, int64_t out[5]);

/* Text for a status code (static storage). */
SDM_GX_API const char* sdm_gx_strerror(int code);
/* The HIP error (hipError_t value) behind the last SDM_GX_ERR_HIP on this host thread; 0 if none. */
SDM_GX_API int sdm_gx_last_hip_error(void);
/* SDM_GX_ABI_VERSION of the loaded library. */
SDM_GX_API int sdm_gx_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDM_GX_GEMM_H */
