// gfx950 kernels of the deterministic FP32 per-step d_u update.
//
// Operation (page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_gemm_cuda.py", module docstring and
// gx_gemm_kernel): for chunk n, row i < C and column c < hd,
//     acc = +0;  acc = fma(x[n, j, i], d_dv[n, j, c], acc) for j = 0..C-1 in order;  d_u[n, i, c] += acc
// with one separately rounded add. One lane owns each output element and runs exactly that chain on the VALU
// (v_fma_f32 / v_fmac_f32, round to nearest even, f32 denormals kept by the kernel descriptor's default mode).
// MFMA is not used: its internal accumulation order is not this chain.
//
// Mapping onto CDNA4 (wave64):
//   * A wavefront owns RI consecutive output rows (i0 .. i0+RI-1) and 64*RC consecutive columns; lane l owns
//     columns c0 + l*RC .. c0 + l*RC + RC-1 of every one of those rows (RI*RC accumulators per lane).
//   * Row block and chunk are wave-uniform, so x[n, j, i0 .. i0+RI-1] -- the value every lane multiplies by in
//     step j -- is read with scalar loads into SGPRs through the constant address space and fed to the FMA as its
//     scalar operand. x therefore costs no LDS bandwidth and no VGPRs.
//   * d_dv[n, j, c..c+RC-1] differs per lane: STAGE 0 reads it straight from global memory (a wavefront row of
//     64*RC floats per j, coalesced, with 4-byte alignment allowed); STAGE 1 stages a slab of d_dv rows for the
//     workgroup's column block in LDS once and every wavefront of the workgroup reads it there.
//   * The last row block of a chunk whose C is not a multiple of RI is shifted back to end at row C. Its leading
//     rows are computed again (the same chain, so the same bits) but only stored by the wavefront that owns them.
//   * d_u is read once, after the chain, added to the accumulators and stored in place; columns >= hd are never
//     loaded or stored, so padding columns of a row stride ld > hd are never touched.
//   * Workgroups may be permuted so that all workgroups of one chunk land on one XCD (blocks are dispatched to the
//     8 XCDs round-robin), keeping the chunk's d_dv reuse inside one L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gx_gemm_kernel.h"


namespace sdm_gx {

typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x2u __attribute__((ext_vector_type(2), aligned(4)));
typedef float f32x4a __attribute__((ext_vector_type(4), aligned(16)));
typedef __attribute__((address_space(4))) const float* cf32p;   // x: read-only, wave-uniform: scalar loads

// RC adjacent floats of one row from global memory. FULL: all RC columns are < hd (one vector load, 4-byte aligned
// is enough); otherwise per column, zero past hd (the pointer is only dereferenced for columns < hd).
template <int RC, bool FULL>
__device__ __forceinline__ void load_cols(const float* row, int c, int hd, float (&d)[RC]) {
    if constexpr (FULL) {
        if constexpr (RC == 4) {
            const f32x4u v = *reinterpret_cast<const f32x4u*>(row + c);
            d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
        } else if constexpr (RC == 2) {
            const f32x2u v = *reinterpret_cast<const f32x2u*>(row + c);
            d[0] = v.x; d[1] = v.y;
        } else {
            d[0] = row[c];
        }
    } else {
#pragma unroll
        for (int q = 0; q < RC; ++q) d[q] = (c + q < hd) ? row[c + q] : 0.0f;
    }
}

// Rows of the chain per software-pipeline batch. Two batches are live at once (the one being consumed and the one in
// flight). Each batch costs one scalar-load round trip, so tiles with few rows per wavefront take long batches (up
// to 16 rows) and few round trips per chain. Limits, found by checking the build for spills: U*RI <= 32 scalar x
// values (16 for RI = 16), U*RC <= 16 d_dv values per lane, U <= 16.
template <int RI, int RC>
struct Batch {
    static constexpr int BY_SGPR = (RI >= 16 ? 16 : 32) / RI, BY_VGPR = 16 / RC;
    static constexpr int U0 = BY_SGPR < BY_VGPR ? BY_SGPR : BY_VGPR;
    static constexpr int U = U0 < 1 ? 1 : (U0 > 16 ? 16 : U0);
};

// Wait until every scalar (and LDS) load issued so far has landed: s_waitcnt lgkmcnt(0), vmcnt/expcnt untouched.
// Scalar loads return out of order, so this is the only way to wait for one batch; issuing the next batch only
// after this wait keeps exactly one batch of x loads in flight while the previous one is consumed.
__device__ __forceinline__ void wait_scalar_loads() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Loads through the constant address space count as invariant, so the compiler may hoist them anywhere. Routing the
// row index of the next batch through an empty volatile asm placed after the wait pins those loads behind it.
__device__ __forceinline__ int after_wait(int j) {
    asm volatile("" : "+s"(j));
    return j;
}

// x[n, j, i0 .. i0+RI-1] for U consecutive rows j (wave-uniform addresses: scalar loads into SGPRs).
template <int RI, int U>
__device__ __forceinline__ void load_x(float (&xv)[U][RI], cf32p xr, int C, int j) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < RI; ++r) xv[u][r] = xr[(j + u) * C + r];
}

// The step's scalar x values copied into VGPRs. gfx950 issues v_fmac_f32 at twice the rate when every operand is a
// VGPR but only at the base rate with an SGPR operand, so copying each x value once per step (v_mov_b64 moves an
// adjacent pair from an SGPR pair) pays for itself as soon as the value feeds two or more FMAs (RC >= 2). Measured on
// the RC = 2 pattern: 100 TFLOP/s with pair copies, 90 with single copies, 75 with the SGPR operand. The copies are
// grouped two pairs to a statement so that they land in distinct registers ahead of the FMAs that read them.
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <int RI>
__device__ __forceinline__ void to_vgprs(const float (&s)[RI], float (&v)[RI]) {
    if constexpr (RI % 4 == 0) {
#pragma unroll
        for (int r = 0; r < RI; r += 4) {
            f32x2 a, b;
            const f32x2 sa = {s[r], s[r + 1]}, sb = {s[r + 2], s[r + 3]};
            asm("v_mov_b64 %0, %2\n\tv_mov_b64 %1, %3" : "=&v"(a), "=&v"(b) : "s"(sa), "s"(sb));
            v[r] = a.x; v[r + 1] = a.y; v[r + 2] = b.x; v[r + 3] = b.y;
        }
    } else {
#pragma unroll
        for (int r = 0; r < RI; ++r) asm("v_mov_b32 %0, %1" : "=v"(v[r]) : "s"(s[r]));
    }
}

// One step j of the chain for the wavefront's RI rows: acc[r][q] = fma(x[n, j, i0+r], d[q], acc[r][q]).
template <int RI, int RC>
__device__ __forceinline__ void chain_step(float (&acc)[RI][RC], const float (&xv)[RI], const float (&d)[RC]) {
    if constexpr (RC >= 2) {
        float xg[RI];
        to_vgprs<RI>(xv, xg);
#pragma unroll
        for (int r = 0; r < RI; ++r)
#pragma unroll
            for (int q = 0; q < RC; ++q) acc[r][q] = __builtin_fmaf(xg[r], d[q], acc[r][q]);
    } else {
#pragma unroll
        for (int r = 0; r < RI; ++r)
#pragma unroll
            for (int q = 0; q < RC; ++q) acc[r][q] = __builtin_fmaf(xv[r], d[q], acc[r][q]);
    }
}

// d_dv rows straight from global memory: row j of the chunk at base + j*ld, this lane's columns c .. c+RC-1.
template <int RC, bool FULL>
struct GlobalRows {
    const float* base;
    int64_t ld;
    int c, hd;
    __device__ __forceinline__ void load(float (&d)[RC], int j) const {
        load_cols<RC, FULL>(base + static_cast<int64_t>(j) * ld, c, hd, d);
    }
};

// d_dv rows from an LDS slab: slab row jj at base + jj*CW (base already offset by this lane's columns).
template <int RC, int CW>
struct LdsRows {
    const float* base;
    int first;       // chain row of slab row 0
    __device__ __forceinline__ void load(float (&d)[RC], int j) const {
        const float* p = base + (j - first) * CW;
        if constexpr (RC == 4) {
            const f32x4a v = *reinterpret_cast<const f32x4a*>(p);
            d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
        } else if constexpr (RC == 2) {
            d[0] = p[0]; d[1] = p[1];
        } else {
            d[0] = p[0];
        }
    }
};

template <int RI, int RC, int U, class Src>
__device__ __forceinline__ void load_batch(float (&xv)[U][RI], float (&d)[U][RC], cf32p xr, int C, const Src& src,
                                           int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) src.load(d[u], j + u);
    load_x<RI, U>(xv, xr, C, j);
}

template <int RI, int RC, int U>
__device__ __forceinline__ void compute_batch(float (&acc)[RI][RC], const float (&xv)[U][RI],
                                              const float (&d)[U][RC]) {
#pragma unroll
    for (int u = 0; u < U; ++u) chain_step<RI, RC>(acc, xv[u], d[u]);
}

// The chain over rows j = j0 .. j1-1 in order. Batches of U rows are software-pipelined: batch b+1's x (scalar) and
// d_dv loads are issued before batch b is computed, in two register sets used alternately.
template <int RI, int RC, class Src>
__device__ __forceinline__ void chain_rows(float (&acc)[RI][RC], cf32p xr, int C, int j0, int j1, const Src& src) {
    constexpr int U = Batch<RI, RC>::U;
    const int nb = (j1 - j0) / U;
    float xa[U][RI], xb[U][RI];
    float da[U][RC], db[U][RC];
    int b = 0;
    if (nb > 0) load_batch<RI, RC, U>(xa, da, xr, C, src, j0);
    // sched_barrier(0) fences keep the order wait -> issue next batch -> compute current batch in the final code.
    for (; b + 2 < nb; b += 2) {                      // batches b, b+1 computed; b+1 and b+2 issued
        wait_scalar_loads();
        load_batch<RI, RC, U>(xb, db, xr, C, src, after_wait(j0 + (b + 1) * U));
        __builtin_amdgcn_sched_barrier(0);
        compute_batch<RI, RC, U>(acc, xa, da);
        __builtin_amdgcn_sched_barrier(0);
        wait_scalar_loads();
        load_batch<RI, RC, U>(xa, da, xr, C, src, after_wait(j0 + (b + 2) * U));
        __builtin_amdgcn_sched_barrier(0);
        compute_batch<RI, RC, U>(acc, xb, db);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (b + 2 == nb) {                                // the last two batches: one more to issue
        wait_scalar_loads();
        load_batch<RI, RC, U>(xb, db, xr, C, src, after_wait(j0 + (b + 1) * U));
        __builtin_amdgcn_sched_barrier(0);
        compute_batch<RI, RC, U>(acc, xa, da);
        __builtin_amdgcn_sched_barrier(0);
        wait_scalar_loads();
        compute_batch<RI, RC, U>(acc, xb, db);
    } else if (b + 1 == nb) {                         // the last batch, already issued
        wait_scalar_loads();
        compute_batch<RI, RC, U>(acc, xa, da);
    }
    for (int j = j0 + nb * U; j < j1; ++j) {      // the last (j1 - j0) % U rows
        float xv[1][RI], d[1][RC];
        load_batch<RI, RC, 1>(xv, d, xr, C, src, j);
        chain_step<RI, RC>(acc, xv[0], d[0]);
    }
}

// d_u[n, i0+r, c .. c+RC-1] for the rows this wavefront owns (i >= i_own), read after the chain (reading it earlier
// costs registers, and occupancy, for no measured gain); columns >= hd are neither read nor written.
template <int RI, int RC, bool FULL>
__device__ __forceinline__ void load_rows(float (&u)[RI][RC], const float* dun, int64_t ld, int i0, int i_own, int c,
                                          int hd) {
    const float* row = dun + static_cast<int64_t>(i0) * ld;
#pragma unroll
    for (int r = 0; r < RI; ++r, row += ld) {
#pragma unroll
        for (int q = 0; q < RC; ++q) u[r][q] = 0.0f;
        if (i0 + r >= i_own) load_cols<RC, FULL>(row, c, hd, u[r]);   // wave-uniform: rows this wavefront owns
    }
}

// d_u[n, i0+r, c+q] = u[r][q] + acc[r][q] (one rounding) for the owned rows and columns < hd.
template <int RI, int RC, bool FULL>
__device__ __forceinline__ void store_rows(const float (&acc)[RI][RC], const float (&u)[RI][RC], float* dun, int64_t ld,
                                           int i0, int i_own, int c, int hd) {
    float* row = dun + static_cast<int64_t>(i0) * ld;
#pragma unroll
    for (int r = 0; r < RI; ++r, row += ld) {
        if (i0 + r < i_own) continue;                       // wave-uniform: rows of the previous row block
        if constexpr (FULL) {
            if constexpr (RC == 4) {
                *reinterpret_cast<f32x4u*>(row + c) =
                    f32x4u{u[r][0] + acc[r][0], u[r][1] + acc[r][1], u[r][2] + acc[r][2], u[r][3] + acc[r][3]};
            } else if constexpr (RC == 2) {
                *reinterpret_cast<f32x2u*>(row + c) = f32x2u{u[r][0] + acc[r][0], u[r][1] + acc[r][1]};
            } else {
                row[c] = u[r][0] + acc[r][0];
            }
        } else {
#pragma unroll
            for (int q = 0; q < RC; ++q)
                if (c + q < hd) row[c + q] = u[r][q] + acc[r][q];
        }
    }
}

template <int RI, int RC, int WAVES, int STAGE>
__global__ __launch_bounds__(64 * WAVES) void gx_chain_kernel(const KernelArgs a) {
    constexpr int CW = 64 * RC;                                   // columns per wavefront / workgroup
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    unsigned b = blockIdx.x;
    if (a.xcd_remap) {                                            // same-chunk workgroups onto one XCD
        const unsigned per = gridDim.x >> 3;
        if (b < per * 8u) b = (b & 7u) * per + (b >> 3);
    }
    const unsigned ncb = static_cast<unsigned>(a.ncb), nrg = static_cast<unsigned>(a.nrg);
    const int cb = static_cast<int>(b % ncb);
    b /= ncb;
    const int rg = static_cast<int>(b % nrg);
    const int64_t n = a.n_begin + static_cast<int64_t>(b / nrg);
    const int C = a.C, hd = a.hd;
    const int i_own = (rg * WAVES + wave) * RI;                   // first row this wavefront owns
    const bool active = i_own < C;                                // wave-uniform
    const int i0 = i_own < C - RI ? i_own : C - RI;               // row block, shifted back at the tail (RI <= C)
    const int c0 = cb * CW;
    const int c = c0 + lane * RC;
    const bool full = c0 + CW <= hd;                              // wave-uniform: every lane's columns < hd

    const float* dvn = a.dv + n * static_cast<int64_t>(C) * a.ld_dv;      // d_dv[n, 0, 0]
    float* dun = a.du + n * static_cast<int64_t>(C) * a.ld_u;              // d_u[n, 0, 0]
    const cf32p xr = (cf32p)(a.x + n * static_cast<int64_t>(C) * C + i0);        // x[n, 0, i0], scalar loads

    float acc[RI][RC];
#pragma unroll
    for (int r = 0; r < RI; ++r)
#pragma unroll
        for (int q = 0; q < RC; ++q) acc[r][q] = 0.0f;              // the chain starts from +0

    float u[RI][RC];

    if constexpr (STAGE == 0) {
        if (!active) return;                                      // no barrier in this variant
        if (full) {
            chain_rows<RI, RC>(acc, xr, C, 0, C, GlobalRows<RC, true>{dvn, a.ld_dv, c, hd});
            load_rows<RI, RC, true>(u, dun, a.ld_u, i0, i_own, c, hd);
            store_rows<RI, RC, true>(acc, u, dun, a.ld_u, i0, i_own, c, hd);
        } else {
            chain_rows<RI, RC>(acc, xr, C, 0, C, GlobalRows<RC, false>{dvn, a.ld_dv, c, hd});
            load_rows<RI, RC, false>(u, dun, a.ld_u, i0, i_own, c, hd);
            store_rows<RI, RC, false>(acc, u, dun, a.ld_u, i0, i_own, c, hd);
        }
    } else {
        // d_dv slab [SJ][CW] in LDS, rows s .. s+SJ-1, columns c0 .. c0+CW-1 (zero past hd).
        extern __shared__ f32x4a lds_vec[];
        float* ds = reinterpret_cast<float*>(lds_vec);
        constexpr int T = 64 * WAVES;
        constexpr int G = CW / 4;                                 // 16-byte groups per slab row
        const int SJ = a.slab_rows;
        for (int s = 0; s < C; s += SJ) {
            const int rows = SJ < C - s ? SJ : C - s;
            if (s) __syncthreads();                               // everyone is done reading the previous slab
            for (int g = static_cast<int>(threadIdx.x); g < rows * G; g += T) {
                const int rr = g / G, cc = (g - rr * G) * 4;
                const float* src = dvn + static_cast<int64_t>(s + rr) * a.ld_dv + c0 + cc;
                f32x4a v;
                if (c0 + cc + 4 <= hd) {
                    const f32x4u t = *reinterpret_cast<const f32x4u*>(src);
                    v = f32x4a{t.x, t.y, t.z, t.w};
                } else {
                    v.x = (c0 + cc + 0 < hd) ? src[0] : 0.0f;
                    v.y = (c0 + cc + 1 < hd) ? src[1] : 0.0f;
                    v.z = (c0 + cc + 2 < hd) ? src[2] : 0.0f;
                    v.w = (c0 + cc + 3 < hd) ? src[3] : 0.0f;
                }
                *reinterpret_cast<f32x4a*>(ds + rr * CW + cc) = v;
            }
            __syncthreads();                                      // the slab is in LDS
            if (active) chain_rows<RI, RC>(acc, xr, C, s, s + rows, LdsRows<RC, CW>{ds + lane * RC, s});
        }
        if (active) {
            if (full) {
                load_rows<RI, RC, true>(u, dun, a.ld_u, i0, i_own, c, hd);
                store_rows<RI, RC, true>(acc, u, dun, a.ld_u, i0, i_own, c, hd);
            } else {
                load_rows<RI, RC, false>(u, dun, a.ld_u, i0, i_own, c, hd);
                store_rows<RI, RC, false>(acc, u, dun, a.ld_u, i0, i_own, c, hd);
            }
        }
    }
}

// ---- instance table -----------------------------------------------------------------------------------------------
// Instances: every (RI, RC) tile for 1, 2, 4 and 8 wavefronts per workgroup; 16 wavefronts (1024 threads, so at
// most 128 VGPRs per lane) only for the tiles that fit without spilling.
#define SDM_GX_INST(RI, RC, W, S) {RI, RC, W, S, reinterpret_cast<const void*>(&gx_chain_kernel<RI, RC, W, S>)},
#define SDM_GX_INST_W(RI, RC, S) SDM_GX_INST(RI, RC, 1, S) SDM_GX_INST(RI, RC, 2, S) SDM_GX_INST(RI, RC, 4, S) \
    SDM_GX_INST(RI, RC, 8, S)
#define SDM_GX_INST_RC(RI, S) SDM_GX_INST_W(RI, 1, S) SDM_GX_INST_W(RI, 2, S) SDM_GX_INST_W(RI, 4, S)
#define SDM_GX_INST_S(S) SDM_GX_INST_RC(1, S) SDM_GX_INST_RC(2, S) SDM_GX_INST_RC(4, S) SDM_GX_INST_RC(8, S) \
    SDM_GX_INST_RC(16, S) \
    SDM_GX_INST(4, 1, 16, S) SDM_GX_INST(4, 2, 16, S) SDM_GX_INST(4, 4, 16, S) SDM_GX_INST(8, 1, 16, S) \
    SDM_GX_INST(8, 2, 16, S) SDM_GX_INST(8, 4, 16, S) SDM_GX_INST(16, 1, 16, S)

static const KernelEntry kTable[] = {SDM_GX_INST_S(0) SDM_GX_INST_S(1)};

const void* find_kernel(int ri, int rc, int waves, int stage) {
    for (const KernelEntry& e : kTable)
        if (e.ri == ri && e.rc == rc && e.waves == waves && e.stage == stage) return e.fn;
    return nullptr;
}

}  // namespace sdm_gx
