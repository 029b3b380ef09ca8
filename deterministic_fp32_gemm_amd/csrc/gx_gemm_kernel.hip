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
typedef __attribute__((address_space(4))) const float* cf32p;

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

// One step j of the chain for the wavefront's RI rows: acc[r][q] = fma(x[n, j, i0+r], d[q], acc[r][q]).
// xrow points at x[n, j, i0] in the constant address space (wave-uniform address: scalar loads).
template <int RI, int RC>
__device__ __forceinline__ void chain_step(float (&acc)[RI][RC], cf32p xrow, const float (&d)[RC]) {
#pragma unroll
    for (int r = 0; r < RI; ++r) {
        const float xv = xrow[r];
#pragma unroll
        for (int q = 0; q < RC; ++q) acc[r][q] = __builtin_fmaf(xv, d[q], acc[r][q]);
    }
}

// The whole chain j = 0 .. C-1 with d_dv read from global memory, U rows of d_dv loaded per batch.
template <int RI, int RC, bool FULL>
__device__ __forceinline__ void chain_direct(float (&acc)[RI][RC], cf32p xr, int C, const float* dvn, int64_t ld,
                                             int c, int hd) {
    constexpr int U = 4;
    int j = 0;
    for (; j + U <= C; j += U) {
        float d[U][RC];
#pragma unroll
        for (int u = 0; u < U; ++u) load_cols<RC, FULL>(dvn + static_cast<int64_t>(j + u) * ld, c, hd, d[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) chain_step<RI, RC>(acc, xr + (j + u) * C, d[u]);
    }
    for (; j < C; ++j) {
        float d[RC];
        load_cols<RC, FULL>(dvn + static_cast<int64_t>(j) * ld, c, hd, d);
        chain_step<RI, RC>(acc, xr + j * C, d);
    }
}

// d_u[n, i0+r, c+q] = d_u[n, i0+r, c+q] + acc[r][q] for the rows this wavefront owns (i >= i_own) and columns < hd.
template <int RI, int RC, bool FULL>
__device__ __forceinline__ void store_rows(const float (&acc)[RI][RC], float* dun, int64_t ld, int i0, int i_own,
                                           int c, int hd) {
#pragma unroll
    for (int r = 0; r < RI; ++r) {
        if (i0 + r < i_own) continue;                       // wave-uniform: rows of the previous row block
        float* row = dun + static_cast<int64_t>(i0 + r) * ld;
        if constexpr (FULL) {
            if constexpr (RC == 4) {
                f32x4u u = *reinterpret_cast<const f32x4u*>(row + c);
                u.x = u.x + acc[r][0]; u.y = u.y + acc[r][1]; u.z = u.z + acc[r][2]; u.w = u.w + acc[r][3];
                *reinterpret_cast<f32x4u*>(row + c) = u;
            } else if constexpr (RC == 2) {
                f32x2u u = *reinterpret_cast<const f32x2u*>(row + c);
                u.x = u.x + acc[r][0]; u.y = u.y + acc[r][1];
                *reinterpret_cast<f32x2u*>(row + c) = u;
            } else {
                row[c] = row[c] + acc[r][0];
            }
        } else {
#pragma unroll
            for (int q = 0; q < RC; ++q)
                if (c + q < hd) row[c + q] = row[c + q] + acc[r][q];
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

    if constexpr (STAGE == 0) {
        if (!active) return;                                      // no barrier in this variant
        if (full) {
            chain_direct<RI, RC, true>(acc, xr, C, dvn, a.ld_dv, c, hd);
            store_rows<RI, RC, true>(acc, dun, a.ld_u, i0, i_own, c, hd);
        } else {
            chain_direct<RI, RC, false>(acc, xr, C, dvn, a.ld_dv, c, hd);
            store_rows<RI, RC, false>(acc, dun, a.ld_u, i0, i_own, c, hd);
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
            if (active) {
                for (int jj = 0; jj < rows; ++jj) {
                    float d[RC];
                    const float* src = ds + jj * CW + lane * RC;
                    if constexpr (RC == 4) {
                        const f32x4a v = *reinterpret_cast<const f32x4a*>(src);
                        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
                    } else if constexpr (RC == 2) {
                        d[0] = src[0]; d[1] = src[1];
                    } else {
                        d[0] = src[0];
                    }
                    chain_step<RI, RC>(acc, xr + (s + jj) * C, d);
                }
            }
        }
        if (active) {
            if (full) store_rows<RI, RC, true>(acc, dun, a.ld_u, i0, i_own, c, hd);
            else store_rows<RI, RC, false>(acc, dun, a.ld_u, i0, i_own, c, hd);
        }
    }
}

// ---- instance table -----------------------------------------------------------------------------------------------
#define SDM_GX_INST(RI, RC, W, S) {RI, RC, W, S, reinterpret_cast<const void*>(&gx_chain_kernel<RI, RC, W, S>)},
#define SDM_GX_INST_W(RI, RC, S) SDM_GX_INST(RI, RC, 1, S) SDM_GX_INST(RI, RC, 2, S) SDM_GX_INST(RI, RC, 4, S) \
    SDM_GX_INST(RI, RC, 8, S)
#define SDM_GX_INST_RC(RI, S) SDM_GX_INST_W(RI, 1, S) SDM_GX_INST_W(RI, 2, S) SDM_GX_INST_W(RI, 4, S)
#define SDM_GX_INST_S(S) SDM_GX_INST_RC(1, S) SDM_GX_INST_RC(2, S) SDM_GX_INST_RC(4, S) SDM_GX_INST_RC(8, S) \
    SDM_GX_INST_RC(16, S) SDM_GX_INST_W(32, 1, S) SDM_GX_INST_W(32, 2, S)

static const KernelEntry kTable[] = {SDM_GX_INST_S(0) SDM_GX_INST_S(1)};

const void* find_kernel(int ri, int rc, int waves, int stage) {
    for (const KernelEntry& e : kTable)
        if (e.ri == ri && e.rc == rc && e.waves == waves && e.stage == stage) return e.fn;
    return nullptr;
}

hipError_t launch_kernel(const void* fn, int waves, unsigned grid, unsigned lds_bytes, hipStream_t stream,
                         const KernelArgs& a) {
    void* args[] = {const_cast<KernelArgs*>(&a)};
    return hipLaunchKernel(fn, dim3(grid), dim3(64u * static_cast<unsigned>(waves)), args, lds_bytes, stream);
}

}  // namespace sdm_gx
