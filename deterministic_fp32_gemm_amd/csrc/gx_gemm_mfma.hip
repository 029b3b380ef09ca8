// Matrix-core engine of the deterministic FP32 per-step d_u update on gfx950.
//
// Operation (page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_gemm_cuda.py", module docstring and
// gx_gemm_kernel): for chunk n, row i < C and column c < hd,
//     acc = +0;  acc = fma(x[n, j, i], d_dv[n, j, c], acc) for j = 0..C-1 in order;  d_u[n, i, c] += acc
// with one separately rounded add.
//
// Why the matrix cores can run this chain: an FP32 MFMA with K = 1 (v_mfma_f32_32x32x1_2b_f32) computes, for every
// element of its 32x32 blocks, d = c + a*b with a single rounding (round to nearest even, subnormals kept): exactly
// one fmaf step. There is no reduction inside the instruction, so issuing one such MFMA per chain step j, in order,
// with the accumulator fed back as c, is the chain itself. (Checked bit for bit against fmaf on tens of millions of
// operand triples, including subnormals, cancellations, signed zeros, Inf and NaN, and by the parity tests.) MFMAs
// with K > 1 sum several products inside one instruction and are not used.
//
// Structure (one persistent workgroup per compute unit; every global access is in long, coalesced streams):
//   * Work items are (chunk, row group, column group) tiles of 64*RW rows x 32*QW columns. Each workgroup takes a
//     contiguous range of items and walks them in order.
//   * Compute wavefronts (RW x QW of them) each own one 64-row x 32-column output tile: two 32x32 MFMA blocks
//     stacked along the rows. Lane l supplies A = x[n, j, i0 + l] and B = d_dv[n, j, c0 + l % 32].
//   * Loader wavefronts (LW of them) stream the x and d_dv rows of all the workgroup's items, 16 chain rows ("a
//     slab") at a time, with float4 loads into an R-deep register ring and from there into an S-stage LDS ring that
//     runs S-1 slabs ahead of the compute wavefronts. One workgroup barrier per slab.
//   * Compute wavefronts read their MFMA operands from the LDS ring, the next group of 4 chain rows always in flight
//     while the MFMAs of the current group issue. Rows past C are filled with x = -0 and d_dv = +0: their product is
//     -0 and acc + (-0) == acc for every acc (including +-0, Inf and NaN), so a partial last slab runs the full 16
//     steps without changing a bit.
//   * d_u of an item is read by the compute wavefronts in accumulator layout (buffer loads with a scalar row offset)
//     and d_u + acc is stored at the end of the item (one rounding). DU_AT_END = 0 prefetches it when the item
//     starts; DU_AT_END = 1 reads it at the end, which saves 32 registers per lane: those instances are built for
//     6 wavefronts per SIMD (MINW), so two workgroups share a compute unit and overlap each other's phases.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gx_gemm_mfma.h"

namespace sdm_gx {
namespace {

typedef float v32f __attribute__((ext_vector_type(32)));
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x4a __attribute__((ext_vector_type(4), aligned(16)));

constexpr int kSlabRows = 16;       // chain rows per LDS ring stage
constexpr int kOperandGroup = 4;    // chain rows whose MFMA operands are read ahead
constexpr int kBufferFlags = 0x00020000;   // buffer resource word 3: 32-bit data format, untyped dword access

// 4 floats of a row at column g, zero past `lim`; only columns < lim are dereferenced.
__device__ __forceinline__ f32x4a load4(const float* p, int g, int lim) {
    if (g + 4 <= lim) {
        const f32x4u v = *reinterpret_cast<const f32x4u*>(p + g);
        return f32x4a{v.x, v.y, v.z, v.w};
    }
    f32x4a v = {0.f, 0.f, 0.f, 0.f};
    if (g + 0 < lim) v.x = p[g + 0];
    if (g + 1 < lim) v.y = p[g + 1];
    if (g + 2 < lim) v.z = p[g + 2];
    if (g + 3 < lim) v.w = p[g + 3];
    return v;
}

// Row (relative to the wavefront's first row) of accumulator register r of a 32x32x1 two-block MFMA, lane half h:
// registers 0-15 hold block 0 (rows 0-31), 16-31 block 1 (rows 32-63); within a block, register r covers rows
// 8*(r/4) + r%4 for lanes 0-31 and 4 rows further down for lanes 32-63; the column is lane % 32.
__device__ __forceinline__ constexpr int acc_row(int r, int h) {
    return 32 * (r >> 4) + (r & 3) + 8 * ((r & 15) >> 2) + 4 * h;
}

// Work item cursor (chunk, row group, column group), column group fastest; advanced without division. Item indices
// are below 2^31 (checked on the host). The fields are wave-uniform and pinned to scalar registers: the chunk base
// built from them goes into buffer resources, which must be scalar.
struct Cursor {
    int n, rg, cg;
    __device__ __forceinline__ void init(int it, int nrg, int ncg) {
        cg = __builtin_amdgcn_readfirstlane(it % ncg);
        it /= ncg;
        rg = __builtin_amdgcn_readfirstlane(it % nrg);
        n = __builtin_amdgcn_readfirstlane(it / nrg);
    }
    __device__ __forceinline__ void next(int nrg, int ncg) {
        if (++cg == ncg) {
            cg = 0;
            if (++rg == nrg) {
                rg = 0;
                ++n;
            }
        }
    }
};

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }
constexpr int lcm_c(int a, int b) { return a / gcd_c(a, b) * b; }

template <int RW, int QW, int S, int R, int LW, int DU_AT_END, int MINW>
__global__ __launch_bounds__(64 * (RW * QW + LW), MINW) void gx_mfma_kernel(const MfmaArgs a) {
    constexpr int J = kSlabRows;
    constexpr int CWV = RW * QW, TLD = 64 * LW;
    constexpr int XW = 64 * RW, DW = 32 * QW;          // x / d_dv columns of a work item
    constexpr int GX = XW / 4, GD = DW / 4, GS = J * (GX + GD);   // float4 groups of one slab
    constexpr int PER = (GS + TLD - 1) / TLD;           // slab groups per loader thread
    constexpr int U = lcm_c(S, R);                      // ring period: slabs per item are padded to a multiple
    constexpr int K = kOperandGroup;
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const bool loader = wave >= CWV;                    // wave-uniform role
    const int C = a.C, hd = a.hd;
    const int first = static_cast<int>(blockIdx.x) * a.per;          // < n_items < 2^31
    const int left = a.n_items - first;
    const int nmine = left < a.per ? left : a.per;
    if (nmine <= 0) return;                             // workgroup-uniform: no barrier reached
    const int ns = (C + J - 1) / J;                     // slabs holding chain rows
    const int nsp = (ns + U - 1) / U * U;               // slabs per item, padded
    const int64_t total = static_cast<int64_t>(nmine) * nsp;

    __shared__ f32x4a ring[S][GS];

    if (loader) {
        const int lt = static_cast<int>(threadIdx.x) - 64 * CWV;
        f32x4a reg[R][PER];
        Cursor lc;
        lc.init(first, a.nrg, a.ncg);
        int litem = 0, lslab = 0;
        auto gload = [&](f32x4a (&r)[PER]) {            // the next slab of the stream into registers
            if (litem < nmine) {
                const int ib = lc.rg * XW, cb = lc.cg * DW;
                const int xlim = C - ib < XW ? C - ib : XW, dlim = hd - cb < DW ? hd - cb : DW;
                const int64_t n = a.n_begin + lc.n;
                const float* xn = a.x + n * C * C + ib;
                const float* dvn = a.dv + n * C * a.ld_dv + cb;
#pragma unroll
                for (int k = 0; k < PER; ++k) {
                    const int g = lt + k * TLD;
                    r[k] = f32x4a{0.f, 0.f, 0.f, 0.f};
                    if (GS % TLD == 0 || g < GS) {
                        if (g < J * GX) {
                            const int jj = g / GX, c4 = (g - jj * GX) * 4, j = lslab * J + jj;
                            r[k] = j < C ? load4(xn + static_cast<int64_t>(j) * C, c4, xlim)
                                         : f32x4a{-0.f, -0.f, -0.f, -0.f};
                        } else {
                            const int h = g - J * GX, jj = h / GD, c4 = (h - jj * GD) * 4, j = lslab * J + jj;
                            if (j < C) r[k] = load4(dvn + static_cast<int64_t>(j) * a.ld_dv, c4, dlim);
                        }
                    }
                }
            }
            if (++lslab == nsp) {
                lslab = 0;
                ++litem;
                lc.next(a.nrg, a.ncg);
            }
        };
        auto lput = [&](const f32x4a (&r)[PER], int stage) {
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int g = lt + k * TLD;
                if (GS % TLD == 0 || g < GS) ring[stage][g] = r[k];
            }
        };
        // prologue: R slabs in registers, the first S-1 of them in LDS
#pragma unroll
        for (int m = 0; m < R; ++m) gload(reg[m]);
#pragma unroll
        for (int m = 0; m < S - 1; ++m) {
            lput(reg[m % R], m);
            gload(reg[m % R]);                          // slab m + R
        }
        __syncthreads();
        // step q (slab q being computed): slab q+S-1 goes from register slot (q+S-1)%R to stage (q+S-1)%S, which
        // last held slab q-1 (computed before the previous barrier); the slot then loads slab q+S-1+R.
        int64_t q = 0;
        for (int t = 0; t < nmine; ++t) {
            for (int s0 = 0; s0 < nsp; s0 += U) {
#pragma unroll
                for (int d = 0; d < U; ++d) {           // q % U == d: nsp is a multiple of U
                    if (q + S - 1 < total) {
                        lput(reg[(d + S - 1) % R], (d + S - 1) % S);
                        gload(reg[(d + S - 1) % R]);
                    }
                    ++q;
                    if (q < total) __syncthreads();
                }
            }
        }
    } else {
        const int rw = wave / QW, qw = wave - (wave / QW) * QW;
        const float* xs0 = reinterpret_cast<const float*>(&ring[0][0]) + rw * 64 + lane;
        const float* ds0 = reinterpret_cast<const float*>(&ring[0][0]) + J * XW + qw * 32 + (lane & 31);
        constexpr int STAGE_FLOATS = GS * 4;
        v32f acc;
        auto compute = [&](int stage) {                 // 16 chain steps from one ring stage
            const float* xs = xs0 + stage * STAGE_FLOATS;
            const float* ds = ds0 + stage * STAGE_FLOATS;
            float ra[2][K], rb[2][K];
            auto rd = [&](int buf, int grp) {
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    ra[buf][k] = xs[(grp * K + k) * XW];
                    rb[buf][k] = ds[(grp * K + k) * DW];
                }
            };
            rd(0, 0);
#pragma unroll
            for (int grp = 0; grp < J / K; ++grp) {
                if (grp + 1 < J / K) rd((grp + 1) & 1, grp + 1);   // next group's operands in flight ...
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int k = 0; k < K; ++k)                        // ... while this group's chain steps issue
                    acc = __builtin_amdgcn_mfma_f32_32x32x1f32(ra[grp & 1][k], rb[grp & 1][k], acc, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        __syncthreads();
        Cursor cc;
        cc.init(first, a.nrg, a.ncg);
        const int h = lane >> 5;
        const int ld4 = static_cast<int>(a.ld_u) * 4;   // < 2^31 / C: checked on the host
        int64_t q = 0;
        float u[32];
        for (int t = 0; t < nmine; ++t) {
            const int64_t n = a.n_begin + cc.n;
            const int i0 = cc.rg * XW + rw * 64, c = cc.cg * DW + qw * 32 + (lane & 31);
            const bool full = i0 + 64 <= C && cc.cg * DW + qw * 32 + 32 <= hd;   // wave-uniform
            float* un = a.du + n * C * a.ld_u;
            const __amdgpu_buffer_rsrc_t ur = __builtin_amdgcn_make_buffer_rsrc(un, (short)0, C * ld4, kBufferFlags);
            const unsigned vo = static_cast<unsigned>(((i0 + 4 * h) * static_cast<int>(a.ld_u) + c) * 4);
            acc = (v32f){0};                             // the chain starts from +0
            auto uload = [&]() {
                if (full) {
#pragma unroll
                    for (int r = 0; r < 32; ++r)
                        u[r] = __builtin_bit_cast(float,
                                                  __builtin_amdgcn_raw_buffer_load_b32(ur, vo, acc_row(r, 0) * ld4, 0));
                } else {
#pragma unroll
                    for (int r = 0; r < 32; ++r) {
                        const int i = i0 + acc_row(r, h);
                        u[r] = (i < C && c < hd) ? un[static_cast<int64_t>(i) * a.ld_u + c] : 0.f;
                    }
                }
            };
            if (!DU_AT_END) uload();
            for (int s0 = 0; s0 < nsp; s0 += U) {
#pragma unroll
                for (int d = 0; d < U; ++d) {
                    if (s0 + d < ns) compute(d % S);    // stage of slab q is q % S == d % S
                    ++q;
                    if (q < total) __syncthreads();
                }
            }
            if (DU_AT_END) uload();
            if (full) {
#pragma unroll
                for (int r = 0; r < 32; ++r)
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, u[r] + acc[r]), ur, vo,
                                                          acc_row(r, 0) * ld4, 0);
            } else {
#pragma unroll
                for (int r = 0; r < 32; ++r) {
                    const int i = i0 + acc_row(r, h);
                    if (i < C && c < hd) un[static_cast<int64_t>(i) * a.ld_u + c] = u[r] + acc[r];
                }
            }
            cc.next(a.nrg, a.ncg);
        }
    }
}

// ---- instance table -----------------------------------------------------------------------------------------------
// (row waves, column waves) tiles from 64x32 to 128x128 and 64x256 per item; S = 4 LDS stages; R = 2 or 4 register
// slabs; 2 or 4 loader wavefronts; d_u prefetched at the item's start. Left out: the combinations whose loader ring
// does not fit the registers that the workgroup size allows (they spill): 64x256 and 128x128 tiles with 2 loader
// wavefronts and 4 register slabs. Two instances read d_u at the item's end and are built for two workgroups per CU.
#define SDM_GX_MF_X(RW, QW, S, R, LW, DE, MW) \
    {RW, QW, S, R, LW, DE, reinterpret_cast<const void*>(&gx_mfma_kernel<RW, QW, S, R, LW, DE, MW>), \
     static_cast<int>(sizeof(f32x4a) * S * kSlabRows * (16 * RW + 8 * QW))},
#define SDM_GX_MF(RW, QW, S, R, LW) SDM_GX_MF_X(RW, QW, S, R, LW, 0, 1)
#define SDM_GX_MF_RL(RW, QW) SDM_GX_MF(RW, QW, 4, 4, 4) SDM_GX_MF(RW, QW, 4, 2, 4) SDM_GX_MF(RW, QW, 4, 4, 2) \
    SDM_GX_MF(RW, QW, 4, 2, 2)

const MfmaEntry kMfmaTable[] = {
    SDM_GX_MF_RL(1, 1) SDM_GX_MF_RL(1, 2) SDM_GX_MF_RL(1, 4)
    SDM_GX_MF(1, 8, 4, 4, 4) SDM_GX_MF(1, 8, 4, 2, 4) SDM_GX_MF(1, 8, 4, 2, 2)
    SDM_GX_MF_RL(2, 1) SDM_GX_MF_RL(2, 2)
    SDM_GX_MF(2, 4, 4, 4, 4) SDM_GX_MF(2, 4, 4, 2, 4) SDM_GX_MF(2, 4, 4, 2, 2)
    SDM_GX_MF_X(2, 4, 4, 2, 4, 1, 6) SDM_GX_MF_X(1, 4, 4, 2, 4, 1, 6)
};

}  // namespace

const MfmaEntry* find_mfma_kernel(int row_waves, int col_waves, int stages, int reg_slabs, int loader_waves,
                                  int du_at_end) {
    for (const MfmaEntry& e : kMfmaTable)
        if (e.row_waves == row_waves && e.col_waves == col_waves && e.stages == stages && e.reg_slabs == reg_slabs &&
            e.loader_waves == loader_waves && e.du_at_end == du_at_end)
            return &e;
    return nullptr;
}

}  // namespace sdm_gx
