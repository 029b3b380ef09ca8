// Matrix-core engine of the deterministic FP32 per-step d_u update on gfx950.
//
// Operation (page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_gemm_cuda.py", module docstring and
// gx_gemm_kernel): for chunk n, row i < C and column c < hd,
//     acc = +0;  acc = fma(x[n, j, i], d_dv[n, j, c], acc) for j = 0..C-1 in order;  d_u[n, i, c] += acc
// with one separately rounded add.
//
// Why the matrix cores can run this chain: an FP32 MFMA with K = 1 (v_mfma_f32_32x32x1_2b_f32,
// v_mfma_f32_16x16x1_4b_f32) computes, for every element of its blocks, d = c + a*b with a single rounding (round to
// nearest even, subnormals kept): exactly one fmaf step. There is no reduction inside the instruction, so issuing one
// such MFMA per chain step j, in order, with the accumulator fed back as c, is the chain itself. (Checked bit for bit
// against fmaf on tens of millions of operand triples, including subnormals, cancellations, signed zeros, Inf and
// NaN, and by the parity tests.) MFMAs with K > 1 sum several products inside one instruction and are not used.
//
// Common structure (persistent workgroups; every global access is in long, coalesced streams):
//   * Work items are (chunk, row group, column group) tiles of 64*RW rows x (block*QW) columns, block = 32 or 16
//     columns per compute wavefront. Each workgroup takes a contiguous range of items and walks them in order.
//   * Compute wavefronts (RW x QW of them) each own one 64-row output tile; lane l supplies A = x[n, j, i0 + l].
//   * Loader wavefronts (LW of them) stream the x and d_dv rows of all the workgroup's items, a slab of chain rows
//     at a time, into an S-stage LDS ring that runs S-1 slabs ahead of the compute wavefronts; one workgroup barrier
//     per slab. Compute wavefronts read their MFMA operands from the ring, the next group of 4 chain rows always in
//     flight while the MFMAs of the current group issue.
//   * d_u of an item is read by the compute wavefronts in accumulator layout (buffer loads with a scalar row offset)
//     and d_u + acc is stored at the end of the item (one rounding).
//
// gx_mfma_kernel (register ring): 32-column wavefronts (two 32x32 blocks stacked along the rows); slabs of 16 rows
// move through an R-deep register ring of float4 loads into LDS. Rows past C are filled with x = -0 and d_dv = +0:
// their product is -0 and acc + (-0) == acc for every acc (including +-0, Inf and NaN), so a partial last slab runs
// the full 16 steps without changing a bit. DU_AT_END = 0 prefetches d_u when the item starts; DU_AT_END = 1 reads
// it at the end, which saves 32 registers per lane: those instances are built for 6 wavefronts per SIMD (MINW), so
// two workgroups share a compute unit and overlap each other's phases.
//
// gx_mfma_dma_kernel (direct to LDS): slabs of 16 or 32 rows move from memory straight into their LDS stage with
// buffer_load_dwordx4 ... lds; 32- or 16-column wavefronts; rows past C are skipped, not padded. Its own comment
// block below has the details.
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
constexpr int kNonTemporal = 2;            // buffer instruction cache policy: nt (streaming)

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

// Work item cursor with the chunk fastest: item it = ((rg * ncg) + cg) * nch + n for the launch's nch chunks.
// Workgroups b and b + nch / per (per items each) then walk the same chunks in step for different column groups;
// workgroups are dealt to the 8 XCDs round-robin, so when nch / per is a multiple of 8 they share an XCD and its L2,
// and a chunk's x (read by every column group) and d_dv (read by every row group) come from HBM once.
struct ChunkCursor {
    int n, rg, cg;
    __device__ __forceinline__ void init(int it, int nch, int ncg) {
        n = __builtin_amdgcn_readfirstlane(it % nch);
        it /= nch;
        cg = __builtin_amdgcn_readfirstlane(it % ncg);
        rg = __builtin_amdgcn_readfirstlane(it / ncg);
    }
    __device__ __forceinline__ void next(int nch, int ncg) {
        if (++n == nch) {
            n = 0;
            if (++cg == ncg) {
                cg = 0;
                ++rg;
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

// ---- direct-to-LDS variant ----------------------------------------------------------------------------------------
// Same work items, LDS stage layout (x rows, then d_dv rows) and d_u handling as gx_mfma_kernel, with 32- or
// 16-column compute wavefronts (MS) and slabs of J = 16 or 32 chain rows; the loader wavefronts move each slab
// straight from memory into its LDS stage with buffer_load_dwordx4 ... lds (one instruction moves 64 x 16 contiguous
// bytes of LDS; each lane names its own source). No register ring: up to S - 1 slabs are in flight per workgroup at
// no register cost. Rows must share one offset from a 16-byte boundary per array (C and ld_dv multiples of 4:
// checked on the host); ALN selects the instances for rows that are off the boundary.
//   * Slab q of the workgroup's stream goes to stage q mod S. Tick q: the loader waits (vmcnt) until slab q has landed,
//     everyone meets at barrier B_q, the compute wavefronts run slab q, and the loader issues slab q + S - 1 into
//     stage (q - 1) mod S, whose reads by the compute wavefronts ended before B_q.
//   * Out-of-range sources are cut by the buffer bounds (the chunk's extent): nothing outside the chunk is read.
//     Rows past C in a slab are never used: the last slab of an item runs only its C - J*s chain steps, so no
//     padding value has to be exact. Stale or zero LDS in columns past hd or rows past C only reaches outputs
//     that are never stored.
//   * The loader meets the barriers with a bare s_barrier (the compute side's barrier would make the compiler wait
//     for every load in flight); an empty asm with a memory clobber keeps the compiler from moving memory
//     operations across it.
typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from buffer offset voff into LDS at lds + 16 * lane (lds wave-uniform)
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, float* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, 0, 0, 0);
}

// 4 bytes per lane from buffer offset voff into LDS at lds + 4 * lane (lds wave-uniform)
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t r, float* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, voff, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {     // s_waitcnt vmcnt(N), other counters unconstrained
    static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// vmcnt(ahead * PERW) for a runtime ahead in [0, A]
template <int PERW, int A>
__device__ __forceinline__ void wait_slabs(int ahead) {
    if constexpr (A == 0) {
        wait_vmcnt<0>();
    } else {
        if (ahead >= A) wait_vmcnt<A * PERW>();
        else wait_slabs<PERW, A - 1>(ahead);
    }
}

__device__ __forceinline__ void loader_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The two K = 1 FP32 MFMA shapes a compute wavefront can run the chain on; both give a 64-row output tile (lane l
// supplies A = x[n, j, i0 + l]).
//   32: v_mfma_f32_32x32x1_2b_f32, 64 rows x 32 columns, B = d_dv[n, j, c0 + l % 32], 64 cycles per step.
//   16: v_mfma_f32_16x16x1_4b_f32, 64 rows x 16 columns, B = d_dv[n, j, c0 + l % 16], 32 cycles per step. Four
//       16x16 blocks; register r holds block r/4 (rows 16*(r/4) ..), row 4*(l/16) + r%4 of it, column l % 16.
template <int MS> struct MfShape;
template <> struct MfShape<32> {
    typedef v32f acc_t;
    static constexpr int NR = 32;
    __device__ static __forceinline__ acc_t step(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x1f32(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ constexpr int row(int r) { return acc_row(r, 0); }
    __device__ static __forceinline__ int lane_row(int lane) { return 4 * (lane >> 5); }
};
template <> struct MfShape<16> {
    typedef float acc_t __attribute__((ext_vector_type(16)));
    static constexpr int NR = 16;
    __device__ static __forceinline__ acc_t step(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x1f32(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ constexpr int row(int r) { return 16 * (r >> 2) + (r & 3); }
    __device__ static __forceinline__ int lane_row(int lane) { return 4 * (lane >> 4); }
};

template <int RW, int QW, int S, int LW, int DU_AT_END, int MINW, int MS, int J, int ALN>
__global__ __launch_bounds__(64 * (RW * QW + LW), MINW) void gx_mfma_dma_kernel(const MfmaArgs a) {
    typedef MfShape<MS> M;
    typedef typename M::acc_t acc_t;
    constexpr int NR = M::NR;
    constexpr int CWV = RW * QW;
    constexpr int XW = 64 * RW, DW = MS * QW;          // x / d_dv columns of a work item
    // LDS rows: for rows that start 4, 8 or 12 bytes past a 16-byte boundary (ALN bit 0: x, bit 1: d_dv) each row
    // is loaded from the boundary below its start, one more 16-byte group per row; the first `shift` floats of such
    // an LDS row are then not the row's. ALN bit 2 moves such d_dv rows with 4-byte DMA instead: 64 floats per
    // instruction at any 4-byte offset, LDS rows exactly DW floats (1-3% faster on 64 x 64 items).
    constexpr int AX = ALN & 1, AD = (ALN >> 1) & 1, D4 = (ALN >> 2) & 1;
    static_assert(!(AD && D4), "one way of moving unaligned d_dv rows");
    static_assert(!D4 || (64 % DW == 0 || DW % 64 == 0), "4-byte DMA: rows of a 64-float instruction");
    constexpr int XR = XW + 4 * AX, DR = DW + 4 * AD;            // LDS row widths in floats
    constexpr int GXR = XR / 4, GDR = DR / 4;                    // 16-byte groups per LDS row
    constexpr int NIX = (J * GXR + 63) / 64;                     // DMA instructions per slab: x, d_dv
    constexpr int NID = D4 ? (J * DW + 63) / 64 : (J * GDR + 63) / 64;
    constexpr int NI = NIX + NID, GS = NIX * 64 + NID * (D4 ? 16 : 64);   // float4 groups of one stage
    constexpr int PERW = NI / LW;                       // per loader wavefront per slab
    constexpr int K = kOperandGroup;
    constexpr int kNoSource = 0x3FFFFFF0;               // padding lanes: a float offset past every buffer range
    static_assert(S >= 2, "S: at least two stages");
    static_assert(NIX % LW == 0 && NID % LW == 0, "loader wavefronts split x and d_dv evenly");
    static_assert((S - 2) * PERW <= 63, "slabs in flight exceed the vmcnt range");
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int C = a.C, hd = a.hd;
    const int first = static_cast<int>(blockIdx.x) * a.per;          // < n_items < 2^31
    const int left = a.n_items - first;
    const int nmine = left < a.per ? left : a.per;
    if (nmine <= 0) return;                             // workgroup-uniform: no barrier reached
    const int ns = (C + J - 1) / J;                     // slabs per item
    const int nfull = C / J;                            // of them holding J chain rows
    const int nch = a.n_items / (a.nrg * a.ncg);        // chunks of the launch
    const int64_t total = static_cast<int64_t>(nmine) * ns;

    __shared__ f32x4a ring[S][GS];

    if (wave >= CWV) {
        const int wl = wave - CWV;
        // instruction k of this wavefront is slab instruction m = wl + k*LW: x for k < NIX/LW, d_dv after;
        // lane offsets within the slab (floats) do not depend on the slab
        int off[PERW];
#pragma unroll
        for (int k = 0; k < PERW; ++k) {
            const int m = wl + k * LW;
            if (k < NIX / LW) {
                const int g = m * 64 + lane, jj = g / GXR;
                off[k] = g < J * GXR ? jj * C + (g - jj * GXR) * 4 : kNoSource;
            } else if (D4) {
                const int h = (m - NIX) * 64 + lane, jj = h / DW;
                off[k] = h < J * DW ? jj * static_cast<int>(a.ld_dv) + (h - jj * DW) : kNoSource;
            } else {
                const int h = (m - NIX) * 64 + lane, jj = h / GDR;
                off[k] = h < J * GDR ? jj * static_cast<int>(a.ld_dv) + (h - jj * GDR) * 4 : kNoSource;
            }
        }
        // floats from the 16-byte boundary below each row start (the same for every row: C and ld_dv are
        // multiples of 4); that boundary is in the same 16-byte block, hence the same page, as the row start
        const int sx = AX ? static_cast<int>(reinterpret_cast<uintptr_t>(a.x) >> 2) & 3 : 0;
        const int sd = AD ? static_cast<int>(reinterpret_cast<uintptr_t>(a.dv) >> 2) & 3 : 0;
        ChunkCursor lc;
        lc.init(first, nch, a.ncg);
        int ls = 0;
        auto issue = [&](int stage) {                   // slab ls of item lc into `stage`
            const int64_t n = a.n_begin + lc.n;
            const int xo = ls * J * C + lc.rg * XW - sx;                 // first float of the slab in x's chunk
            const int64_t dvo = static_cast<int64_t>(ls * J) * a.ld_dv + lc.cg * DW - sd;
            const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(a.x) + n * C * C + xo, (short)0, (C * C - xo) * 4, kBufferFlags);
            const int dv_end = static_cast<int>((static_cast<int64_t>(C - 1) * a.ld_dv + hd - dvo) * 4);
            const __amdgpu_buffer_rsrc_t dr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(a.dv) + n * C * a.ld_dv + dvo, (short)0, dv_end, kBufferFlags);
            float* st = reinterpret_cast<float*>(&ring[stage][0]);
#pragma unroll
            for (int k = 0; k < PERW; ++k) {
                const int m = wl + k * LW;
                if (k < NIX / LW)
                    load_lds16(xr, st + m * 256, static_cast<int>(static_cast<unsigned>(off[k]) * 4u));
                else if (D4)
                    load_lds4(dr, st + NIX * 256 + (m - NIX) * 64,
                              static_cast<int>(static_cast<unsigned>(off[k]) * 4u));
                else
                    load_lds16(dr, st + m * 256, static_cast<int>(static_cast<unsigned>(off[k]) * 4u));
            }
            if (++ls == ns) {
                ls = 0;
                lc.next(nch, a.ncg);
            }
        };
#pragma unroll
        for (int m = 0; m < S - 1; ++m)
            if (m < total) issue(m);
        int ist = S - 1;                                // stage of slab q + S - 1: (q + S - 1) mod S
        for (int64_t q = 0; q < total; ++q) {
            const int64_t rest = total - 1 - q;         // slabs after q already issued: min(S - 2, rest)
            wait_slabs<PERW, S - 2>(rest < S - 2 ? static_cast<int>(rest) : S - 2);
            loader_barrier();                           // B_q: slab q is in LDS
            if (q + S - 1 < total) issue(ist);
            ist = ist + 1 == S ? 0 : ist + 1;
        }
    } else {
        const int rw = wave / QW, qw = wave - (wave / QW) * QW;
        const int sx = AX ? static_cast<int>(reinterpret_cast<uintptr_t>(a.x) >> 2) & 3 : 0;
        const int sd = AD ? static_cast<int>(reinterpret_cast<uintptr_t>(a.dv) >> 2) & 3 : 0;
        const float* xs0 = reinterpret_cast<const float*>(&ring[0][0]) + rw * 64 + lane + sx;
        const float* ds0 = reinterpret_cast<const float*>(&ring[0][0]) + NIX * 256 + qw * MS + (lane & (MS - 1)) + sd;
        constexpr int STAGE_FLOATS = GS * 4;
        acc_t acc;
        auto compute = [&](const float* xs, const float* ds) {   // J chain steps from one ring stage
            float ra[2][K], rb[2][K];
            auto rd = [&](int buf, int grp) {
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    ra[buf][k] = xs[(grp * K + k) * XR];
                    rb[buf][k] = ds[(grp * K + k) * DR];
                }
            };
            rd(0, 0);
#pragma unroll
            for (int grp = 0; grp < J / K; ++grp) {
                if (grp + 1 < J / K) rd((grp + 1) & 1, grp + 1);   // next group's operands in flight ...
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int k = 0; k < K; ++k)                        // ... while this group's chain steps issue
                    acc = M::step(ra[grp & 1][k], rb[grp & 1][k], acc);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto compute_tail = [&](const float* xs, const float* ds, int nk) {   // the first nk < J chain steps
            for (int k = 0; k < nk; ++k) acc = M::step(xs[k * XR], ds[k * DR], acc);
        };
        ChunkCursor cc;
        cc.init(first, nch, a.ncg);
        const int lr = M::lane_row(lane);
        const int ld4 = static_cast<int>(a.ld_u) * 4;   // < 2^31 / C: checked on the host
        int cst = 0;                                    // stage of the next slab
        float u[NR];
        for (int t = 0; t < nmine; ++t) {
            const int64_t n = a.n_begin + cc.n;
            const int i0 = cc.rg * XW + rw * 64, c = cc.cg * DW + qw * MS + (lane & (MS - 1));
            const bool full = i0 + 64 <= C && cc.cg * DW + qw * MS + MS <= hd;   // wave-uniform
            float* un = a.du + n * C * a.ld_u;
            const __amdgpu_buffer_rsrc_t ur = __builtin_amdgcn_make_buffer_rsrc(un, (short)0, C * ld4, kBufferFlags);
            const unsigned vo = static_cast<unsigned>(((i0 + lr) * static_cast<int>(a.ld_u) + c) * 4);
            acc = (acc_t){0};                            // the chain starts from +0
            auto uload = [&]() {
                if (full) {
#pragma unroll
                    for (int r = 0; r < NR; ++r)
                        u[r] = __builtin_bit_cast(float,
                                                  __builtin_amdgcn_raw_buffer_load_b32(ur, vo, M::row(r) * ld4, 0));
                } else {
#pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        const int i = i0 + M::row(r) + lr;
                        u[r] = (i < C && c < hd) ? un[static_cast<int64_t>(i) * a.ld_u + c] : 0.f;
                    }
                }
            };
            if (!DU_AT_END) uload();
            // full slabs, then the partial last one: two loops, so the accumulator keeps its registers across
            // slabs (one loop with both paths had the compiler copy it between register sets at every slab)
            for (int s = 0; s < nfull; ++s) {
                __syncthreads();                        // B_q: slab q is in LDS
                const int off = cst * STAGE_FLOATS;
                compute(xs0 + off, ds0 + off);
                cst = cst + 1 == S ? 0 : cst + 1;
            }
            if (nfull < ns) {
                __syncthreads();
                const int off = cst * STAGE_FLOATS;
                compute_tail(xs0 + off, ds0 + off, C - nfull * J);
                cst = cst + 1 == S ? 0 : cst + 1;
            }
            if (DU_AT_END) uload();
            if (full && a.stream_du) {                  // non-temporal hint (nt): written once, not re-read here
#pragma unroll
                for (int r = 0; r < NR; ++r)
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, u[r] + acc[r]), ur, vo,
                                                          M::row(r) * ld4, kNonTemporal);
            } else if (full) {
#pragma unroll
                for (int r = 0; r < NR; ++r)
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, u[r] + acc[r]), ur, vo,
                                                          M::row(r) * ld4, 0);
            } else {
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const int i = i0 + M::row(r) + lr;
                    if (i < C && c < hd) un[static_cast<int64_t>(i) * a.ld_u + c] = u[r] + acc[r];
                }
            }
            cc.next(nch, a.ncg);
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
     static_cast<int>(sizeof(f32x4a) * S * kSlabRows * (16 * RW + 8 * QW)), 32, kSlabRows, 0},
#define SDM_GX_MF(RW, QW, S, R, LW) SDM_GX_MF_X(RW, QW, S, R, LW, 0, 1)
#define SDM_GX_MF_RL(RW, QW) SDM_GX_MF(RW, QW, 4, 4, 4) SDM_GX_MF(RW, QW, 4, 2, 4) SDM_GX_MF(RW, QW, 4, 4, 2) \
    SDM_GX_MF(RW, QW, 4, 2, 2)

// Direct-to-LDS instances (reg_slabs = 0). 32-column tiles: S = 4 stages of 16 chain rows and 1 loader wavefront,
// and S = 8 and 2 loader wavefronts; the 128 x 128 tile also reading d_u at the item's end, built for two
// workgroups per CU; 64 x 128 tiles (1 x 4 wavefronts) with S = 3 stages of 32 rows: with 2 loader wavefronts
// (also with d_dv rows by 4-byte DMA, ALN 4), and with 1 (also with rows from the 16-byte boundary below, ALN 2 and 3,
// for unaligned x). 16-column tiles: S = 3 stages of 16 or 32 chain rows and 1 loader wavefront (also for rows off
// a 16-byte boundary, chosen at launch from the pointers: ALN 4 d_dv rows by 4-byte DMA, or ALN 2 from the boundary
// below where 4-byte DMA would exceed the vmcnt range (64 x 128 tiles with 32-row stages); ALN 3 x rows too), and
// S = 8 of 16 rows with 2 loader wavefronts.
#define SDM_GX_MD_A(RW, QW, S, LW, DE, MW, MS, J, ALN) \
    {RW, QW, S, 0, LW, DE, reinterpret_cast<const void*>(&gx_mfma_dma_kernel<RW, QW, S, LW, DE, MW, MS, J, ALN>), \
     static_cast<int>(sizeof(f32x4a) * S * \
                      (64 * ((J * (16 * RW + (ALN & 1)) + 63) / 64) + \
                       (ALN & 4 ? 16 * ((J * MS * QW + 63) / 64) \
                                : 64 * ((J * (MS / 4 * QW + ((ALN >> 1) & 1)) + 63) / 64)))), \
     MS, J, ALN},
#define SDM_GX_MD(RW, QW, S, LW, DE, MW, MS, J) SDM_GX_MD_A(RW, QW, S, LW, DE, MW, MS, J, 0)
#define SDM_GX_MD2(RW, QW, MS) SDM_GX_MD(RW, QW, 4, 1, 0, 1, MS, 16) SDM_GX_MD(RW, QW, 8, 2, 0, 1, MS, 16)
#define SDM_GX_MD3(RW, QW) SDM_GX_MD(RW, QW, 3, 1, 0, 1, 16, 16) SDM_GX_MD(RW, QW, 8, 2, 0, 1, 16, 16) \
    SDM_GX_MD(RW, QW, 3, 1, 0, 1, 16, 32) \
    SDM_GX_MD_A(RW, QW, 3, 1, 0, 1, 16, 16, 2) SDM_GX_MD_A(RW, QW, 3, 1, 0, 1, 16, 32, 2) \
    SDM_GX_MD_A(RW, QW, 3, 1, 0, 1, 16, 16, 3) SDM_GX_MD_A(RW, QW, 3, 1, 0, 1, 16, 32, 3)
#define SDM_GX_MD4(RW, QW) SDM_GX_MD_A(RW, QW, 3, 1, 0, 1, 16, 16, 4) SDM_GX_MD_A(RW, QW, 3, 1, 0, 1, 16, 32, 4)

const MfmaEntry kMfmaTable[] = {
    SDM_GX_MD2(1, 1, 32) SDM_GX_MD2(1, 2, 32) SDM_GX_MD2(1, 4, 32) SDM_GX_MD2(1, 8, 32) SDM_GX_MD2(2, 1, 32)
    SDM_GX_MD2(2, 2, 32) SDM_GX_MD2(2, 4, 32) SDM_GX_MD(2, 4, 4, 1, 1, 5, 32, 16)
    SDM_GX_MD(1, 4, 3, 1, 0, 1, 32, 32) SDM_GX_MD_A(1, 4, 3, 1, 0, 1, 32, 32, 2) SDM_GX_MD_A(1, 4, 3, 1, 0, 1, 32, 32, 3)
    SDM_GX_MD(1, 4, 3, 2, 0, 1, 32, 32) SDM_GX_MD_A(1, 4, 3, 2, 0, 1, 32, 32, 4)
    SDM_GX_MD3(1, 2) SDM_GX_MD3(1, 4) SDM_GX_MD3(1, 8) SDM_GX_MD3(2, 2) SDM_GX_MD3(2, 4)
    SDM_GX_MD4(1, 2) SDM_GX_MD4(1, 4) SDM_GX_MD4(2, 2) SDM_GX_MD4(2, 4) SDM_GX_MD_A(1, 8, 3, 1, 0, 1, 16, 16, 4)
    SDM_GX_MF_RL(1, 1) SDM_GX_MF_RL(1, 2) SDM_GX_MF_RL(1, 4)
    SDM_GX_MF(1, 8, 4, 4, 4) SDM_GX_MF(1, 8, 4, 2, 4) SDM_GX_MF(1, 8, 4, 2, 2)
    SDM_GX_MF_RL(2, 1) SDM_GX_MF_RL(2, 2)
    SDM_GX_MF(2, 4, 4, 4, 4) SDM_GX_MF(2, 4, 4, 2, 4) SDM_GX_MF(2, 4, 4, 2, 2)
    SDM_GX_MF_X(2, 4, 4, 2, 4, 1, 6) SDM_GX_MF_X(1, 4, 4, 2, 4, 1, 6)
};

}  // namespace

const MfmaEntry* find_mfma_kernel(int row_waves, int col_waves, int stages, int reg_slabs, int loader_waves,
                                  int du_at_end, int block, int slab_rows, int aln) {
    for (const MfmaEntry& e : kMfmaTable)
        if (e.row_waves == row_waves && e.col_waves == col_waves && e.stages == stages && e.reg_slabs == reg_slabs &&
            e.loader_waves == loader_waves && e.du_at_end == du_at_end && e.block == block &&
            e.slab_rows == slab_rows && e.aln == aln)
            return &e;
    return nullptr;
}

}  // namespace sdm_gx
