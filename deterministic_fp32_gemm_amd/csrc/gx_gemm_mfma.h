// Internal interface between the matrix-core kernels and the host entry points of libsdm_gx_gemm (not the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm_gx {

// Work items are (chunk, row group, column group) tiles; workgroup b takes items b*per .. b*per + per - 1 of chunks
// n_begin .. n_begin + n_items / (nrg * ncg) - 1. Item order: column group fastest in the register-ring kernel,
// chunk fastest in the direct-to-LDS kernel.
struct MfmaArgs {
    float* du;
    const float* x;
    const float* dv;
    int64_t ld_u;
    int64_t ld_dv;
    int64_t n_begin;
    int32_t n_items;    // work items of the launch (< 2^31)
    int32_t per;        // items per workgroup
    int32_t C;
    int32_t hd;
    int32_t nrg;        // row groups per chunk: ceil(ceil(C / 64) / row_waves)
    int32_t ncg;        // column groups per chunk: ceil(hd / (block * col_waves))
    int32_t stream_du;  // direct-to-LDS kernel: 1 = d_u stores carry the non-temporal (streaming) hint
};

struct MfmaEntry {
    int row_waves, col_waves, stages, reg_slabs, loader_waves, du_at_end;
    const void* fn;
    int lds_bytes;      // static LDS of the instance
    int block;          // MFMA block: 32 (64x32 tile per compute wavefront) or 16 (64x16)
    int slab_rows;      // chain rows per LDS stage (16, or 32 in some direct-to-LDS instances)
    int aln;            // direct-to-LDS only: for rows that start off a 16-byte boundary, 2: d_dv rows, 3: x too
};

// The kernel instance for the given shape parameters, or nullptr. Launched with a
// 64 * (row_waves * col_waves + loader_waves) thread block and one MfmaArgs argument passed by value.
const MfmaEntry* find_mfma_kernel(int row_waves, int col_waves, int stages, int reg_slabs, int loader_waves,
                                  int du_at_end, int block, int slab_rows, int aln);

}  // namespace sdm_gx
