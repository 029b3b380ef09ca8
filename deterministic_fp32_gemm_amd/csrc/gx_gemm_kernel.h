// Internal interface between the HIP kernels and the host entry points of libsdm_gx_gemm (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm_gx {

// Kernel arguments (passed by value). One launch covers chunks n_begin .. n_begin + grid/(nrg*ncb) - 1.
struct KernelArgs {
    float* du;
    const float* x;
    const float* dv;
    int64_t n_begin;
    int64_t ld_u;
    int64_t ld_dv;
    int32_t C;
    int32_t hd;
    int32_t nrg;        // row groups per chunk: ceil(ceil(C / RI) / waves)
    int32_t ncb;        // column blocks per chunk: ceil(hd / (64 * RC))
    int32_t xcd_remap;  // 0 / 1
    int32_t slab_rows;  // LDS-staged variant: d_dv rows per LDS slab
};

struct KernelEntry {
    int ri, rc, waves, stage;
    const void* fn;
};

// The kernel instance for (rows per wave, columns per lane, waves per workgroup, staging), or nullptr. Launched
// with a 64 * waves thread block and one KernelArgs argument passed by value.
const void* find_kernel(int ri, int rc, int waves, int stage);

}  // namespace sdm_gx
