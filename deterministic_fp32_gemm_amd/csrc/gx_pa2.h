// Internal interface between the Phase A kernel and the host entry points of libsdm_gx_gemm (not the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm_gx {

// One launch = one step ti: grid P * npair * ctas workgroups (slice pair fastest, then chunk, then cta).
struct Pa2Args {
    float* grad;            // [slots][hd]
    float* bank;            // [slots][hd]
    const float* snap;      // [snap_rows][hd]
    const float* du;        // token rows [N*C] of ld_u
    const float* beta;      // [N*C]
    const int32_t* kpay;    // [N][n]
    const int32_t* rec;     // [N][n][4]
    const int32_t* bpre;    // [N][nb + 1] (dense snapshot rows)
    float* out_eff;         // planes of `plane` floats
    float* out_g;
    int64_t slots, snap_rows, ssr, ld_u, plane;
    int32_t ti, P, C, W, n, hd, nsl, slw, npair, ctas, L;
    int32_t stage_out;      // 1: outputs gathered in LDS and written out by the workgroup's last wavefront
};

// The kernel instance for (slices per wavefront, wavefronts per workgroup, outputs staged in LDS), or nullptr.
// Launched with 64 * waves threads, lds bytes of dynamic LDS, one Pa2Args argument by value (stage_out == staged).
const void* find_pa2_kernel(int slices_per_wave, int waves, bool staged);

}  // namespace sdm_gx
