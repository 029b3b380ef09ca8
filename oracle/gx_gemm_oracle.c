/*
 * CPU oracle for the deterministic FP32 per-step d_u update.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load this file or the library built
 * from it: only the tests, the package's smoke check and the benchmark's CPU-baseline leg do. It shares no source,
 * header, table or helper with the HIP library.
 *
 * What it computes (page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_gemm_cuda.py", module docstring,
 * and the j-chain and epilogue of gx_gemm_kernel on the same page):
 *
 *   for each chunk n = ti*P + p (0 <= p < P), row i < C and column c < hd:
 *       acc = +0
 *       for j = 0, 1, ..., C-1 in that order:   acc = fmaf(x[n, j, i], d_dv[n, j, c], acc)
 *       d_u[n, i, c] = d_u[n, i, c] + acc       (one IEEE single-precision add, round to nearest even)
 *
 * x is used transposed: row j of chunk n of x holds x[n, j, 0..C-1] contiguously, and x[n, j, i] multiplies row j
 * of d_dv into output row i. Layouts (same page, gx_gemm_kernel's pointer set-up and the host entry gx_gemm):
 *   x     [N][C][C] contiguous:       x[n, j, i]    at n*C*C + j*C + i
 *   d_dv  [N][C][ld_dv], ld_dv >= hd: d_dv[n, j, c] at (n*C + j)*ld_dv + c
 *   d_u   [N][C][ld_u],  ld_u >= hd:  d_u[n, i, c]  at (n*C + i)*ld_u + c
 * Columns hd..ld-1 and chunks outside step ti are neither read nor written.
 *
 * The arithmetic is the definition itself: fmaf from the C library (correctly rounded by ISO C), applied in the
 * stated j order, then the separate add. Build flags keep the compiler from contracting or reassociating it
 * (-O2 -ffp-contract=off -fno-fast-math). Subnormals must be kept: the entry refuses to run when the SSE control
 * register has flush-to-zero or denormals-are-zero set, or when the rounding mode is not round-to-nearest.
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <xmmintrin.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS (-1)
#define ORACLE_BAD_FPENV (-2)

/* 1 when the host floating-point environment gives IEEE single-precision results with subnormals: MXCSR bit 15
 * (flush-to-zero) and bit 6 (denormals-are-zero) clear, MXCSR rounding field (bits 13-14) round-to-nearest, and the
 * C rounding mode FE_TONEAREST. */
int sdm_gx_oracle_fpenv_ok(void) {
    const unsigned int csr = _mm_getcsr();
    if (csr & (1u << 15)) return 0;
    if (csr & (1u << 6)) return 0;
    if (csr & (3u << 13)) return 0;
    if (fegetround() != FE_TONEAREST) return 0;
    return 1;
}

/* One step ti of the update on host memory, in place on d_u. Returns ORACLE_OK, ORACLE_BAD_ARGS when the arguments
 * do not describe step ti of N chunks (1 <= P <= N, 0 <= ti < N / P, 1 <= C, 1 <= hd <= ld_u, ld_dv, non-null
 * pointers), or ORACLE_BAD_FPENV (see sdm_gx_oracle_fpenv_ok). */
int sdm_gx_oracle_step(float* d_u, int64_t ld_u, const float* x, const float* d_dv, int64_t ld_dv, int64_t N,
                       int64_t ti, int64_t P, int64_t C, int64_t hd) {
    if (!d_u || !x || !d_dv) return ORACLE_BAD_ARGS;
    if (N < 1 || P < 1 || P > N || ti < 0 || ti >= N / P) return ORACLE_BAD_ARGS;
    if (C < 1 || hd < 1 || ld_u < hd || ld_dv < hd) return ORACLE_BAD_ARGS;
    if (!sdm_gx_oracle_fpenv_ok()) return ORACLE_BAD_FPENV;
    for (int64_t p = 0; p < P; ++p) {
        const int64_t n = ti * P + p;
        for (int64_t i = 0; i < C; ++i) {
            for (int64_t c = 0; c < hd; ++c) {
                float acc = +0.0f;
                for (int64_t j = 0; j < C; ++j) {
                    const float xv = x[(n * C + j) * C + i];
                    const float dv = d_dv[(n * C + j) * ld_dv + c];
                    acc = fmaf(xv, dv, acc);
                }
                float* u = &d_u[(n * C + i) * ld_u + c];
                *u = *u + acc;
            }
        }
    }
    return ORACLE_OK;
}
