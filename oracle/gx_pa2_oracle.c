/*
 * CPU oracle for Phase A of the deterministic backward step (the consumer of the updated d_u).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load this file or the library built
 * from it: only the tests, the package's smoke check and the benchmark's CPU-baseline leg do. It shares no source,
 * header, table or helper with the HIP library.
 *
 * What it computes: page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_pa2_cuda.py", gx_pa2_kernel (its
 * record walk, the group chains, the per-lane dot products and the fixed-order butterfly, the LAST stores and the
 * per-entry outputs), for float32 grad, bank and snapshot rows. It follows the kernel's arithmetic in the order the
 * page gives it, written as a plain sequential walk:
 *
 *   For step ti, chunk k = ti*P + p (0 <= p < P), and each column slice sl of the head (nsl = 1 + (hd-1)/128 slices of
 *   slw = 4*ceil(ceil(hd/4)/nsl) columns): walk the chunk's n = C*W records j = 0 .. n-1 in order, with a state of
 *   acc, gdw, sn (one value per slice column, all +0 at the start) and gp (one value per lane, +0 at the start).
 *   A slice is seen as 32 lanes of 4 columns; a column past the slice or past hd reads as +0.
 *     record j = {payload, slot, sck bits, cpe bits}; payload bits: 31 FIRST, 30 LAST, 17 INVALID, 9-16 token t,
 *     0-7 write w (18-29: distance to the group's FIRST, used by the kernel's tiling only)
 *     x = row t of chunk k of d_u (the slice's columns)
 *     FIRST: acc = +0; if the record is valid, gdw = grad row `slot`, sn = the group's snapshot row (else both +0);
 *            per lane q: gp[q] = fmaf(gdw[4q+3], sn[4q+3], fmaf(gdw[4q+2], sn[4q+2], fmaf(gdw[4q+1], sn[4q+1],
 *                                gdw[4q] * sn[4q])))
 *     every record: acc[c] = fmaf(sck, x[c], acc[c]) for every slice column c
 *                   part[q] = fmaf(x[4q+3], sn[4q+3], fmaf(x[4q+2], sn[4q+2], fmaf(x[4q+1], sn[4q+1], x[4q] * sn[4q])))
 *                   dot = tree(part[0..31]), g = tree(gp[0..31]), tree: the balanced pairwise sum in lane order
 *                   ((v0+v1)+(v2+v3)) + ... (the xor butterfly over offsets 1, 2, 4, 8, 16)
 *     LAST and valid: grad row `slot` = fmaf(gdw, cpe, acc) and bank row `slot` = sn, on the slice's columns < hd
 *     output o = k*n + t*W + w:
 *       one slice:  out_eff[o] = valid ? (-beta[k*C + t]) * dot : +0,   out_g[o] = valid ? cpe * g : +0
 *       nsl slices: out_eff[sl*plane + o] = valid ? dot : +0,           out_g[sl*plane + o] = valid ? g : +0
 *   The group's snapshot row (valid FIRST records only):
 *     dense rows (ssr < 0):    k*n + (the number of valid FIRST records before j in chunk k)
 *     per-entry rows (ssr >= 0): ti*ssr + p*C*W + t*W + w of the FIRST record
 *
 * Every multiply, fused multiply-add and add rounds to nearest even in IEEE binary32 with subnormals kept (the page
 * uses the _rn intrinsics); the build keeps the compiler from contracting or reassociating (-O2 -ffp-contract=off
 * -fno-fast-math). The entry refuses to run in a non-IEEE host floating-point environment, as the update oracle does.
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <xmmintrin.h>

#define PA2_OK 0
#define PA2_BAD_ARGS (-1)
#define PA2_BAD_FPENV (-2)
#define PA2_BAD_RECORD (-3)

#define PA2_FIRST 0x80000000u
#define PA2_LAST 0x40000000u
#define PA2_INVALID 0x00020000u
#define PA2_LANES 32
#define PA2_SLICE_MAX 128

static int fpenv_ok(void) {
    const unsigned int csr = _mm_getcsr();
    if (csr & ((1u << 15) | (1u << 6) | (3u << 13))) return 0;
    return fegetround() == FE_TONEAREST;
}

static float bits_to_float(int32_t b) {
    float f;
    memcpy(&f, &b, sizeof f);
    return f;
}

/* balanced pairwise sum of v[0..31] in lane order (destroys v) */
static float lane_tree(float* v) {
    for (int span = 1; span < PA2_LANES; span *= 2)
        for (int i = 0; i < PA2_LANES; i += 2 * span) v[i] = v[i] + v[i + span];
    return v[0];
}

/* the per-lane 4-column chain: fmaf(a3, b3, fmaf(a2, b2, fmaf(a1, b1, a0 * b0))) */
static float lane_dot4(const float* a, const float* b) {
    float s = a[0] * b[0];
    s = fmaf(a[1], b[1], s);
    s = fmaf(a[2], b[2], s);
    s = fmaf(a[3], b[3], s);
    return s;
}

int sdm_pa2_oracle_fpenv_ok(void) { return fpenv_ok(); }

/*
 * One step ti of Phase A on host memory.
 *   grad, bank   [slots][hd]         grad rows are read at valid FIRST records and written at valid LAST records; bank
 *                                    rows are written at valid LAST records
 *   snap         [snap_rows][hd]     snapshot rows; ssr < 0: dense rows, ssr >= 0: per-entry rows (see above)
 *   du           [N*C] rows of ld_u  d_u's token rows, column c < hd at (k*C + t)*ld_u + c
 *   beta         [N*C]
 *   rec          [N][C*W][4]         int32 {payload, slot, sck bits, cpe bits}
 *   out_eff, out_g                   planes of `plane` floats (one plane when hd <= 128, else nsl planes)
 * Returns PA2_OK; PA2_BAD_ARGS for shapes that do not describe step ti; PA2_BAD_FPENV; or PA2_BAD_RECORD when a
 * record names a token >= C, a write >= W, or (valid FIRST / LAST records) a slot or snapshot row out of range: such
 * records are outside the definition (nothing has been written when it is returned, since all records of the step
 * are checked first).
 */
int sdm_pa2_oracle_step(float* grad, float* bank, int64_t slots, const float* snap, int64_t snap_rows, int64_t ssr,
                        const float* du, int64_t ld_u, const float* beta, const int32_t* rec, float* out_eff,
                        float* out_g, int64_t plane, int64_t N, int64_t ti, int64_t P, int64_t C, int64_t W,
                        int64_t hd) {
    if (!grad || !bank || !snap || !du || !beta || !rec || !out_eff || !out_g) return PA2_BAD_ARGS;
    if (N < 1 || P < 1 || P > N || ti < 0 || ti >= N / P) return PA2_BAD_ARGS;
    if (C < 1 || C > 256 || W < 1 || W > 256 || hd < 1 || ld_u < hd || slots < 1 || snap_rows < 0) return PA2_BAD_ARGS;
    const int64_t n = C * W;
    const int64_t nsl = 1 + (hd - 1) / 128;
    const int64_t slw = 4 * (((hd + 3) / 4 + nsl - 1) / nsl);
    if (plane < N * n) return PA2_BAD_ARGS;
    if (!fpenv_ok()) return PA2_BAD_FPENV;

    /* the records of the step must lie inside the definition */
    for (int64_t p = 0; p < P; ++p) {
        const int64_t k = ti * P + p;
        int64_t ordinal = 0;
        for (int64_t j = 0; j < n; ++j) {
            const int32_t* r = rec + (k * n + j) * 4;
            const uint32_t pay = (uint32_t)r[0];
            const int64_t t = (pay >> 9) & 0xFF, w = pay & 0xFF;
            const int valid = !(pay & PA2_INVALID);
            if (t >= C || w >= W) return PA2_BAD_RECORD;
            if (valid && (pay & (PA2_FIRST | PA2_LAST)) && (r[1] < 0 || r[1] >= slots)) return PA2_BAD_RECORD;
            if (valid && (pay & PA2_FIRST)) {
                const int64_t srow = ssr < 0 ? k * n + ordinal : ti * ssr + p * C * W + t * W + w;
                if (srow >= snap_rows) return PA2_BAD_RECORD;
                ++ordinal;
            }
        }
    }

    for (int64_t p = 0; p < P; ++p) {
        const int64_t k = ti * P + p;
        for (int64_t sl = 0; sl < nsl; ++sl) {
            float acc[PA2_SLICE_MAX], gdw[PA2_SLICE_MAX], sn[PA2_SLICE_MAX], x[PA2_SLICE_MAX];
            float gp[PA2_LANES], part[PA2_LANES], tmp[PA2_LANES];
            for (int c = 0; c < PA2_SLICE_MAX; ++c) acc[c] = gdw[c] = sn[c] = 0.0f;
            for (int q = 0; q < PA2_LANES; ++q) gp[q] = 0.0f;
            int64_t ordinal = 0;
            for (int64_t j = 0; j < n; ++j) {
                const int32_t* r = rec + (k * n + j) * 4;
                const uint32_t pay = (uint32_t)r[0];
                const int64_t t = (pay >> 9) & 0xFF, w = pay & 0xFF;
                const int valid = !(pay & PA2_INVALID);
                const float sck = bits_to_float(r[2]), cpe = bits_to_float(r[3]);
                for (int c = 0; c < PA2_SLICE_MAX; ++c) {
                    const int64_t col = sl * slw + c;
                    x[c] = (c < slw && col < hd) ? du[(k * C + t) * ld_u + col] : 0.0f;
                }
                if (pay & PA2_FIRST) {
                    for (int c = 0; c < PA2_SLICE_MAX; ++c) acc[c] = 0.0f;
                    if (valid) {
                        const int64_t srow = ssr < 0 ? k * n + ordinal : ti * ssr + p * C * W + t * W + w;
                        ++ordinal;
                        for (int c = 0; c < PA2_SLICE_MAX; ++c) {
                            const int64_t col = sl * slw + c;
                            const int on = c < slw && col < hd;
                            gdw[c] = on ? grad[(int64_t)r[1] * hd + col] : 0.0f;
                            sn[c] = on ? snap[srow * hd + col] : 0.0f;
                        }
                    } else {
                        for (int c = 0; c < PA2_SLICE_MAX; ++c) gdw[c] = sn[c] = 0.0f;
                    }
                    for (int q = 0; q < PA2_LANES; ++q) gp[q] = lane_dot4(gdw + 4 * q, sn + 4 * q);
                }
                for (int c = 0; c < PA2_SLICE_MAX; ++c) acc[c] = fmaf(sck, x[c], acc[c]);
                for (int q = 0; q < PA2_LANES; ++q) part[q] = lane_dot4(x + 4 * q, sn + 4 * q);
                const float dot = lane_tree(part);
                for (int q = 0; q < PA2_LANES; ++q) tmp[q] = gp[q];
                const float g = lane_tree(tmp);
                if ((pay & PA2_LAST) && valid) {
                    for (int c = 0; c < PA2_SLICE_MAX; ++c) {
                        const int64_t col = sl * slw + c;
                        if (c < slw && col < hd) {
                            grad[(int64_t)r[1] * hd + col] = fmaf(gdw[c], cpe, acc[c]);
                            bank[(int64_t)r[1] * hd + col] = sn[c];
                        }
                    }
                }
                const int64_t o = k * n + t * W + w;
                if (nsl == 1) {
                    out_eff[o] = valid ? (-beta[k * C + t]) * dot : 0.0f;
                    out_g[o] = valid ? cpe * g : 0.0f;
                } else {
                    out_eff[sl * plane + o] = valid ? dot : 0.0f;
                    out_g[sl * plane + o] = valid ? g : 0.0f;
                }
            }
        }
    }
    return PA2_OK;
}
