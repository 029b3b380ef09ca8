// Phase A of the deterministic backward step on gfx950: the consumer of the updated d_u.
//
// Operation (page "sparse-delta-memory 2.0.0 -- sparse_delta_memory/cuda/gx_pa2_cuda.py", gx_pa2_kernel, float32
// grad / bank / snapshot rows): for chunk k = ti*P + p and each 128-column slice of the head, the chunk's n = C*W
// records are walked in order. A group opens at a FIRST record (acc = +0; at a valid FIRST the group's grad row gdw
// and snapshot row sn are read, else both are +0); every record adds sck * x to acc with one fmaf per column (x: the
// record's token row of d_u); each record's dot(x, sn) and the group's dot(gdw, sn) are a fmul + 3 fmaf chain over a
// lane's 4 columns followed by the balanced pairwise sum over the slice's 32 lanes (padding lanes and columns +0); a
// valid LAST record stores grad = fmaf(gdw, cpe, acc) and bank = sn; each record writes -beta[t] * dot and cpe * g
// (the raw dot and g into per-slice planes when the head has several slices; +0 for INVALID records).
//
// gfx950 structure:
//   * A wavefront holds two of the page's 32-lane warps: lanes 0-31 are slice 2q's lanes, lanes 32-63 slice 2q+1's
//     (SG = 2), each lane 4 columns, so one record's walk covers 256 columns; with SG = 1 (one slice, or C > 128 where
//     two slices of token rows would not fit in LDS) lanes 32-63 hold no columns.
//   * A workgroup of WAVES wavefronts takes one (chunk, slice pair) and a range of tiles: it stages the chunk's token
//     rows of d_u (C rows of the pair's columns) and its beta values in LDS once; wavefront w walks tile
//     cta*WAVES + w: records [snap_back(tile*L), snap_back((tile+1)*L)), tile boundaries moved back to a group's
//     FIRST through the payload's distance field (the page's snap_back), so every group is walked by one wavefront.
//   * Records are loaded 64 at a time (lane l: record jb + l) and broadcast with readlane. The batch is walked in
//     segments from one FIRST to the next, so a group's grad and snapshot rows stay in the same registers over its
//     records.
//   * A group's grad and snapshot rows are loaded one group ahead (at a batch's start those of its first FIRST, at
//     each FIRST those of the next) through a buffer resource per row, whose range is the row, or empty for an
//     INVALID record or a row index out of range: the loads need no branch and land in fixed registers.
//   * A tile's set-up takes three memory round trips: the first token rows, beta and the payloads at the tile's ends;
//     the snapshot ordinal's inputs and the first record batch, in flight across the staging barrier; the first
//     group's rows.
//   * The 32-lane sums are four DPP adds (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror),
//     after which every lane of a 16-lane row holds the row's sum, and a row_bcast:15 DPP add that joins the lower
//     row's sum to the upper row's. After each xor-butterfly level every lane of an aligned block holds the same block
//     sum, so pairing a lane with any lane of the partner block (the mirrors, the broadcast) gives the page's tree,
//     bit for bit. The sums are read from lanes 31 and 63.
//   * Per record, lane k of the batch collects the record's dot values (readlane, compare and select); each FIRST
//     hands its group's g to the lanes from its own on. Each batch writes its outputs with one store per plane,
//     scattered over the chunk (entry t*W + w); when one workgroup covers the chunk they go to LDS instead, and the
//     workgroup's last wavefront to finish (an LDS count) writes each output plane of the chunk in one contiguous run.
//     That instance is capped at 80 SGPRs, so that a SIMD holds 8 of its wavefronts and a CU's two workgroups run
//     from the start.
//   * Record fields are bounds-checked before any access they steer (token < C, write < W, slot < slots, snapshot
//     row < snap_rows): a record outside the definition gives unspecified values but never reaches outside the
//     buffers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gx_pa2.h"

namespace sdm_gx {
namespace {

constexpr uint32_t kFirst = 0x80000000u;
constexpr uint32_t kLast = 0x40000000u;
constexpr uint32_t kInvalid = 0x00020000u;
constexpr int kDistShift = 18;
constexpr uint32_t kDistMax = 4095u;
constexpr int kBufferFlags = 0x00020000;   // buffer resource word 3: 32-bit data format, untyped dword access

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// the balanced pairwise sum over each 32-lane half, in lane order, held by lanes 16-31 and 48-63 (the upper row of
// each half; the lower rows hold their own 16-lane sums)
__device__ __forceinline__ float tree32(float v) {
    v = v + dpp<0xB1>(v);          // quad_perm [1,0,3,2]: lanes l, l^1
    v = v + dpp<0x4E>(v);          // quad_perm [2,3,0,1]: 2-blocks
    v = v + dpp<0x141>(v);         // row_half_mirror: 4-blocks of an 8-lane half row
    v = v + dpp<0x140>(v);         // row_mirror: 8-blocks of a 16-lane row
    // row_bcast:15 into rows 1 and 3: the lower row's sum (its lane 15) joins the upper row's (16-blocks)
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF,
                                                                     false));
}

__device__ __forceinline__ float lane_value(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// fmul then three fmaf over a lane's 4 columns
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) {
    float s = a.x * b.x;
    s = __builtin_fmaf(a.y, b.y, s);
    s = __builtin_fmaf(a.z, b.z, s);
    s = __builtin_fmaf(a.w, b.w, s);
    return s;
}

// nv (0..4) floats of a row from column position p (4-byte aligned), +0 past them
__device__ __forceinline__ f32x4 load_cols(const float* p, int nv) {
    if (nv == 4) {
        const f32x4u v = *reinterpret_cast<const f32x4u*>(p);
        return f32x4{v.x, v.y, v.z, v.w};
    }
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (nv > 0) v.x = p[0];
    if (nv > 1) v.y = p[1];
    if (nv > 2) v.z = p[2];
    return v;
}

__device__ __forceinline__ void store_cols(float* p, f32x4 v, int nv) {
    if (nv == 4) {
        *reinterpret_cast<f32x4u*>(p) = f32x4u{v.x, v.y, v.z, v.w};
        return;
    }
    if (nv > 0) p[0] = v.x;
    if (nv > 1) p[1] = v.y;
    if (nv > 2) p[2] = v.z;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// 16 bytes at byte offset voff of row `row` of a [rows][hd] array, through a buffer resource of `cols` columns from
// the row's start (0: an empty range). Every dword past the range reads +0 and touches no memory.
__device__ __forceinline__ f32x4 row_load(const float* base, int64_t row, int cols, int hd, int voff) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base) + row * hd, (short)0,
                                                                       cols * 4, kBufferFlags);
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}


// The FIRST position of the group holding position j (0 for j <= 0, n for j >= n), from p = the payload at j (any
// value where j <= 0 or j >= n): the payload's distance field, or for distances of kDistMax and more a scan back 64
// records at a time. Wavefront-uniform.
__device__ __forceinline__ int snap_back(const int32_t* kp, int j, int n, int lane, uint32_t p) {
    if (j <= 0) return 0;
    if (j >= n) return n;
    if (p & kFirst) return j;
    const uint32_t d = (p >> kDistShift) & kDistMax;
    if (d < kDistMax) return j - static_cast<int>(d);
    for (int base = j - static_cast<int>(kDistMax);; base -= 64) {      // ends: q <= 0 holds for every lane at last
        const int q = base - lane;
        const bool f = q <= 0 || (static_cast<uint32_t>(kp[q > 0 ? q : 0]) & kFirst);
        const uint64_t m = __ballot(f);
        if (m) {
            const int r = base - static_cast<int>(__builtin_ctzll(m));
            return r > 0 ? r : 0;
        }
    }
}

// The step for one workgroup. STG: outputs staged in LDS and written out whole at the end; else one store per record
// and plane.
template <int SG, int WAVES, bool STG>
__device__ __forceinline__ void pa2_workgroup(const Pa2Args& a) {
    extern __shared__ f32x4 tok_s[];                   // [C][32 * SG] token rows, beta [C], then (stage_out) the
                                                       // finished-wavefront count and the outputs [np][n]
    float* const beta_s = reinterpret_cast<float*>(tok_s + a.C * 32 * SG);
    uint32_t* const done_s = reinterpret_cast<uint32_t*>(beta_s + a.C);
    float* const out_s = beta_s + a.C + 1;
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int wave = uniform(static_cast<int>(threadIdx.x) >> 6);
    const int half = lane >> 5, hl = lane & 31;
    int b = static_cast<int>(blockIdx.x);
    const int units = a.P * a.npair;                   // (chunk, slice pair) units of the step, cta slowest:
    const int cta = b / units;                         // workgroups are dealt to the 8 XCDs round-robin, so when
    b -= cta * units;                                  // units is a multiple of 8 a chunk's workgroups share one L2
    const int sp = b % a.npair;
    const int p = b / a.npair;
    const int C = a.C, W = a.W, n = a.n, hd = a.hd;
    const int64_t chunk = static_cast<int64_t>(a.ti) * a.P + p;
    const int sl = sp * SG + (SG == 2 ? half : 0);     // this lane's slice
    const bool lane_slice = SG == 2 ? sl < a.nsl : half == 0;
    const int col0 = sl * a.slw + 4 * hl;
    const bool on = lane_slice && 4 * hl < a.slw && col0 < hd;
    const int nv = on ? (hd - col0 < 4 ? hd - col0 : 4) : 0;
    const int tl = SG == 2 ? lane : hl;                // this lane's entry of a token row in LDS
    const int s0 = sp * SG;                            // the workgroup's first slice
    const bool two = a.nsl > 1 && SG == 2 && s0 + 1 < a.nsl;   // outputs of a second slice (planes 2 and 3)

    // Set-up loads in three round trips: (1) the first token rows, beta and the payloads at both tile ends; (2) the
    // snapshot ordinal's block prefix and payloads, and the tile's first record batch, in flight across the staging
    // barrier; (3) after it, the first group's rows.
    const float* rows = a.du + chunk * C * a.ld_u;
    const int32_t* kp = a.kpay + chunk * n;
    const int32_t* rp = a.rec + chunk * n * 4;
    const int tile = cta * WAVES + wave;
    const int64_t t0 = static_cast<int64_t>(tile) * a.L;
    const int j0 = t0 < n ? static_cast<int>(t0) : n, j1 = t0 + a.L < n ? static_cast<int>(t0 + a.L) : n;
    f32x4 v0[4];                                       // this wavefront's first 4 token rows (rows wave + u * WAVES)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int t = wave + u * WAVES;
        v0[u] = on && t < C ? load_cols(rows + static_cast<int64_t>(t) * a.ld_u + col0, nv) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int bi = static_cast<int>(threadIdx.x);      // beta of token bi (C <= 256 <= the workgroup's threads)
    const float bv = bi < C ? a.beta[chunk * C + bi] : 0.f;
    // both payloads in flight at once (clamped reads, no branch: n >= 1)
    const int32_t q0 = kp[j0 < n ? j0 : n - 1], q1 = kp[j1 < n ? j1 : n - 1];
    const uint32_t p0 = static_cast<uint32_t>(uniform(q0)), p1 = static_cast<uint32_t>(uniform(q1));
    const int s = snap_back(kp, j0, n, lane, p0);
    const int e = snap_back(kp, j1, n, lane, p1);
    // stage the chunk's token rows (the pair's columns, +0 past the slice or the head) and beta
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int t = wave + u * WAVES;
        if (t < C && (SG == 2 || half == 0)) tok_s[t * 32 * SG + tl] = v0[u];
    }
    if (bi < C) beta_s[bi] = bv;
    if (STG) {                                         // +0 in every staged output, the count at 0
        for (int i = bi; i < (two ? 4 : 2) * n; i += 64 * WAVES) out_s[i] = 0.f;
        if (bi == 0) *done_s = 0u;
    }
    // dense snapshot rows: the ordinal of the tile's first valid FIRST is the block prefix plus the valid FIRSTs in
    // the block before s
    int bp = 0;
    uint32_t pq = 0u;                                  // payload of record 32 * (s / 32) + lane (masked at use)
    const bool before_s = lane < 32 && 32 * (s >> 5) + lane < s;
    if (a.ssr < 0 && s < e) {                          // (clamped read: s < n; bs <= n / 32)
        const int bs = s >> 5;
        pq = static_cast<uint32_t>(kp[before_s ? 32 * bs + lane : s]);
        bp = a.bpre[chunk * ((n + 31) / 32 + 1) + bs];
    }
    // records jb .. jb + 63 (lane l: record jb + l; 16-byte records, 16-byte aligned: checked on the host). Lanes
    // past the batch (jb + l >= e) read record jb again, a clamped read with no branch; every use of a batch lane is
    // for records below e, so nothing waits for the load until the walk needs it.
    int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
    auto load_batch = [&](int jb) {
        const int4 q = reinterpret_cast<const int4*>(rp)[jb + lane < e ? jb + lane : jb];
        r0 = q.x;
        r1 = q.y;
        r2 = q.z;
        r3 = q.w;
    };
    if (s < e) load_batch(s);
    for (int t = wave + 4 * WAVES; t < C; t += WAVES) {   // the rest of the token rows (C > 4 * WAVES)
        const f32x4 v = on ? load_cols(rows + static_cast<int64_t>(t) * a.ld_u + col0, nv) : f32x4{0.f, 0.f, 0.f, 0.f};
        if (SG == 2 || half == 0) tok_s[t * 32 * SG + tl] = v;
    }
    __syncthreads();
    // With staged outputs each wavefront counts itself done once its LDS output writes have completed; the last one
    // of the workgroup then writes the chunk's outputs out, each plane in one contiguous run.
    auto arrive = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0): this wavefront's output writes are in LDS
        uint32_t prev = 0u;
        if (lane == 0) prev = __hip_atomic_fetch_add(done_s, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(prev), 0)) != WAVES - 1) return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        const int64_t ob = chunk * n;
        float* const e0 = a.out_eff + (a.nsl == 1 ? 0 : s0 * a.plane) + ob;
        float* const g0 = a.out_g + (a.nsl == 1 ? 0 : s0 * a.plane) + ob;
        for (int i = lane; i < n; i += 64) {
            e0[i] = out_s[i];
            g0[i] = out_s[n + i];
        }
        if (two)
            for (int i = lane; i < n; i += 64) {
                e0[a.plane + i] = out_s[2 * n + i];
                g0[a.plane + i] = out_s[3 * n + i];
            }
    };
    if (s >= e) {                                      // no barrier follows
        if (STG) arrive();
        return;
    }
    asm volatile("" : "+v"(pq));                       // the ordinal's payload is examined here, not at its load
    int gw = 0;
    if (a.ssr < 0) {
        const uint64_t before = __ballot(before_s && (pq & kFirst) && !(pq & kInvalid));
        gw = uniform(bp + static_cast<int>(__builtin_popcountll(before)));
    }
    const int64_t srow_base = a.ssr < 0 ? chunk * n : static_cast<int64_t>(a.ti) * a.ssr + static_cast<int64_t>(p) * n;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, gdw = {0.f, 0.f, 0.f, 0.f}, sn = {0.f, 0.f, 0.f, 0.f};
    f32x4 pg = {0.f, 0.f, 0.f, 0.f}, ps = {0.f, 0.f, 0.f, 0.f};   // the next group's grad and snapshot columns
    float g = 0.f;                                     // the group's dot(gdw, sn): lanes 16-31 slice A, 48-63 slice B
    const int voff = on ? col0 * 4 : 0x7FFFFFF0;       // this lane's byte offset in a row; past any row when off
    const int64_t obase = chunk * n;
    for (int jb = s; jb < e; jb += 64) {
        const int nrec = e - jb < 64 ? e - jb : 64;
        if (jb != s) load_batch(jb);
        // The batch is needed at once. Waiting for it here, outside the record loop, keeps the compiler from placing
        // that wait at the loop's head, where it would also wait for every store of the records before.
        __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)
        const uint64_t fm = __ballot(lane < nrec && (static_cast<uint32_t>(r0) & kFirst));   // the batch's FIRSTs
        // Lane l collects record jb + l's dot values and its group's g (the group open at the batch start for the
        // records before the batch's first FIRST; each FIRST takes over the lanes from its own on).
        float effA = 0.f, effB = 0.f;
        float gA = lane_value(g, 31), gB = lane_value(g, 63);
        // the records k0 .. k1 - 1 of one group
        auto walk = [&](int k0, int k1) {
            for (int k = k0; k < k1; ++k) {
                const uint32_t pay = static_cast<uint32_t>(__builtin_amdgcn_readlane(r0, k));
                int tok = static_cast<int>((pay >> 9) & 0xFFu);
                tok = tok < C ? tok : C - 1;
                const float sck = __builtin_bit_cast(float, __builtin_amdgcn_readlane(r2, k));
                // +0 for lanes off the head (staged so); with one slice per wavefront, lanes 32-63 read lanes 0-31's
                // entries and their results are never used
                const f32x4 x = tok_s[tok * 32 * SG + tl];
                acc.x = __builtin_fmaf(sck, x.x, acc.x);
                acc.y = __builtin_fmaf(sck, x.y, acc.y);
                acc.z = __builtin_fmaf(sck, x.z, acc.z);
                acc.w = __builtin_fmaf(sck, x.w, acc.w);
                const float dot = tree32(dot4(x, sn));
                if ((pay & kLast) && !(pay & kInvalid)) {
                    const int64_t slot = __builtin_amdgcn_readlane(r1, k);
                    const float cpe = __builtin_bit_cast(float, __builtin_amdgcn_readlane(r3, k));
                    if (on && slot >= 0 && slot < a.slots) {
                        f32x4 o;
                        o.x = __builtin_fmaf(gdw.x, cpe, acc.x);
                        o.y = __builtin_fmaf(gdw.y, cpe, acc.y);
                        o.z = __builtin_fmaf(gdw.z, cpe, acc.z);
                        o.w = __builtin_fmaf(gdw.w, cpe, acc.w);
                        store_cols(a.grad + slot * hd + col0, o, nv);
                        store_cols(a.bank + slot * hd + col0, sn, nv);
                    }
                }
                const float dA = lane_value(dot, 31), dB = lane_value(dot, 63);
                if (lane == k) {
                    effA = dA;
                    effB = dB;
                }
            }
        };
        // The rows a FIRST record opens its group with are loaded one group ahead: at the batch start those of its
        // first FIRST, at each FIRST those of the next one, while the group is walked. Each row is read through a
        // buffer resource spanning its hd columns (none for an INVALID record or a row out of range), so lanes past
        // the head or the row's end, and records without rows, read +0 with no branch, and the loads are unconditional.
        auto fetch = [&](int k2) {                     // the rows of the batch's FIRST record k2 (k2 >= nrec: none)
            bool use = false;
            int64_t slot = 0, srow = 0;
            if (k2 < nrec) {
                const uint32_t pay = static_cast<uint32_t>(__builtin_amdgcn_readlane(r0, k2));
                use = !(pay & kInvalid);
                slot = __builtin_amdgcn_readlane(r1, k2);
                srow = a.ssr < 0 ? srow_base + gw
                                 : srow_base + static_cast<int64_t>((pay >> 9) & 0xFFu) * W + (pay & 0xFFu);
            }
            const bool gok = use && slot >= 0 && slot < a.slots, sok = use && srow >= 0 && srow < a.snap_rows;
            pg = row_load(a.grad, gok ? slot : 0, gok ? hd : 0, hd, voff);
            ps = row_load(a.snap, sok ? srow : 0, sok ? hd : 0, hd, voff);
        };
        const int kf = fm ? static_cast<int>(__builtin_ctzll(fm)) : nrec;
        fetch(kf);
        walk(0, kf);                                   // the group open at the batch start
        for (int k = kf; k < nrec;) {                  // from each FIRST to the record before the next one
            const uint32_t pay = static_cast<uint32_t>(__builtin_amdgcn_readlane(r0, k));
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
            gdw = pg;
            sn = ps;
            if (!(pay & kInvalid)) ++gw;
            const uint64_t later = k >= 63 ? 0ull : fm & (~0ull << (k + 1));
            const int kend = later ? static_cast<int>(__builtin_ctzll(later)) : nrec;
            fetch(kend);
            g = tree32(dot4(gdw, sn));
            const float g0 = lane_value(g, 31), g1 = lane_value(g, 63);
            if (lane >= k) {
                gA = g0;
                gB = g1;
            }
            walk(k, kend);
            k = kend;
        }
        // outputs of records jb .. jb + nrec - 1 (lane l: record jb + l)
        if (lane < nrec) {
            const uint32_t pay = static_cast<uint32_t>(r0);
            const int tok = static_cast<int>((pay >> 9) & 0xFFu), w = static_cast<int>(pay & 0xFFu);
            if (tok < C && w < W) {
                const bool valid = !(pay & kInvalid);
                const int64_t o = obase + static_cast<int64_t>(tok) * W + w;
                const int so = tok * W + w;
                if (STG) {
                    out_s[so] = valid ? (a.nsl == 1 ? (-beta_s[tok]) * effA : effA) : 0.f;
                    out_s[n + so] = valid ? (a.nsl == 1 ? __builtin_bit_cast(float, r3) * gA : gA) : 0.f;
                    if (two) {
                        out_s[2 * n + so] = valid ? effB : 0.f;
                        out_s[3 * n + so] = valid ? gB : 0.f;
                    }
                } else if (a.nsl == 1) {
                    a.out_eff[o] = valid ? (-beta_s[tok]) * effA : 0.f;
                    a.out_g[o] = valid ? __builtin_bit_cast(float, r3) * gA : 0.f;
                } else {
                    a.out_eff[s0 * a.plane + o] = valid ? effA : 0.f;
                    a.out_g[s0 * a.plane + o] = valid ? gA : 0.f;
                    if (two) {
                        a.out_eff[(s0 + 1) * a.plane + o] = valid ? effB : 0.f;
                        a.out_g[(s0 + 1) * a.plane + o] = valid ? gB : 0.f;
                    }
                }
            }
        }
    }
    if (STG) arrive();
}

template <int SG, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gx_pa2_kernel(const Pa2Args a) {
    pa2_workgroup<SG, WAVES, false>(a);
}

// With every output plane of a chunk in LDS, 80 SGPRs (some spilled to VGPR lanes) let a SIMD hold 8 of these
// wavefronts, so both workgroups of a CU run from the start; at 90 and more it holds 7.
template <int SG, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_num_sgpr(80))) void gx_pa2_staged_kernel(
    const Pa2Args a) {
    pa2_workgroup<SG, WAVES, true>(a);
}

}  // namespace

const void* find_pa2_kernel(int slices_per_wave, int waves, bool staged) {
#define SDM_PA2_K(SG, WV)                                                                                  \
    if (slices_per_wave == SG && waves == WV)                                                              \
        return staged ? reinterpret_cast<const void*>(&gx_pa2_staged_kernel<SG, WV>)                       \
                      : reinterpret_cast<const void*>(&gx_pa2_kernel<SG, WV>);
    SDM_PA2_K(1, 4) SDM_PA2_K(1, 8) SDM_PA2_K(1, 16) SDM_PA2_K(2, 4) SDM_PA2_K(2, 8) SDM_PA2_K(2, 16)
#undef SDM_PA2_K
    return nullptr;
}

}  // namespace sdm_gx
