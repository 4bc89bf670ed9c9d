// smallb.hip -- small-batch dequant-GEMM on MFMA, gfx950.
//
// Same product as gemv.hip (MatGPTQ: Efficient and Accurate Inference over
// Nested Quantized Models, Abstract: kernels supporting batch sizes beyond
// one; Figure 1: batch sweep), for small batches: 16 batch rows per pass over
// the planes, or 32 (two slices) for r <= 4.  Beyond
// one batch row the bf16 dot products would take more VALU issue slots than
// the plane decode itself, so the contraction moves to the matrix cores; the
// product is still bound by HBM, so the kernel streams like the batch-1 one:
//
//  - one v_mfma_f32_16x16x32_bf16 multiplies 32 columns of up to 16 batch
//    rows (A operand) by a 32-column x 16-row weight fragment (B operand).
//    Lane l supplies batch row l%16, k-quarter l/16 of the activations and
//    weight row l%16, k-quarter l/16 of the weights, and ends holding batch
//    rows 4(l/16)..4(l/16)+3 of weight row l%16: one scale per lane and
//    group.  The k-slot order inside a quarter only has to agree between the
//    two operands, so each lane feeds its decoded plane word in the order the
//    decoder produces it (pairs 4j..4j+3 -> MFMA j).
//  - lane (row c, quarter d) of a wave loads the whole 16-byte chunk of row c
//    of group 4*set + d for each plane (one wave load covers the 1 KB of a
//    16-row tile's four groups), and a 4 x 4 transpose across the quarter
//    lanes (v_permlane16_swap, v_permlane32_swap) then leaves in lane (c, d)
//    word d of row c's chunk of every group of the set.  (Loading those words
//    directly takes four times the load instructions, and the texture
//    addresser's time went with the count of instructions, not of bytes.)
//  - a workgroup owns a run of T 16-row tiles and all of k (about one
//    workgroup per CU); its waves split k into 4-group sets (wave w: sets w,
//    w+W, ...).  A wave's steps are (set, tile) pairs, set-major: when a set
//    starts, the wave loads its activation operands (16 batch rows x 512
//    columns per slice, 64 registers per lane), and the planes and scales
//    run PD steps ahead across set boundaries.  Loads are unconditional
//    (clamped at the end), so the loads in flight between a load and its use
//    are a static count.
//  - with two slices (NB = 2), every decoded weight fragment feeds the MFMAs
//    of both, so the plane decode is paid once per 32 batch rows.
//  - every MFMA chain covers one 128-wide group and starts from zero; the
//    group scale is folded in fp32 right after it (one FMA per output), and
//    the corrections that remove the decoded operands' constant offsets
//    enter through one fp32 MFMA per step (corrections x scales over the
//    set's four groups).
//  - each lane adds its four outputs per slice of a step to its own LDS
//    slots for the tile; the waves meet there at the end.
#include <cstdio>

#include "decode.h"
#include "launch.h"

namespace nbw {

constexpr int SMALLB_WAVES = 8;      // waves per workgroup
constexpr int SMALLB_MAX_TILES = 14; // tiles per workgroup
// Activation transpose buffer per wave: 16 batch rows x 256 bytes (one group),
// rows padded to 272 bytes so that both the row-wise writes and the
// column-wise reads hit 16 distinct 16-byte bank groups per 16 lanes.
constexpr int SMALLB_XROW = 272;
constexpr int SMALLB_XBUF = 16 * SMALLB_XROW;
constexpr int SMALLB_DEPTH = 2;      // steps of planes in flight per wave

__device__ __forceinline__ float sb_bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Sum over the four 16-lane rows (lanes l, l^16, l^32, l^48), in every
// lane, as (row0 + row1) + (row2 + row3): one permlane16_swap and one
// permlane32_swap of a value with itself give each lane its partner rows.
__device__ __forceinline__ float sb_cross_row_sum(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t us = __float_as_uint(s);
    const auto b = __builtin_amdgcn_permlane32_swap(us, us, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 4 x 4 transpose across the four 16-lane rows of a wave: on entry, register
// q of lane (c, row d) holds element (d, q); on exit, register q holds
// element (q, d).  permlane16_swap exchanges odd rows of its first operand
// with even rows of its second; permlane32_swap the first operand's upper
// half with the second's lower half.
__device__ __forceinline__ void sb_quad_transpose(uint32_t &r0, uint32_t &r1, uint32_t &r2,
                                                  uint32_t &r3) {
    const auto a = __builtin_amdgcn_permlane16_swap(r0, r1, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(r2, r3, false, false);
    const auto e = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
    const auto f = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
    r0 = e[0];
    r1 = f[0];
    r2 = e[1];
    r3 = f[1];
}

// Dynamic LDS: fp32 [W][T][NB][4][64] partial sums (tile t, batch slice s,
// output v of lane l), then one activation transpose buffer per wave.
__host__ __device__ constexpr size_t smallb_lds_bytes(int waves, int slots, int nb) {
    return (size_t)waves * slots * nb * 4 * 64 * 4 + (size_t)waves * SMALLB_XBUF;
}
// Two 16-row batch slices per workgroup (32 batch rows per pass over the
// planes) for r <= 4 without zero points, when the tile run is at most this
// long (LDS: 2 KB of partial sums per wave and tile).
constexpr int SMALLB_NB2_MAX_TILES = 7;

// grid: (ceil(tiles / tiles_per_wg), ceil(batch / (16 NB))); block 64 * SMALLB_WAVES.
// S4: k/128 is a multiple of 4, so the scales (and zero points) of a row's
// four groups of a set are one aligned 8-byte word.
// NB: 16-row batch slices per workgroup.  Each decoded weight fragment feeds
// the MFMAs of every slice, so the plane decode, the dominant cost, is paid
// once per NB slices.
// One workgroup's work: tile run bx (tiles bx*tiles_per_wg ...) and batch
// pass by of one product.  red: the dynamic LDS, [W][tiles_per_wg][NB][4][64]
// partial sums, then [W] activation buffers.
template <int R, int PD, bool ASYM, bool S4, int NB>
__device__ __forceinline__ void smallb_tiles(
    const uint16_t *__restrict__ x, int64_t batch, int64_t ldx, const uint8_t *__restrict__ planes,
    int64_t plane_bytes, const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    int n, int k, int tiles_total, int tiles_per_wg, float *__restrict__ y, int64_t ldy,
    int ybf16, int bx, int by, float *red) {
    constexpr int NPH = Phases<R>::count;
    const int G = k >> 7;
    const int nsets = (G + 3) >> 2;
    const int W = SMALLB_WAVES;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, d = lane >> 4;
    const int t_begin = bx * tiles_per_wg;
    const int T = min(tiles_per_wg, tiles_total - t_begin);
    const int64_t b0 = (int64_t)by * 16 * NB;

    // This wave's sets: ordinal s = 0 .. my_sets-1 is set w + s*W.
    const int my_sets = nsets > w ? (nsets - w + W - 1) / W : 0;
    float *slot = red + (size_t)w * tiles_per_wg * 256 * NB;
    uint8_t *xbuf = reinterpret_cast<uint8_t *>(red + (size_t)W * tiles_per_wg * 256 * NB) + w * SMALLB_XBUF;
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int q = 0; q < 4 * NB; ++q) slot[(t * 4 * NB + q) * 64 + lane] = 0.f;

    // Step loads: the lane's 16-byte plane chunks (row c, group 4*set + d)
    // and the scales (and zero points) of its output row c for the set's 4
    // groups.  Addresses are a wave-uniform base plus a per-lane 32-bit
    // offset, so the loads take a scalar base and no 64-bit vector adds.
    uint32_t pl[PD][4][R];
    uint32_t sw[PD][2];
    uint32_t zw[ASYM ? PD : 1][2];
    auto load_step = [&](int j, int set, int t) {
        const int tile = t_begin + min(t, T - 1);
        // (scales first: loads retire in issue order, and the plane words,
        // used first, should not be the last ones issued)
        const uint32_t srow = (uint32_t)min(c, n - 1 - 16 * tile) * (uint32_t)G;
        const int64_t sbase = (int64_t)16 * tile * G + 4 * set;
        if constexpr (S4) {
            const uint2 sv = *reinterpret_cast<const uint2 *>(scales + sbase + srow);
            sw[j][0] = sv.x;
            sw[j][1] = sv.y;
            if constexpr (ASYM) {
                const uint2 zv = *reinterpret_cast<const uint2 *>(zeros + sbase + srow);
                zw[j][0] = zv.x;
                zw[j][1] = zv.y;
            }
        } else {
            uint32_t h[4], hz[4];
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                // a group past k gets scale 0: its activations are a repeat
                // of the last group's, not zeros
                const int64_t gb = (int64_t)16 * tile * G + min(4 * set + gi, G - 1);
                h[gi] = 4 * set + gi < G ? scales[gb + srow] : 0u;
                if constexpr (ASYM) hz[gi] = zeros[gb + srow];
            }
            sw[j][0] = h[0] | (h[1] << 16);
            sw[j][1] = h[2] | (h[3] << 16);
            if constexpr (ASYM) {
                zw[j][0] = hz[0] | (hz[1] << 16);
                zw[j][1] = hz[2] | (hz[3] << 16);
            }
        }
        // row c's chunk of group 4*set + d, words q = 0..3 in pl[j][q][p]
        // (transposed across the quarter lanes just before the decode)
        const uint8_t *pbase = planes + ((int64_t)tile * G + 4 * set) * 256;
        const uint32_t poff = (uint32_t)(S4 ? d : min(d, G - 1 - 4 * set)) * 256u + 16u * (uint32_t)c;
#pragma unroll
        for (int p = 0; p < R; ++p) {
            const u32x4_t v =
                __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(pbase + p * plane_bytes + poff));
            pl[j][0][p] = v.x;
            pl[j][1][p] = v.y;
            pl[j][2][p] = v.z;
            pl[j][3][p] = v.w;
        }
    };

    // Activation operands of the current set: XB[sl][gi][4j+e] is the bf16 pair
    // of columns 128g + 32d + 8j + 2e (+1) of batch row b0 + 16 sl + c.
    //
    // The lane needs 64 contiguous bytes of its row per group, but loading
    // them directly puts a wave's 16-byte pieces 64 bytes apart: each
    // instruction then touches 32 cache lines and uses a quarter of each, and
    // the activation loads cost more than the planes.  Instead instruction j
    // of group gi reads 16-byte piece l%16 of batch row 4j + l/16 (four whole
    // rows of the group, 8 full lines), and the wave transposes the pieces
    // through its LDS buffer when the set starts (xstage).
    // (Unconditional loads: batch rows past the end repeat the last row and
    // are never stored; groups past k repeat the last group and have scale 0.
    // A load under a lane condition made the compiler wait for the
    // activations before issuing the plane loads.)
    uint32_t XB[NB][4][16];
    auto load_x = [&](int set) {
#pragma unroll
        for (int sl = 0; sl < NB; ++sl)
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int gc = min(4 * set + gi, G - 1);
                const uint16_t *xg = x + b0 * ldx + 128 * gc;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t row = min((int64_t)(16 * sl + 4 * j + d), batch - 1 - b0);
                    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(xg + row * ldx + 8 * c);
                    XB[sl][gi][4 * j] = v.x;
                    XB[sl][gi][4 * j + 1] = v.y;
                    XB[sl][gi][4 * j + 2] = v.z;
                    XB[sl][gi][4 * j + 3] = v.w;
                }
            }
    };
    // XB[gi][4j..4j+3] holds piece c of row 4j + d; afterwards piece 4d + j of
    // row c.  (In-order LDS access within a wave: no barrier.)
    auto xstage = [&](uint32_t (&xs)[4][16]) {
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<u32x4_t *>(xbuf + (4 * j + d) * SMALLB_XROW + 16 * c) =
                    u32x4_t{xs[gi][4 * j], xs[gi][4 * j + 1], xs[gi][4 * j + 2], xs[gi][4 * j + 3]};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(xbuf + c * SMALLB_XROW + 16 * (4 * d + j));
                xs[gi][4 * j] = v.x;
                xs[gi][4 * j + 1] = v.y;
                xs[gi][4 * j + 2] = v.z;
                xs[gi][4 * j + 3] = v.w;
            }
        }
    };
    // Corrections per batch row and group, formed in the lanes of their own
    // batch row (row c of the slice): cr_d[sl] is the one of group 4*set + d,
    // and for zero points xs_d[sl] the group sum of X.  Each step adds
    // sum_g corr[b][g] * s[row][g] (and the zero-point term) to its outputs
    // with one fp32 MFMA per slice (16x16x4: A = corrections, rows batch, k
    // the set's four groups; B = scales, columns weight rows), so the chains
    // start from zero.
    float cr_d[NB], xs_d[NB];
    // A set's start: its activations into the operand layout, then its
    // corrections (waits for the activations only).
    auto start_set = [&]() {
#pragma unroll
        for (int sl = 0; sl < NB; ++sl) {
            xstage(XB[sl]);
            float cr[4], sx[4];
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                cr[gi] = sb_cross_row_sum(correction<R, 16>(XB[sl][gi]));
                if constexpr (ASYM) {
                    const uint32_t one = 0x3F803F80u;
                    float a = 0.f;
#pragma unroll
                    for (int m = 0; m < 16; ++m)
                        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, one),
                                                            __builtin_bit_cast(bf16x2_t, XB[sl][gi][m]), a, false);
                    sx[gi] = sb_cross_row_sum(a);
                }
            }
            cr_d[sl] = d == 0 ? cr[0] : d == 1 ? cr[1] : d == 2 ? cr[2] : cr[3];
            if constexpr (ASYM) xs_d[sl] = d == 0 ? sx[0] : d == 1 ? sx[1] : d == 2 ? sx[2] : sx[3];
        }
    };

    auto compute = [&](int j, f32x4_t (&out)[NB]) {
        // now pl[j][gi][p] = word d of row c's chunk of group 4*set + gi
#pragma unroll
        for (int p = 0; p < R; ++p) sb_quad_transpose(pl[j][0][p], pl[j][1][p], pl[j][2][p], pl[j][3][p]);
#pragma unroll
        for (int sl = 0; sl < NB; ++sl) out[sl] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            uint32_t D0[16], D1[16];
            decode_word<R>(pl[j][gi], D0, D1);
            // (A group past k has scale 0; rows past n are never stored.)
            const uint32_t word = sw[j][gi >> 1];
            const float sc = sb_bf16_to_f32((gi & 1) ? (word >> 16) : (word & 0xFFFFu));
#pragma unroll
            for (int sl = 0; sl < NB; ++sl) {
                // activations are the A operand (rows: batch), weights the B
                // operand (columns: weight rows): lane (c, d) ends with batch
                // rows 4d..4d+3 of the slice for weight row c
                f32x4_t P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const u32x4_t xb = {XB[sl][gi][4 * jj], XB[sl][gi][4 * jj + 1], XB[sl][gi][4 * jj + 2],
                                        XB[sl][gi][4 * jj + 3]};
                    const u32x4_t a0 = {D0[4 * jj], D0[4 * jj + 1], D0[4 * jj + 2], D0[4 * jj + 3]};
                    P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xb),
                                                                __builtin_bit_cast(bf16x8_t, a0), P, 0, 0, 0);
                    if constexpr (NPH == 2) {
                        const u32x4_t a1 = {D1[4 * jj], D1[4 * jj + 1], D1[4 * jj + 2], D1[4 * jj + 3]};
                        P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xb),
                                                                    __builtin_bit_cast(bf16x8_t, a1), P, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int v = 0; v < 4; ++v) out[sl][v] = fmaf(sc, P[v], out[sl][v]);
            }
        }
        // The set's corrections (and zero-point terms): B = this lane's weight
        // row c, group 4*set + d.
        const uint32_t wd = (d >> 1) ? sw[j][1] : sw[j][0];
        const float s_d = sb_bf16_to_f32((d & 1) ? (wd >> 16) : (wd & 0xFFFFu));
#pragma unroll
        for (int sl = 0; sl < NB; ++sl)
            out[sl] = __builtin_amdgcn_mfma_f32_16x16x4f32(cr_d[sl], s_d, out[sl], 0, 0, 0);
        if constexpr (ASYM) {  // + (127.5 - z) * 2^(R-8) * s * sum of the group's X
            const uint32_t zd = (d >> 1) ? zw[j][1] : zw[j][0];
            const float z = sb_bf16_to_f32((d & 1) ? (zd >> 16) : (zd & 0xFFFFu));
            const float sz = s_d * ((127.5f - z) * (1.0f / (float)(1 << (8 - R))));
#pragma unroll
            for (int sl = 0; sl < NB; ++sl)
                out[sl] = __builtin_amdgcn_mfma_f32_16x16x4f32(xs_d[sl], sz, out[sl], 0, 0, 0);
        }
    };
    // Add a step's outputs (four per slice) to this lane's slots for the
    // tile.  One writer per slot (this lane), so no atomic is needed and the
    // order of the additions is fixed: the wave's first set stores, later sets
    // read, add and store.  (LDS float atomics serialize across the CU: four
    // wave-wide ds_add_f32 per step doubled the kernel's time.)
    auto commit = [&](int si, int t, const f32x4_t (&o)[NB]) {
#pragma unroll
        for (int sl = 0; sl < NB; ++sl)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float *p = &slot[((t * NB + sl) * 4 + v) * 64 + lane];
                if (si == 0)
                    *p = o[sl][v];
                else
                    *p += o[sl][v];
            }
    };

    // The wave's steps are (set ordinal si, tile t), set-major.  Loads run PD
    // steps ahead across set boundaries (past the last step they repeat it);
    // a new set's activations are loaded when its first step comes up.
    const int nsteps = my_sets * T;
    int lsi = 0, lt = 0;  // the next step to load
    auto load_next = [&](int j) {
        const bool past = lsi >= my_sets;
        load_step(j, w + (past ? my_sets - 1 : lsi) * W, past ? T - 1 : lt);
        if (++lt == T) {
            lt = 0;
            ++lsi;
        }
    };
    if (nsteps > 0) {
        load_x(w);
#pragma unroll
        for (int j = 0; j < PD; ++j) {
            // (in order: the loads in flight at the loop top then match the
            // steady state, and the waits there stay partial)
            __builtin_amdgcn_sched_barrier(0);
            load_next(j);
        }
        __builtin_amdgcn_sched_barrier(0);
        start_set();  // (waits for the activations only: they were issued first)
        __builtin_amdgcn_sched_barrier(0);
    }
    int csi = 0, ct = 0;  // the step being computed
    const int nfull = nsteps / PD * PD;
    for (int i0 = 0; i0 < nfull; i0 += PD) {
#pragma unroll
        for (int j = 0; j < PD; ++j) {
            if (ct == 0 && csi > 0) {
                load_x(w + csi * W);
                start_set();
            }
            f32x4_t o[NB];
            compute(j, o);
            load_next(j);  // refill as soon as the buffer is free
            commit(csi, ct, o);
            if (++ct == T) {
                ct = 0;
                ++csi;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < PD; ++j)  // the last < PD steps are already loaded
        if (nfull + j < nsteps) {
            if (ct == 0 && csi > 0) {
                load_x(w + csi * W);
                start_set();
            }
            f32x4_t o[NB];
            compute(j, o);
            commit(csi, ct, o);
            if (++ct == T) {
                ct = 0;
                ++csi;
            }
        }

    // Outputs: add the waves' slots in a fixed order.
    __syncthreads();
    const float post = (float)(1 << (8 - R));
    for (int e = threadIdx.x; e < T * NB * 256; e += blockDim.x) {
        const int ts = e >> 8, v = (e >> 6) & 3, l = e & 63;  // ts = t * NB + slice
        float sum = 0.f;
        for (int ww = 0; ww < W; ++ww) sum += red[((size_t)ww * tiles_per_wg * NB + ts) * 256 + v * 64 + l];
        const int row = 16 * (t_begin + ts / NB) + (l & 15);
        const int64_t b = b0 + 16 * (ts % NB) + 4 * (l >> 4) + v;
        if (row < n && b < batch) store_y(y, ybf16, b * ldy + row, sum * post);
    }
}

template <int R, int PD, bool ASYM, bool S4, int NB>
__global__ __launch_bounds__(64 * SMALLB_WAVES) void smallb_kernel(
    const uint16_t *__restrict__ x, int64_t batch, int64_t ldx, const uint8_t *__restrict__ planes,
    int64_t plane_bytes, const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    int n, int k, int tiles_total, int tiles_per_wg, float *__restrict__ y, int64_t ldy,
    int ybf16) {
    extern __shared__ __align__(16) float red[];
    smallb_tiles<R, PD, ASYM, S4, NB>(x, batch, ldx, planes, plane_bytes, scales, zeros, n, k, tiles_total,
                                      tiles_per_wg, y, ldy, ybf16, blockIdx.x, blockIdx.y, red);
}

// ---------------------------------------------------------------- grouped launch

// Several batch-2..16 products, each with its own r (MatGPTQ: Accurate and
// Efficient Post-Training Matryoshka Quantization, abstract: mixed-precision
// execution over heterogeneous per-layer bit-widths), as one dispatch.
// Workgroup b runs item b; items are numbered product by product, each product
// with its own tile run length.  Eligible: symmetric children, k/128 a
// multiple of 4, dense X and fp32 Y -- the single launch's smallb_kernel<R,
// SMALLB_DEPTH, false, true, 1>, so a grouped product is bit-identical to it.
constexpr int SMALLB_MAX_GROUP = 32;

struct SmallbJob {
    const uint16_t *x;
    const uint8_t *planes;
    int64_t plane_bytes;
    const uint16_t *scales;
    float *y;
    int batch, n, k, r, tiles, tpw, item_begin;
};

struct SmallbGroup {
    SmallbJob job[SMALLB_MAX_GROUP];
    int count;
};

__global__ __launch_bounds__(64 * SMALLB_WAVES) void smallb_group_kernel(SmallbGroup grp) {
    extern __shared__ __align__(16) float red[];
    const int item = blockIdx.x;
    int jb = 0;
    while (jb + 1 < grp.count && item >= grp.job[jb + 1].item_begin) ++jb;
    const SmallbJob &J = grp.job[jb];
    const int bx = item - J.item_begin;
    switch (J.r) {
#define NBW_SMALLB_CASE(RR)                                                                          \
    case RR:                                                                                         \
        smallb_tiles<RR, SMALLB_DEPTH, false, true, 1>(J.x, J.batch, J.k, J.planes, J.plane_bytes,   \
                                                       J.scales, nullptr, J.n, J.k, J.tiles, J.tpw, \
                                                       J.y, J.n, 0, bx, 0, red);                     \
        break;
        NBW_SMALLB_CASE(1)
        NBW_SMALLB_CASE(2)
        NBW_SMALLB_CASE(3)
        NBW_SMALLB_CASE(4)
        NBW_SMALLB_CASE(5)
        NBW_SMALLB_CASE(6)
        NBW_SMALLB_CASE(7)
        NBW_SMALLB_CASE(8)
#undef NBW_SMALLB_CASE
    }
}

// About one workgroup per CU, each owning a run of 16-row tiles.
static int smallb_tpw(const QgemmArgs &a, int cu_count) {
    const int tiles = (a.n + 15) / 16;
    int tpw = (tiles + cu_count / 2) / cu_count;
    if (tpw > SMALLB_MAX_TILES) tpw = SMALLB_MAX_TILES;
    if (tpw < 1) tpw = 1;
    return tpw;
}

// Batch rows per pass over the planes: 32 (two slices per workgroup) where
// the second slice's activations fit in registers (r <= 4) and its partial
// sums in LDS, else 16.
int smallb_pass_rows(int r, int n, int cu_count) {
    QgemmArgs a = {};
    a.n = n;
    return r <= 4 && smallb_tpw(a, cu_count) <= SMALLB_NB2_MAX_TILES ? 32 : 16;
}

static int smallb_nb(int r, const QgemmArgs &a, int cu_count) {
    return a.batch > 16 && smallb_pass_rows(r, a.n, cu_count) == 32 ? 2 : 1;
}

template <int R, bool ASYM, bool S4, int NB>
static void launch_v(const QgemmArgs &a, int cu_count, hipStream_t stream) {
    const int tiles = (a.n + 15) / 16;
    const int tpw = smallb_tpw(a, cu_count);
    dim3 grid((unsigned)((tiles + tpw - 1) / tpw), (unsigned)((a.batch + 16 * NB - 1) / (16 * NB)));
    hipLaunchKernelGGL((smallb_kernel<R, SMALLB_DEPTH, ASYM, S4, NB>), grid, dim3(64 * SMALLB_WAVES),
                       smallb_lds_bytes(SMALLB_WAVES, tpw, NB), stream, a.x, a.batch, a.ldx, a.planes,
                       a.plane_bytes, a.scales, a.zeros, a.n, a.k, tiles, tpw, a.y, a.ldy, a.ybf16);
}

template <int R>
static void launch_r(const QgemmArgs &a, int cu_count, hipStream_t stream) {
    const bool s4 = ((a.k / 128) & 3) == 0;
    if constexpr (R <= 4) {
        if (smallb_nb(R, a, cu_count) == 2) {
            if (a.zeros) {
                if (s4) launch_v<R, true, true, 2>(a, cu_count, stream);
                else launch_v<R, true, false, 2>(a, cu_count, stream);
            } else {
                if (s4) launch_v<R, false, true, 2>(a, cu_count, stream);
                else launch_v<R, false, false, 2>(a, cu_count, stream);
            }
            return;
        }
    }
    if (a.zeros) {
        if (s4) launch_v<R, true, true, 1>(a, cu_count, stream);
        else launch_v<R, true, false, 1>(a, cu_count, stream);
    } else {
        if (s4) launch_v<R, false, true, 1>(a, cu_count, stream);
        else launch_v<R, false, false, 1>(a, cu_count, stream);
    }
}

void smallb_name(int r, const QgemmArgs &a, int cu_count, char *out, size_t len) {
    snprintf(out, len, "nbw::smallb_kernel<%d, %d, %s, %s, %d>", r, SMALLB_DEPTH, a.zeros ? "true" : "false",
             ((a.k / 128) & 3) == 0 ? "true" : "false", smallb_nb(r, a, cu_count));
}

int smallb_group_capacity() { return SMALLB_MAX_GROUP; }

bool smallb_group_eligible(const QgemmArgs &a) {
    return a.batch >= 2 && a.batch <= 16 && ((a.k / 128) & 3) == 0 && !a.zeros && !a.ybf16 &&
           (a.ldx == 0 || a.ldx == a.k) && (a.ldy == 0 || a.ldy == a.n);
}

hipError_t launch_smallb_group(const QgemmArgs *probs, const int *rs, int count, int cu_count,
                               hipStream_t stream) {
    SmallbGroup grp = {};
    grp.count = count;
    int items = 0, slots = 1;
    for (int j = 0; j < count; ++j) {
        const QgemmArgs &a = probs[j];
        SmallbJob &J = grp.job[j];
        J.x = a.x;
        J.planes = a.planes;
        J.plane_bytes = a.plane_bytes;
        J.scales = a.scales;
        J.y = a.y;
        J.batch = (int)a.batch;
        J.n = a.n;
        J.k = a.k;
        J.r = rs[j];
        J.tiles = (a.n + 15) / 16;
        J.tpw = smallb_tpw(a, cu_count);
        if (J.tpw > slots) slots = J.tpw;
        J.item_begin = items;
        items += (J.tiles + J.tpw - 1) / J.tpw;
    }
    hipLaunchKernelGGL(smallb_group_kernel, dim3(items), dim3(64 * SMALLB_WAVES),
                       smallb_lds_bytes(SMALLB_WAVES, slots, 1), stream, grp);
    return hipGetLastError();
}

hipError_t launch_smallb(int r, const QgemmArgs &a, int cu_count, hipStream_t stream) {
    switch (r) {
    case 1: launch_r<1>(a, cu_count, stream); break;
    case 2: launch_r<2>(a, cu_count, stream); break;
    case 3: launch_r<3>(a, cu_count, stream); break;
    case 4: launch_r<4>(a, cu_count, stream); break;
    case 5: launch_r<5>(a, cu_count, stream); break;
    case 6: launch_r<6>(a, cu_count, stream); break;
    case 7: launch_r<7>(a, cu_count, stream); break;
    case 8: launch_r<8>(a, cu_count, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace nbw
