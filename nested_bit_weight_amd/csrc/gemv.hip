// gemv.hip -- streaming dequant-GEMV for batch 1..4, gfx950, single and
// grouped launches.
//
// y[b][i] = sum_j x[b][j] * s[i][j/128] * 2^(8-r) * (q_r[i][j] + 1/2 - 2^(r-1)),
// the r-bit child of a sliceable parent (MatGPTQ: Efficient and Accurate
// Inference over Nested Quantized Models, Abstract: lower precisions read
// fewer bits of the weights; Figure 1: the kernels run at 2..8 bits).  The
// grouped launch runs several such products -- say all linears of a decoder
// layer, each with its own r (MatGPTQ: Accurate and Efficient Post-Training
// Matryoshka Quantization, abstract: mixed-precision execution) -- as one
// dispatch.
//
// At batch 1 the product is bound by HBM (r/8 bytes of planes per weight, one
// multiply-add per weight) and, at r <= 3, nearly as much by the VALU issue
// rate of the decode; up to four batch rows share one decode (below).  The
// layout of the work:
//
//  - a workgroup owns a range of T 16-row tiles of one product and all of k;
//    its W waves split k into 4-group sets (wave w: sets w, w+W, ...).
//  - lane (i, gg) of a wave holds row i of the tile and group 4*set+gg: the
//    wave's four 16-lane quarters read 4 x 256 contiguous plane bytes per
//    plane and tile with 128-bit loads.
//  - each wave walks its (set, tile) steps as one stream with PD steps of
//    planes and scales in flight; the loads are unconditional (clamped at
//    the end; on long tile runs a set's X comes with its first tile only),
//    so the loads-in-flight count between a load and its use is static, and
//    every address is a scalar base plus a fixed lane offset.
//  - the activations are staged in LDS by each wave for its set, in a layout
//    free of bank conflicts; a set switch reloads the lane's MFMA operand
//    from LDS without touching the memory pipeline.
//  - decode: bit-plane transpose network + one shift / and-or per bf16 pair
//    (decode.h) on the VALU; the products on the matrix cores, with a block
//    diagonal activation operand that keeps the set's four groups -- of up
//    to four batch rows -- in separate output rows (see gemv_tiles); the
//    group scales are folded in fp32 once per (row, group), and the waves
//    meet in LDS in a fixed order.
#include <algorithm>
#include <cstdio>

#include "decode.h"
#include "launch.h"

namespace nbw {


constexpr int GEMV_MAX_WAVES = 8;   // waves per workgroup
constexpr int GEMV_ODD_WAVES = 4;   // waves per workgroup of the odd-group-count kernel
constexpr int GEMV_MAX_TILES = 16;  // tiles per workgroup
constexpr int GEMV_MAX_GROUP = 32;  // products per grouped launch
// Workgroups per CU the launch plans for.  (Measured on 70B- and
// Llama-3.1-8B-sized linears: two workgroups per CU, with the MFMA operand
// read from LDS to fit the registers, were 5-15% slower than one.)
constexpr int GEMV_WGS_PER_CU = 1;

// Steps a wave keeps in flight (prefetch depth).  Every wave of the grid
// prefetches this many steps at once, so the total in flight must stay near
// what HBM delivers in one memory latency, not a large share of the matrix:
// a deeper queue only delays each wave's first step.  Waves with only a few
// steps take depth 1 (a second buffer would hold repeats of the last step).
// (Measured on 70B- and Qwen3-8B-sized linears: depth 3 or 4 at r = 2, 3 is
// slower than 2; at r = 6 depth 2 beats 1 by 7%.)
constexpr int GEMV_DEPTH_SHORT = 1;
__host__ __device__ constexpr int gemv_depth(int r) { return r <= 6 ? 2 : 1; }

// Batch rows one launch of the streaming kernel takes: 1, or up to 4 (the
// batch rows fill the rows of the MFMA's activation operand that batch 1
// leaves at zero; see gemv_tiles).
constexpr int GEMV_MAX_BATCH = 4;

// Dynamic LDS: per wave, one set of X for each of the NBR batch rows (4
// groups x 128 bf16 a row, each group padded by 16 bytes) and a run of zeros,
// then the partial sums fp32 [W][slots][16 NBR], one slot per tile.
// In one A-operand load a few lanes of each quarter read a group and the rest
// read zeros; quarter g's zero lanes read at offset 4 g + 8 of the zero run.
// Bank offsets (words mod 64, and mod 32):
//  - NBR = 4: groups 68 words apart, rows 272: group g of row b at 16 b + 4 g,
//    so the four active lanes of quarter g (rows 0..3 of group g) hit
//    4 g + 16 b, none of them at 4 g + 8; the correction reads (lane (i, b):
//    word i + 16 q of group v of row b) hit 16 b + 4 v + i, distinct.
//  - NBR = 1: groups 80 words apart: the active lane of quarter g reads at
//    16 g, its zero lanes at 4 g + 8; the correction reads (lane (i, g): word
//    i + 16 q of group g) hit 16 g + i, distinct.
// (A shared zero block at one offset made every A-operand load of a set
// switch conflict.)
__host__ __device__ constexpr int gemv_xgroup(int nbr) { return nbr > 1 ? 68 : 80; }  // words
__host__ __device__ constexpr int gemv_xrow(int nbr) { return 4 * gemv_xgroup(nbr); }
__host__ __device__ constexpr int gemv_round64(int v) { return (v + 63) / 64 * 64; }
// zero run (words from the wave's base; a multiple of 64): 8 + 12 + 64 words used
__host__ __device__ constexpr int gemv_zoff(int nbr) { return gemv_round64(gemv_xrow(nbr) * nbr); }
__host__ __device__ constexpr int gemv_wave_lds(int nbr) { return 4 * gemv_round64(gemv_zoff(nbr) + 96); }
__host__ __device__ constexpr size_t gemv_lds_bytes(int waves, int slots, int nbr) {
    return (size_t)waves * gemv_wave_lds(nbr) + (size_t)waves * slots * 16 * nbr * 4;
}

// Sum over each 16-lane row of the wave, in every lane of the row: DPP quad
// permutes [1,0,3,2] and [2,3,0,1], then row_half_mirror (lane i of each
// half-row reads lane 7-i: the other quad) and row_mirror (lane i reads
// lane 15-i: the other half).  VALU only, no LDS round trip.  Each add sums
// two equal partial sums in swapped order, so every lane of the row ends
// with the same bits -- provided no add is fused with a product that made
// its input (the fused lane would keep the unrounded product while its
// partner adds the rounded one), hence no contraction here.
__device__ __forceinline__ float row16_sum(float v) {
#pragma clang fp contract(off)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// A wave-uniform global address, pinned to scalar registers: a load from it
// plus a 32-bit lane offset then takes the scalar-base addressing form (no
// 64-bit vector address arithmetic), which the compiler otherwise loses when
// it folds the lane offset in before a uniform plane offset.  Loads go
// through global (address space 1) pointers, not flat ones.
template <class T> using gptr = const __attribute__((address_space(1))) T *;
__device__ __forceinline__ uint64_t uniform_addr(const void *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float lane_value(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// One workgroup: tiles [t_begin, t_begin + T) of one product, all of k;
// `slots` partial-sum slots per wave in LDS (T <= slots).  k/128 is a
// multiple of 4: a set is four whole groups.
//
// The dot products run on the matrix cores, the decode on the VALU.  One
// v_mfma_f32_16x16x32_bf16 takes 32 columns: lane (i, h) of the wave (i =
// lane % 16, h = lane / 16) supplies 8 decoded weights of row i, group
// 4*set + h (B operand) and, as row i of the A operand, the same 8 columns
// of batch row i / 4's X if i % 4 == h and zeros otherwise.  Row 4b + v of A
// thus holds only batch row b's group 4*set + v, and so does output row
// 4b + v: after the 16 MFMAs of a step (4 words x 4 pair quads), lane
// (i, b) holds weight row i's four group sums for batch row b in its four
// accumulator registers, and scales them there.  At batch 1 (NBR = 1) rows
// 4..15 of A are zero: the matrix cores are otherwise idle, and up to four
// batch rows cost the same MFMAs and the same decode as one.  Each batch
// row's sums are formed exactly as at batch 1 (one row of A, the same
// summation order), so the results do not depend on NBR.
//
// Waves are independent until the final reduction: a wave loads the X of its
// current set itself (one 16-byte load per lane, part of the step's load
// stream), stages it in its own 1 KB of LDS and reads back its lanes' A
// operands, so no barrier -- and no wait for every load in flight -- stands
// between a wave's first loads and its first step.
//
// XO: load a set's X only with its first tile (runs of 3 or more tiles per
// workgroup, where the reloads' memory-pipe traffic costs more than the
// looser load-wait counts that a conditional load leaves).
template <int R, int PD, bool ASYM, int NBR, bool XO>
__device__ __forceinline__ void gemv_tiles(const uint16_t *__restrict__ x, int64_t ldx, int batch,
                                           const uint8_t *__restrict__ planes,
                                           int64_t plane_bytes,
                                           const uint16_t *__restrict__ scales,
                                           const uint16_t *__restrict__ zeros, int n, int k,
                                           int t_begin, int T, int slots, float *__restrict__ y,
                                           int64_t ldy, int ybf16, unsigned char *lds) {
    static_assert(NBR == 1 || NBR == GEMV_MAX_BATCH, "one batch row, or up to four");
    constexpr int NPH = Phases<R>::count;
    constexpr int RW = 16 * NBR;  // partial sums per slot
    const int G = k >> 7;
    const int nsets = (G + 3) >> 2;
    const int W = blockDim.x >> 6;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int i = lane & 15, gg = lane >> 4;
    // this wave's set of X, group g of batch row b at xw + XROW b + XGROUP g;
    // then the zero run, read by quarter g at offset 4 g + 8
    constexpr int XGROUP = gemv_xgroup(NBR), XROW = gemv_xrow(NBR);
    uint32_t *xw = reinterpret_cast<uint32_t *>(lds + (size_t)w * gemv_wave_lds(NBR));
    uint32_t *zrun = xw + gemv_zoff(NBR);
    const uint32_t *zblk = zrun + 8 + 4 * gg;
    float *red = reinterpret_cast<float *>(lds + (size_t)W * gemv_wave_lds(NBR));  // [W][slots][RW]

    // This wave's (set, tile) steps: set ordinal s = 0 .. my_sets-1 is set
    // w + s*W, tile t = 0 .. T-1; step u = s*T + t.
    const int my_sets = nsets > w ? (nsets - w + W - 1) / W : 0;
    const int U = my_sets * T;

    // Step loads: R plane chunks (row i, group 4*set + gg), the two aligned
    // 32-bit words of the scales of row i's four groups of the set, and the
    // lane's 16 bytes of the set's X of each batch row (the same chunks for
    // every tile of a set; batch rows past the last repeat it).  Unless XO,
    // all loads are unconditional (X reloaded with every tile, steps past the
    // end clamped), so the loads-in-flight count between a load and its use
    // is static.
    u32x4_t buf[PD][R];
    u32x4_t xbuf[PD][NBR];
    u32x2_t sbuf[PD];
    u32x2_t zbuf[ASYM ? PD : 1];
    int ps = 0, pt = 0;  // next step to prefetch
    // Every address of a step is a wave-uniform base (scalar arithmetic) plus
    // a per-lane offset fixed for the whole kernel: with k/128 a multiple of
    // 4, the chunk of (row i, group 4*set + gg) of a tile lies lane*16 bytes
    // into the tile's run of the set's chunks, and the lane's X lies lane*16
    // bytes into the set's 1 KB.  Only the scales' row needs a clamp (the
    // padding rows of a ragged last tile read row n-1's, and are dropped).
    const uint32_t lane16 = (uint32_t)lane * 16u;
    const uint32_t srow = (uint32_t)i * (uint32_t)G * 2u;  // row i's scales, bytes into a tile's
    auto load_step = [&](int j) {
        int s = ps, t = pt;
        if (s >= my_sets) {
            s = my_sets - 1;
            t = T - 1;
        }
        const int set = w + s * W;
        const int tile = t_begin + t;
        // (a fresh copy of the lane offset in each step: the compiler
        // otherwise hoists its 64-bit extension out of the loop and then
        // adds it to the base with vector arithmetic)
        uint32_t lo16 = lane16;
        asm volatile("" : "+v"(lo16));
#pragma unroll
        for (int b = 0; b < NBR; ++b) {
            const uint64_t xs = uniform_addr(reinterpret_cast<const uint8_t *>(x + (int64_t)min(b, batch - 1) * ldx) +
                                             (int64_t)set * 1024);
            if (!XO || t == 0) xbuf[j][b] = *(gptr<u32x4_t>)(xs + lo16);
        }
        const uint8_t *c = planes + ((int64_t)tile * G + 4 * set) * 256;
#pragma unroll
        for (int p = 0; p < R; ++p)
            buf[j][p] = __builtin_nontemporal_load((gptr<u32x4_t>)(uniform_addr(c + (int64_t)p * plane_bytes) + lo16));
        // groups 4*set .. 4*set+3 of row min(16 tile + i, n - 1): one aligned
        // 8-byte word
        const int64_t sb = ((int64_t)16 * tile * G + 4 * set) * 2;
        const uint32_t so = min(srow, (uint32_t)(n - 1 - 16 * tile) * (uint32_t)G * 2u);
        sbuf[j] = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint8_t *>(scales) + sb + so);
        if constexpr (ASYM)
            zbuf[j] = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint8_t *>(zeros) + sb + so);
        if (++pt == T) {
            pt = 0;
            ++ps;
        }
    };
    if (U > 0) {  // (first: everything below waits for nothing)
#pragma unroll
        for (int j = 0; j < PD; ++j) load_step(j);
    }

    // The zero run, and the partial sums of a wave without steps (any other
    // wave stores every slot of its own with its first set; only this wave
    // writes them until the final barrier).
    zrun[lane] = 0u;
    if (lane < 32) zrun[64 + lane] = 0u;
    if (U == 0 && (NBR > 1 || gg == 0))
        for (int t = 0; t < T; ++t) red[(w * slots + t) * RW + (NBR > 1 ? lane : i)] = 0.f;

    // Coefficient of this lane's pair sums in the group correction
    // sum_k x_k * (1/2 - 2^(R-1) - offset_k): lane (i, gg) takes the pairs
    // i, i+16, i+32, i+48 of its group, which share one offset.
    float my_coef = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m)
        if (i == m) my_coef = pair_coef<R>(m);

    uint32_t X2[64];  // A operand: group gg of batch row i / 4's X if i % 4 == gg, else zeros
    // the set's group corrections and group sums of X (asymmetric term), for
    // the batch row of the lane's outputs (wave-uniform at NBR = 1)
    float corr[4] = {0.f, 0.f, 0.f, 0.f};
    float sgv[4] = {0.f, 0.f, 0.f, 0.f};
    int cs = 0, ct = 0;  // step being computed
    auto compute = [&](int j) {
        const int set = w + cs * W;
        if (ct == 0) {
            // New set: stage its X (LDS operations of one wave complete in
            // order, so the previous set's reads are done), read back this
            // lane's A operand, and form each group's correction over 16
            // lanes (lane i takes the pairs i, i+16, i+32, i+48 of a group).
#pragma unroll
            for (int b = 0; b < NBR; ++b)  // (lane l holds words 4l..4l+3 of the set: group l / 16)
                *reinterpret_cast<u32x4_t *>(xw + XROW * b + XGROUP * gg + 4 * i) = xbuf[j][b];
            const uint32_t *src = (NBR > 1 ? (i & 3) == gg : i == gg)
                                      ? xw + XROW * (i >> 2) + XGROUP * gg : zblk;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const u32x4_t v = reinterpret_cast<const u32x4_t *>(src)[q];
                X2[4 * q] = v.x; X2[4 * q + 1] = v.y; X2[4 * q + 2] = v.z; X2[4 * q + 3] = v.w;
            }
            const uint32_t one = 0x3F803F80u;  // bf16 (1.0, 1.0)
            if constexpr (NBR == 1) {
                // quarter gg forms group gg's sums; every lane takes all four
                float sx = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) sx = dot2(one, xw[XGROUP * gg + i + 16 * q], sx);
                const float cg = row16_sum(my_coef * sx);
                float sg = 0.f;
                if constexpr (ASYM) sg = row16_sum(sx);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    corr[v] = lane_value(cg, 16 * v);
                    if constexpr (ASYM) sgv[v] = lane_value(sg, 16 * v);
                }
            } else {
                // quarter gg forms the four group sums of batch row gg, the
                // row of its outputs
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float sx = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        sx = dot2(one, xw[XROW * gg + XGROUP * v + i + 16 * q], sx);
                    corr[v] = row16_sum(my_coef * sx);
                    if constexpr (ASYM) sgv[v] = row16_sum(sx);
                }
            }
        }
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t Pw[R];
#pragma unroll
            for (int p = 0; p < R; ++p) Pw[p] = buf[j][p][d];
            uint32_t D0[16], D1[16];
            decode_word<R>(Pw, D0, D1);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4_t a = {X2[16 * d + 4 * c], X2[16 * d + 4 * c + 1], X2[16 * d + 4 * c + 2],
                                   X2[16 * d + 4 * c + 3]};
                const u32x4_t b0 = {D0[4 * c], D0[4 * c + 1], D0[4 * c + 2], D0[4 * c + 3]};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                              __builtin_bit_cast(bf16x8_t, b0), acc, 0, 0, 0);
                if constexpr (NPH == 2) {
                    const u32x4_t b1 = {D1[4 * c], D1[4 * c + 1], D1[4 * c + 2], D1[4 * c + 3]};
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                                  __builtin_bit_cast(bf16x8_t, b1), acc, 0, 0, 0);
                }
            }
        }
        // lane (i, b): acc[v] = group 4*set + v of weight row i for batch
        // row b (at NBR = 1 the lanes of quarters 1..3 hold the zero rows of
        // A; batch rows past the last are computed and dropped)
        // (rows past n of a ragged last tile carry row n-1's scales and are
        // never stored)
        float out = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const uint32_t wd = (v >> 1) ? sbuf[j].y : sbuf[j].x;
            const uint32_t sbits = (v & 1) ? (wd & 0xFFFF0000u) : (wd << 16);
            const float s = __uint_as_float(sbits);
            float term = acc[v] + corr[v];
            if constexpr (ASYM) {
                // asymmetric child = symmetric child + s * (127.5 - z) per
                // weight; in the units of acc (scaled by 2^(8-R) at the end):
                const uint32_t zw = (v >> 1) ? zbuf[j].y : zbuf[j].x;
                const uint32_t zbits = (v & 1) ? (zw & 0xFFFF0000u) : (zw << 16);
                const float zc = (127.5f - __uint_as_float(zbits)) * (1.0f / (float)(1 << (8 - R)));
                term = fmaf(zc, sgv[v], term);
            }
            out = fmaf(s, term, out);
        }
        return out;
    };
    // Accumulate into this output's own LDS slot for the tile.  Each slot
    // has a single writer (lane i of quarter 0 at NBR = 1, else every lane),
    // so no atomic is needed and the order of the additions is fixed: the
    // wave's first set stores, later sets read, add and store.
    auto commit = [&](float v) {
        if (NBR > 1 || gg == 0) {
            float *slot = &red[(w * slots + ct) * RW + (NBR > 1 ? lane : i)];
            if (cs == 0)
                *slot = v;
            else
                *slot += v;
        }
        if (++ct == T) {
            ct = 0;
            ++cs;
        }
    };

    const int Ufull = U / PD * PD;
    for (int u0 = 0; u0 < Ufull; u0 += PD) {
#pragma unroll
        for (int j = 0; j < PD; ++j) {
            const float v = compute(j);
            // The refill goes after every use of the buffer's registers: a
            // load issued while the old value is still to be read would need
            // a second register, and the copy between the two at the loop's
            // back edge would wait for every load in flight.  (The empty asm
            // keeps the step's result -- and its reads of the scales -- here,
            // instead of sunk into the branch of the lanes that store it.)
            asm volatile("" : : "v"(v));
            __builtin_amdgcn_sched_barrier(0);
            load_step(j);  // refill as soon as the buffer is free
            commit(v);
            // Keep the next step's uses of the refilled registers in the next
            // step, so the wait for them stays PD - 1 steps deep.
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int j = 0; j < PD; ++j)  // the last < PD steps are already loaded
        if (Ufull + j < U) commit(compute(j));

    // Outputs: add the waves, in a fixed order.
    __syncthreads();
    const float post = (float)(1 << (8 - R));
    for (int e = threadIdx.x; e < T * RW; e += blockDim.x) {
        const int t = e / RW, l = e % RW;
        const int b = l >> 4, row = 16 * (t_begin + t) + (l & 15);
        float sum = 0.f;
        for (int ww = 0; ww < W; ++ww) sum += red[(ww * slots + t) * RW + l];
        if (row < n && b < batch) store_y(y, ybf16, (int64_t)b * ldy + row, sum * post);
    }
}

// Group counts that are not multiples of 4 (k = 128 * g, g % 4 != 0) would
// need narrower scale loads; these rare shapes take this plain one-tile
// kernel: one workgroup per 16-row tile.
template <int R>
__global__ __launch_bounds__(256) void gemv_odd_kernel(const uint16_t *__restrict__ x,
                                                       const uint8_t *__restrict__ planes,
                                                       int64_t plane_bytes,
                                                       const uint16_t *__restrict__ scales,
                                                       const uint16_t *__restrict__ zeros,
                                                       int n, int k, float *__restrict__ y,
                                                       int ybf16) {
    __shared__ float red[GEMV_ODD_WAVES][16];
    const int G = k >> 7;
    const int W = blockDim.x >> 6;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = lane & 15, gg = lane >> 4;
    const int tile = blockIdx.x;
    const int row = 16 * tile + i;
    float acc = 0.f;
    for (int g = 4 * w + gg; g - gg < G; g += 4 * W) {
        const bool gvalid = g < G;
        const int gc = gvalid ? g : G - 1;
        const uint8_t *c = planes + (((int64_t)tile * G + gc) * 16 + i) * 16;
        u32x4_t pl[R];
#pragma unroll
        for (int p = 0; p < R; ++p) pl[p] = *reinterpret_cast<const u32x4_t *>(c + p * plane_bytes);
        uint32_t X2[64];
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(x + 128 * gc);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const u32x4_t v = src[q];
            X2[4 * q] = v.x; X2[4 * q + 1] = v.y; X2[4 * q + 2] = v.z; X2[4 * q + 3] = v.w;
        }
        float P = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t Pw[R];
#pragma unroll
            for (int p = 0; p < R; ++p) Pw[p] = pl[p][d];
            uint32_t D0[16], D1[16];
            decode_word<R>(Pw, D0, D1);
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                P = dot2(D0[m], X2[16 * d + m], P);
                if constexpr (Phases<R>::count == 2) P = dot2(D1[m], X2[16 * d + m], P);
            }
        }
        const int64_t sidx = (int64_t)min(row, n - 1) * G + gc;
        const uint32_t sb = (uint32_t)scales[sidx] << 16;
        const float s = (gvalid && row < n) ? __uint_as_float(sb) : 0.f;
        float Pc = P + correction<R, 64>(X2);
        if (zeros) {  // asymmetric: + (127.5 - z) * 2^(R-8) * sum of the group's X
            const uint32_t one = 0x3F803F80u;
            float sx = 0.f;
#pragma unroll
            for (int m = 0; m < 64; ++m) sx = dot2(one, X2[m], sx);
            const float z = __uint_as_float((uint32_t)zeros[sidx] << 16);
            Pc = fmaf((127.5f - z) * (1.0f / (float)(1 << (8 - R))), sx, Pc);
        }
        acc = fmaf(s, Pc, acc);
    }
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    if (gg == 0) red[w][i] = acc;
    __syncthreads();
    if (threadIdx.x < 16) {
        float sum = 0.f;
        for (int ww = 0; ww < W; ++ww) sum += red[ww][threadIdx.x];
        if (16 * tile + (int)threadIdx.x < n)
            store_y(y, ybf16, 16 * tile + threadIdx.x, sum * (float)(1 << (8 - R)));
    }
}

// grid: ceil(tiles / tiles_per_wg); batch rows 1..NBR of x (row stride ldx)
// and y (row stride ldy).
template <int R, int PD, bool ASYM, int NBR, bool XO>
__global__ __launch_bounds__(64 * GEMV_MAX_WAVES, GEMV_WGS_PER_CU) void gemv_kernel(const uint16_t *__restrict__ x,
                                                                  int64_t ldx, int batch,
                                                                  const uint8_t *__restrict__ planes,
                                                                  int64_t plane_bytes,
                                                                  const uint16_t *__restrict__ scales,
                                                                  const uint16_t *__restrict__ zeros,
                                                                  int n, int k, int tiles_total,
                                                                  int tiles_per_wg,
                                                                  float *__restrict__ y, int64_t ldy,
                                                                  int ybf16) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int t_begin = blockIdx.x * tiles_per_wg;
    const int T = min(tiles_per_wg, tiles_total - t_begin);
    gemv_tiles<R, PD, ASYM, NBR, XO>(x, ldx, batch, planes, plane_bytes, scales, zeros, n, k, t_begin, T,
                                 tiles_per_wg, y, ldy, ybf16, lds);
}

// ---------------------------------------------------------------- grouped launch

struct GemvJob {
    const uint16_t *x;  // [batch][k], y [batch][n]
    const uint8_t *planes;
    int64_t plane_bytes;
    const uint16_t *scales;
    float *y;
    int batch, n, k, r, tiles, tpw, item_begin;
};

struct GemvGroup {
    GemvJob job[GEMV_MAX_GROUP];
    int count, slots;
};

// Workgroup b runs item b; items are numbered product by product.  Every
// item has `slots` partial-sum slots per wave (the largest tpw of the group).
// NBR = 1: batch-1 products; NBR = 4: batch 2..4.
template <int NBR>
__global__ __launch_bounds__(64 * GEMV_MAX_WAVES, GEMV_WGS_PER_CU) void gemv_group_kernel(GemvGroup grp) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int item = blockIdx.x;
    int jb = 0;
    while (jb + 1 < grp.count && item >= grp.job[jb + 1].item_begin) ++jb;
    const GemvJob &J = grp.job[jb];
    const int t_begin = (item - J.item_begin) * J.tpw;
    const int T = min(J.tpw, J.tiles - t_begin);
    switch (J.r) {
#define NBW_GEMV_CASE(RR)                                                                    \
    case RR:                                                                                 \
        gemv_tiles<RR, gemv_depth(RR), false, NBR, false>(J.x, J.k, J.batch, J.planes, J.plane_bytes,   \
                                                   J.scales, nullptr, J.n, J.k, t_begin, T,      \
                                                   grp.slots, J.y, J.n, 0, lds);                 \
        break;
        NBW_GEMV_CASE(1)
        NBW_GEMV_CASE(2)
        NBW_GEMV_CASE(3)
        NBW_GEMV_CASE(4)
        NBW_GEMV_CASE(5)
        NBW_GEMV_CASE(6)
        NBW_GEMV_CASE(7)
        NBW_GEMV_CASE(8)
#undef NBW_GEMV_CASE
    }
}

// ---------------------------------------------------------------- host side

// Launch shape of the streaming kernel.  Eight waves per workgroup and about
// GEMV_WGS_PER_CU workgroups per CU, each owning a run of 16-row tiles.
struct GemvPlan {
    int waves, tpw;
    bool deep;  // prefetch depth gemv_depth(r), else GEMV_DEPTH_SHORT
    bool xo;    // (deep only) each set's X loaded with its first tile only
};

// Tile runs from which a set's X is loaded once, not with every tile.
constexpr int GEMV_XO_MIN_TILES = 3;

static GemvPlan gemv_plan(int n, int k, int r, int cu_count) {
    const int tiles = (n + 15) / 16;
    GemvPlan p;
    p.waves = GEMV_MAX_WAVES;
    const int wgs = GEMV_WGS_PER_CU * cu_count;
    int tpw = (tiles + wgs / 2) / wgs;  // about GEMV_WGS_PER_CU workgroups per CU
    if (tpw > GEMV_MAX_TILES) tpw = GEMV_MAX_TILES;
    if (tpw < 1) tpw = 1;
    p.tpw = tpw;
    const int nsets = (k / 128 + 3) / 4;
    const int steps = (nsets + p.waves - 1) / p.waves * tpw;  // per wave, at most
    p.deep = gemv_depth(r) > GEMV_DEPTH_SHORT && steps >= 4;
    p.xo = p.deep && tpw >= GEMV_XO_MIN_TILES;
    return p;
}

static bool gemv_streamable(int k);

template <int R, bool ASYM, int NBR>
static void launch_stream(const GemvPlan &p, int tiles, const QgemmArgs &a, const uint16_t *x,
                          int nb, float *y, hipStream_t stream) {
    const dim3 grid((tiles + p.tpw - 1) / p.tpw), block(64 * p.waves);
    const size_t lds = gemv_lds_bytes(p.waves, p.tpw, NBR);
    if (p.deep && p.xo)
        hipLaunchKernelGGL((gemv_kernel<R, gemv_depth(R), ASYM, NBR, true>), grid, block, lds, stream, x,
                           a.ldx, nb, a.planes, a.plane_bytes, a.scales, a.zeros, a.n, a.k, tiles,
                           p.tpw, y, a.ldy, a.ybf16);
    else if (p.deep)
        hipLaunchKernelGGL((gemv_kernel<R, gemv_depth(R), ASYM, NBR, false>), grid, block, lds, stream, x,
                           a.ldx, nb, a.planes, a.plane_bytes, a.scales, a.zeros, a.n, a.k, tiles,
                           p.tpw, y, a.ldy, a.ybf16);
    else
        hipLaunchKernelGGL((gemv_kernel<R, GEMV_DEPTH_SHORT, ASYM, NBR, false>), grid, block, lds, stream,
                           x, a.ldx, nb, a.planes, a.plane_bytes, a.scales, a.zeros, a.n, a.k, tiles,
                           p.tpw, y, a.ldy, a.ybf16);
}

template <int R>
static void launch_r(const QgemmArgs &a, int cu_count, hipStream_t stream) {
    const int tiles = (a.n + 15) / 16;
    const bool stream_k = gemv_streamable(a.k);
    // Up to GEMV_MAX_BATCH batch rows per launch of the streaming kernel
    // (one per launch of the odd-group-count kernel).
    for (int64_t b = 0; b < a.batch;) {
        const int nb = stream_k ? (int)std::min<int64_t>(GEMV_MAX_BATCH, a.batch - b) : 1;
        const uint16_t *x = a.x + b * a.ldx;
        // (y advances by ldy elements of the output type)
        float *y = a.ybf16 ? reinterpret_cast<float *>(reinterpret_cast<uint16_t *>(a.y) + b * a.ldy)
                           : a.y + b * a.ldy;
        if (!stream_k) {
            hipLaunchKernelGGL(gemv_odd_kernel<R>, dim3(tiles), dim3(64 * GEMV_ODD_WAVES), 0, stream,
                               x, a.planes, a.plane_bytes, a.scales, a.zeros, a.n, a.k, y, a.ybf16);
        } else {
            const GemvPlan p = gemv_plan(a.n, a.k, R, cu_count);
            if (nb == 1) {
                if (a.zeros)
                    launch_stream<R, true, 1>(p, tiles, a, x, 1, y, stream);
                else
                    launch_stream<R, false, 1>(p, tiles, a, x, 1, y, stream);
            } else {
                if (a.zeros)
                    launch_stream<R, true, GEMV_MAX_BATCH>(p, tiles, a, x, nb, y, stream);
                else
                    launch_stream<R, false, GEMV_MAX_BATCH>(p, tiles, a, x, nb, y, stream);
            }
        }
        b += nb;
    }
}

hipError_t launch_gemv(int r, const QgemmArgs &a, int cu_count, hipStream_t stream) {
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

void gemv_name(int r, const QgemmArgs &a, int cu_count, char *out, size_t len) {
    if (!gemv_streamable(a.k)) {
        snprintf(out, len, "nbw::gemv_odd_kernel<%d>", r);
    } else {
        // (the kernel of the first launch: batch rows 1..4)
        const GemvPlan p = gemv_plan(a.n, a.k, r, cu_count);
        snprintf(out, len, "nbw::gemv_kernel<%d, %d, %s, %d, %s>", r,
                 p.deep ? gemv_depth(r) : GEMV_DEPTH_SHORT, a.zeros ? "true" : "false",
                 a.batch > 1 ? GEMV_MAX_BATCH : 1, p.xo ? "true" : "false");
    }
}

int gemv_group_capacity() { return GEMV_MAX_GROUP; }
int gemv_max_batch() { return GEMV_MAX_BATCH; }

// The streaming kernel reads the scales of a set's four groups as one aligned
// 8-byte word: it takes group counts that are multiples of 4 (every other
// shape goes to the plain one-tile kernel).
static bool gemv_streamable(int k) { return ((k / 128) & 3) == 0; }

// (contiguous rows: x [batch][k], y [batch][n])
bool gemv_group_eligible(const QgemmArgs &a) {
    return a.batch >= 1 && a.batch <= GEMV_MAX_BATCH && gemv_streamable(a.k) && !a.zeros && !a.ybf16;
}

// One launch per kernel variant: the batch-1 products, then those of batch
// 2..4, each in the order given.
hipError_t launch_gemv_group(const QgemmArgs *probs, const int *rs, int count, int cu_count,
                             hipStream_t stream) {
    for (int nbr : {1, GEMV_MAX_BATCH}) {
        GemvGroup grp = {};
        int items = 0, slots = 1;
        for (int j0 = 0; j0 < count; ++j0) {
            const QgemmArgs &a = probs[j0];
            if ((a.batch > 1 ? GEMV_MAX_BATCH : 1) != nbr) continue;
            GemvJob &J = grp.job[grp.count++];
            J.x = a.x;
            J.planes = a.planes;
            J.plane_bytes = a.plane_bytes;
            J.scales = a.scales;
            J.y = a.y;
            J.batch = (int)a.batch;
            J.n = a.n;
            J.k = a.k;
            J.r = rs[j0];
            J.tiles = (a.n + 15) / 16;
            J.tpw = gemv_plan(a.n, a.k, rs[j0], cu_count).tpw;
            if (J.tpw > slots) slots = J.tpw;
            J.item_begin = items;
            items += (J.tiles + J.tpw - 1) / J.tpw;
        }
        if (grp.count == 0) continue;
        grp.slots = slots;
        if (nbr == 1)
            hipLaunchKernelGGL(gemv_group_kernel<1>, dim3(items), dim3(64 * GEMV_MAX_WAVES),
                               gemv_lds_bytes(GEMV_MAX_WAVES, slots, 1), stream, grp);
        else
            hipLaunchKernelGGL(gemv_group_kernel<GEMV_MAX_BATCH>, dim3(items), dim3(64 * GEMV_MAX_WAVES),
                               gemv_lds_bytes(GEMV_MAX_WAVES, slots, GEMV_MAX_BATCH), stream, grp);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace nbw
