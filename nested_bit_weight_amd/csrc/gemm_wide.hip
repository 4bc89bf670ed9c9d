// gemm_wide.hip -- large-batch dequant-GEMM for symmetric children, gfx950.
//
// Y[b][i] = sum_j X[b][j] * s[i][j/128] * 2^(8-r) * (q_r[i][j] + 1/2 - 2^(r-1)),
// the r-bit child of a sliceable parent (MatGPTQ: Efficient and Accurate
// Inference over Nested Quantized Models, Abstract: kernels that serve batch
// sizes beyond one; Figure 1: kernel speed-up swept over batch sizes).  At
// batch 128-256 the product is a dense contraction bound by the MFMA rate, and
// decoding the bit-planes is the VALU work that has to hide under it.  This
// kernel decodes every weight once per workgroup and keeps the VALU work per
// matrix instruction small:
//
//  - a workgroup owns 256 weight rows x BM = 32*NBT batch rows (NBT = 4: 128
//    batch rows) and a range of 128-wide groups; each of its 8 waves (two per
//    SIMD) owns 32 weight rows and ALL BM batch rows, so a weight row is
//    decoded by one wave per BM batch rows.  D = A.B with
//    v_mfma_f32_32x32x16_bf16, A = X (rows: batch), B = decoded weights
//    (columns: weight rows).
//  - B operands are decoded in registers at the start of each group
//    (decode.h; lane (weight row l%32, half h) decodes columns 64h..64h+63 of
//    its row's group, k-step j takes its pairs 4j..4j+3, i.e. columns
//    64h+8j..64h+8j+7), while the next group's planes are in flight.
//  - A operands come from LDS.  X reaches LDS by direct global->LDS loads
//    (global_load_lds_dwordx4, no registers), double buffered per group and
//    spread over the chain steps.  One load instruction fills a 1 KB block
//    holding four batch rows 16 apart; a 16-byte pad after each block puts the
//    16 rows a quarter-wave reads at 16 different bank groups, and every
//    fragment address is a per-lane base plus a constant.
//  - each group's 8-MFMA chain per 32-row batch tile starts from zero and the
//    group scale (one per lane: the lane's weight row) is folded in fp32
//    after it (software-pipelined: the previous tile's fold runs two FMAs per
//    MFMA of the next chain), so every operand of the chain is exact in bf16.
//  - the decode's constant offsets leave, per batch row and group, a
//    correction sum_k x_k * (1/2 - 2^(r-1) - offset_k) (X only) times the
//    group scale.  Each of waves 0..3 forms the corrections of one batch tile
//    from the X fragments it reads anyway (waves 4..7 read the same fragments
//    and leave it to them), splits each fp32 value exactly into three
//    bf16 parts, and parks them in LDS; every 8 groups the block of
//    corrections enters the accumulators as a small bf16 product (corrections
//    [batch row][part, group] times scales [part, group][weight row], the
//    scales from per-lane LDS slots): two MFMAs per batch tile per 8 groups,
//    exact products, fp32 sums.
//  - the waves rotate the order of their batch tiles so that the tiles whose
//    corrections they form come first; one barrier per group hands over the X
//    buffers and the corrections.  For r <= 4 half the waves decode the next
//    group right after their chains instead of at the group's start, so that
//    the workgroup does not decode and multiply in lockstep.
//  - where the output tiles leave CUs idle, k splits over workgroups into a
//    caller workspace and a second launch adds the splits in order.
#include <cstdio>
#include <type_traits>

#include "decode.h"
#include "launch.h"

namespace nbw {

typedef float gw_f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t gw_u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void gw_lds_void;

constexpr int GW_WAVES = 8;                 // two waves per SIMD
constexpr int GW_THREADS = 64 * GW_WAVES;
constexpr int GW_BN = 32 * GW_WAVES;        // weight rows per workgroup
constexpr int GW_BLOCK = 1024 + 16;         // one DMA block (4 batch rows) + pad
constexpr int GW_SET = 16 * GW_BLOCK;       // 64 batch rows
constexpr int GW_CB = 8;                    // groups per correction block

// LDS of one workgroup: two X buffers and two correction blocks (each: three
// bf16 parts [part][batch row][8 groups]).
template <int NBT> struct GwLayout {
    static_assert(NBT == 4 || NBT == 8, "batch tiles per workgroup: 4 or 8");
    static constexpr int BM = 32 * NBT;
    static constexpr int xbuf = (BM / 64) * GW_SET;
    static constexpr int cblk = 3 * BM * GW_CB * 2;
    static constexpr int sblk = GW_THREADS * GW_CB * 2;  // each lane's scales of a block
    static constexpr int bytes = 2 * xbuf + 2 * cblk + 2 * sblk;
    static constexpr int tile = GW_BN * BM;  // fp32 values of one partial tile
};

__device__ __forceinline__ float gw_dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ gw_f32x16_t gw_mfma(const u32x4_t &a, const u32x4_t &b,
                                               const gw_f32x16_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Round-to-nearest-even bf16 of v, as the bit pattern in the low 16 bits and
// as the fp32 value it stands for.
__device__ __forceinline__ uint32_t gw_bf16_bits(float v, float &as_f32) {
    uint32_t u = __float_as_uint(v);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    as_f32 = __uint_as_float(u << 16);
    return u;
}

// Correction coefficient of X pair p of k-step j (columns 64h + 8j + 2p, +1):
// it multiplies the bf16 pair m = 4(j%4) + p of the lane's decoded word.
template <int R> __device__ constexpr float gw_coef(int j, int p) {
    if constexpr (R > 4)
        return (0.5f - (float)(1 << (R - 1))) * (float)(1 << (8 - R));
    else
        return pair_coef<R>(4 * (j & 3) + p);
}
// Class (offset) of that pair: equal classes share a coefficient.
template <int R> __device__ constexpr int gw_class(int j, int p) {
    if constexpr (R > 4)
        return 0;
    else
        return lsb0<R>(4 * (j & 3) + p);
}

// Offset (in floats) of thread tid's accumulators (tile bt, values 4qv..4qv+3)
// in a partial tile: one float4 per thread and (bt, qv), in thread order.
__device__ __forceinline__ int gw_part_offset(int bt, int qv, int tid) {
    return ((bt * 4 + qv) * GW_THREADS + tid) * 4;
}

// Stores one 32 x 32 accumulator block: the lane of half h and weight row
// nrow holds batch rows brow + 8(v/4) + 4h + v%4 of column nrow, scaled by post.
__device__ __forceinline__ void gw_store_block(const gw_f32x16_t &a, int brow, int h, int nrow,
                                               int n, int batch, float post, float *y,
                                               int64_t ldy, int ybf16) {
    if (nrow >= n) return;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int b = brow + 8 * (v >> 2) + 4 * h + (v & 3);
        if (b < batch) store_y(y, ybf16, (int64_t)b * ldy + nrow, a[v] * post);
    }
}

// grid: (ceil(n / 128), ceil(batch / BM), splits); block 256.  Groups
// [z * gps, min(G, (z + 1) * gps)).  With part != null (split k) the raw
// partial tile is stored for gemm_wide_reduce_kernel; otherwise Y.
template <int R, int NBT>
__global__ __launch_bounds__(GW_THREADS, 1) void gemm_wide_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int batch, const uint8_t *__restrict__ planes,
    int64_t plane_bytes, const uint16_t *__restrict__ scales, int n, int k, int gps,
    float *__restrict__ y, int64_t ldy, int ybf16, float *__restrict__ part) {
    using L = GwLayout<NBT>;
    __shared__ __align__(16) unsigned char lds[L::bytes];
    constexpr int BM = L::BM;
    constexpr bool BYTES = R > 4;
    constexpr float POST = BYTES ? 1.0f : (float)(1 << (8 - R));
    // batch tiles whose corrections a wave forms; waves w and w + NBT have the
    // same ones, and only waves 0..3 form them
    constexpr int CT = 1;
    static_assert(2 * NBT == GW_WAVES, "waves w and w + NBT share their batch tiles");

    const int G = k >> 7;
    const int g_begin = blockIdx.z * gps;
    const int g_end = min(G, g_begin + gps);
    if (g_begin >= g_end) return;  // uniform over the workgroup

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int b0 = blockIdx.y * BM;
    const int npad = (n + 15) & ~15;
    const int nrow = blockIdx.x * GW_BN + 32 * w + l32;
    const bool nvalid = nrow < n;
    const int rc = min(nrow, npad - 1);
    const uint8_t *pbase = planes + ((int64_t)(rc >> 4) * G * 16 + (rc & 15)) * 16 + 8 * h;
    const uint16_t *srow = scales + (int64_t)min(nrow, n - 1) * G;

    unsigned char *const xs = lds;
    unsigned char *const cb = lds + 2 * L::xbuf;
    // Each lane's scales of the groups of a correction block, [lane][slot],
    // written by the lane itself group by group (its own slots only).
    unsigned char *const sbl = lds + 2 * L::xbuf + 2 * L::cblk;

    // Correction blocks start as zeros: a partial last block reads finite
    // values (times a zero scale) in its unused slots.
    for (int i = tid; i < 2 * L::cblk / 16; i += GW_THREADS)
        *reinterpret_cast<u32x4_t *>(cb + 16 * i) = (u32x4_t){0u, 0u, 0u, 0u};

    // X of group g into buffer qb: wave w fills blocks w, w+4, ...; block blk
    // of 64-row set s = blk/16 holds batch rows 64s + blk%16 + 16t (t = 0..3),
    // lane L moving 16 bytes (columns 8(L%16)..+7) of row slot t = L/16.
    auto stage_x_block = [&](int g, int qb, int i) {
        const int blk = GW_WAVES * i + w;
        const int set = blk >> 4, bi = blk & 15;
        const int row = 64 * set + bi + 16 * (lane >> 4);
        const uint16_t *src = x + (int64_t)min(b0 + row, batch - 1) * ldx + 128 * g + 8 * (lane & 15);
        __builtin_amdgcn_global_load_lds(
            src, (gw_lds_void *)(xs + qb * L::xbuf + set * GW_SET + bi * GW_BLOCK), 16, 0, 0);
    };
    auto stage_x = [&](int g, int qb) {
#pragma unroll
        for (int i = 0; i < BM / (4 * GW_WAVES); ++i) stage_x_block(g, qb, i);
    };
    // Fragment of batch tile bt, k-step j: lane (row l32 of the tile, half h)
    // reads columns 64h + 8j .. +7 of its row.
    const int xlane = (l32 & 15) * GW_BLOCK + (l32 >> 4) * 256 + 128 * h;
    auto xfrag = [&](int qb, int bt, int j) {
        return *reinterpret_cast<const u32x4_t *>(xs + qb * L::xbuf + xlane + (bt >> 1) * GW_SET +
                                                  (bt & 1) * 512 + 16 * j);
    };

    gw_u32x2_t pw[R];
    auto load_planes = [&](int g) {
        const uint8_t *c = pbase + (int64_t)g * 256;
#pragma unroll
        for (int p = 0; p < R; ++p)
            pw[p] = __builtin_nontemporal_load(
                reinterpret_cast<const gw_u32x2_t *>(c + (int64_t)p * plane_bytes));
    };
    auto decode = [&](uint32_t *W) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            uint32_t P[R];
#pragma unroll
            for (int p = 0; p < R; ++p) P[p] = q ? pw[p].y : pw[p].x;
            if constexpr (BYTES) {
                decode_word_bytes<R>(P, W + 16 * q);
            } else {
                uint32_t D1[16];
                decode_word<R>(P, W + 16 * q, D1);
            }
        }
    };
    gw_f32x16_t acc[NBT];
#pragma unroll
    for (int t = 0; t < NBT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[t][v] = 0.f;

    // The block of corrections of parity cp enters the accumulators:
    // A = parts [batch row][part, group] (k-step 0: lanes h read part h;
    // k-step 1: lanes h = 0 read part 2, lanes h = 1 zeros), B = the block's
    // scales for both halves.
    auto consume = [&](int cp) {
        const unsigned char *cbp = cb + cp * L::cblk;
        // (slots past the range were written as zeros)
        const u32x4_t sb = *reinterpret_cast<const u32x4_t *>(sbl + cp * L::sblk + tid * GW_CB * 2);
#pragma unroll
        for (int pos = 0; pos < NBT; ++pos) {
            const int bt = (pos + CT * w) & (NBT - 1);
            const int rb = 32 * bt + l32;
            const u32x4_t a0 = *reinterpret_cast<const u32x4_t *>(cbp + ((h * BM + rb) * GW_CB) * 2);
            u32x4_t a1 = *reinterpret_cast<const u32x4_t *>(cbp + ((2 * BM + rb) * GW_CB) * 2);
            if (h) a1 = (u32x4_t){0u, 0u, 0u, 0u};
            acc[pos] = gw_mfma(a0, sb, acc[pos]);
            acc[pos] = gw_mfma(a1, sb, acc[pos]);
        }
    };

    // Two teams of waves (r <= 4): team A decodes a group's weights at the
    // group's start, team B right after its chains, one group ahead.  The
    // barrier at each group's end otherwise keeps all waves in step, all
    // decoding (the matrix unit idle) and then all issuing MFMAs, with their
    // memory requests in bursts.  (Measured at batch 256: 2-5% faster for
    // r <= 4 on one MI355X, with either pairing of waves into teams, the same
    // speed on another; at r = 5..8 team B's copy of the loop spills
    // registers, so those widths keep one team.)
    // Waves 4..7 (team B for r <= 4) leave the corrections to waves 0..3.
    const bool upper = (w >> 2) & 1;
    const bool team_b = R <= 4 && upper;
    uint32_t W[32];      // the decoded weights of the group being computed
    uint32_t s_nx = 0u;  // the scale of the next group (team B: loaded a group early)

    // Prologue: X and scales of the first group, its planes in flight.
    stage_x(g_begin, 0);
    uint32_t s_raw = srow[g_begin];
    load_planes(g_begin);
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(R) : "memory");
    __builtin_amdgcn_s_barrier();

    // One group: its weights decoded (team A; the planes arrived during the
    // previous group), the next group's planes and X requested, then the
    // chains over the batch tiles (team B then decodes the next group).  The
    // team is a compile-time argument: each team runs its own copy of the
    // loop, so the decoded weights are live across a group boundary in team
    // B's copy only.
    // (always inlined: six call sites, and a call would put the accumulators
    // and the decoded weights in scratch memory)
    auto group = [&](auto tb, auto form, int g, int qb) __attribute__((always_inline)) {
        constexpr bool TB = decltype(tb)::value;
        constexpr bool FORM = decltype(form)::value;  // this wave forms its tiles' corrections
        const int gi = g - g_begin;
        if (gi > 0 && (gi & 7) == 0) consume(((gi >> 3) - 1) & 1);  // a block is complete
        if ((gi & 7) == 0) {
            // a new block: its slots past the range stay zero (a zero scale)
            *reinterpret_cast<u32x4_t *>(sbl + ((gi >> 3) & 1) * L::sblk + tid * GW_CB * 2) =
                (u32x4_t){0u, 0u, 0u, 0u};
        }
        const int gnext = min(g + 1, g_end - 1);
        if constexpr (!TB) {
            decode(W);
            // (the planes of g are the oldest loads in flight; nothing may be
            // requested ahead of the decode, or the wait for them waits for it too)
            __builtin_amdgcn_sched_barrier(0);
            s_nx = srow[gnext];
            load_planes(gnext);
        }
        const float s = nvalid ? __uint_as_float(s_raw << 16) : 0.f;
        reinterpret_cast<uint16_t *>(sbl + ((gi >> 3) & 1) * L::sblk)[tid * GW_CB + (gi & 7)] =
            (uint16_t)(nvalid ? s_raw : 0u);
        __builtin_amdgcn_sched_barrier(0);

        float cls[CT][7];
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int a = 0; a < 7; ++a) cls[c][a] = 0.f;
        const uint32_t one = 0x3F803F80u;  // bf16 (1.0, 1.0)

        // The chains, software-pipelined in program order (each step pinned
        // by a scheduling barrier): step (pos, j) requests the X fragment
        // XD steps ahead, feeds the MFMA of k-step j of batch tile pos, and
        // folds two values of the previous tile's finished chain, so the
        // matrix unit never waits for a fold or for LDS.
        constexpr int XD = 4;
        constexpr int NSTEP = NBT * 8;
        u32x4_t ring[XD];
#pragma unroll
        for (int i = 0; i < XD; ++i) ring[i] = xfrag(qb, (CT * w + i / 8) & (NBT - 1), i % 8);
        gw_f32x16_t Pprev;
#pragma unroll
        for (int v = 0; v < 16; ++v) Pprev[v] = 0.f;
#pragma unroll
        for (int pos = 0; pos < NBT; ++pos) {
            gw_f32x16_t P;
#pragma unroll
            for (int v = 0; v < 16; ++v) P[v] = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int idx = 8 * pos + j;
                // X of the next group, one DMA block every other step of the
                // first half: issued all at once, they back up the compute
                // unit's memory pipeline and hold up the matrix instructions
                if (idx % 2 == 0 && idx / 2 < BM / (4 * GW_WAVES)) stage_x_block(gnext, qb ^ 1, idx / 2);
                const u32x4_t a = ring[idx % XD];
                if (idx + XD < NSTEP) {
                    const int nidx = idx + XD;
                    ring[idx % XD] = xfrag(qb, (nidx / 8 + CT * w) & (NBT - 1), nidx % 8);
                }
                if (FORM && pos < CT) {
                    cls[pos][gw_class<R>(j, 0)] = gw_dot2(one, a.x, cls[pos][gw_class<R>(j, 0)]);
                    cls[pos][gw_class<R>(j, 1)] = gw_dot2(one, a.y, cls[pos][gw_class<R>(j, 1)]);
                    cls[pos][gw_class<R>(j, 2)] = gw_dot2(one, a.z, cls[pos][gw_class<R>(j, 2)]);
                    cls[pos][gw_class<R>(j, 3)] = gw_dot2(one, a.w, cls[pos][gw_class<R>(j, 3)]);
                }
                const u32x4_t wv = {W[4 * j], W[4 * j + 1], W[4 * j + 2], W[4 * j + 3]};
                P = gw_mfma(a, wv, P);
                if (pos > 0) {
                    acc[pos - 1][2 * j] = fmaf(s, Pprev[2 * j], acc[pos - 1][2 * j]);
                    acc[pos - 1][2 * j + 1] = fmaf(s, Pprev[2 * j + 1], acc[pos - 1][2 * j + 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            Pprev = P;
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[NBT - 1][v] = fmaf(s, Pprev[v], acc[NBT - 1][v]);

        // Corrections of this wave's tiles for group g: both halves of each
        // row, split into three exact bf16 parts for the block.
        unsigned char *cbp = cb + ((gi >> 3) & 1) * L::cblk;
        const int slot = gi & 7;
#pragma unroll
        for (int c = 0; c < (FORM ? CT : 0); ++c) {
            float corr = 0.f;
#pragma unroll
            for (int a = 0; a < 7; ++a) {
                float coef = 0.f;
                bool used = false;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        if (gw_class<R>(j, p) == a) {
                            coef = gw_coef<R>(j, p);
                            used = true;
                        }
                if (used) corr = fmaf(coef, cls[c][a], corr);
            }
            corr += __shfl_xor(corr, 32);
            const int bt = (c + CT * w) & (NBT - 1);
            const int rb = 32 * bt + l32;
            float f_hi, f_mid, f_lo;
            const uint32_t hi = gw_bf16_bits(corr, f_hi);
            const float r1 = corr - f_hi;
            const uint32_t mid = gw_bf16_bits(r1, f_mid);
            const uint32_t lo = gw_bf16_bits(r1 - f_mid, f_lo);
            // lanes h = 0 write part 0, lanes h = 1 part 1; both halves hold the
            // same value of part 2 and write it to the same place
            uint16_t *dst = reinterpret_cast<uint16_t *>(cbp) + rb * GW_CB + slot;
            dst[h * BM * GW_CB] = (uint16_t)(h ? mid : hi);
            dst[2 * BM * GW_CB] = (uint16_t)lo;
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (TB) {
            // the next group's weights (its planes came in during this group),
            // then the planes and scale of the one after
            decode(W);
            __builtin_amdgcn_sched_barrier(0);
            const int g2 = min(g + 2, g_end - 1);
            const uint32_t s2 = srow[g2];
            load_planes(g2);
            s_raw = s_nx;
            s_nx = s2;
            __builtin_amdgcn_sched_barrier(0);
            // X of the next group and this group's corrections are in LDS for
            // every wave after the barrier; the R + 1 loads just issued (planes
            // and scale of g + 2, after the X blocks) stay in flight: loads
            // complete in order.
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(R + 1) : "memory");
        } else {
            s_raw = s_nx;
            __builtin_amdgcn_sched_barrier(0);
            // X of the next group and this group's corrections are in LDS for
            // every wave after the barrier (the planes of g + 1, requested
            // before the X blocks, have arrived too: loads complete in order).
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        }
        __builtin_amdgcn_s_barrier();
    };

    auto run = [&](auto tb, auto form) __attribute__((always_inline)) {
        if constexpr (decltype(tb)::value) {  // the first group's weights, the next group's planes
            decode(W);
            __builtin_amdgcn_sched_barrier(0);
            const int g1 = min(g_begin + 1, g_end - 1);
            s_nx = srow[g1];
            load_planes(g1);
            __builtin_amdgcn_sched_barrier(0);
        }
        int g = g_begin;
        for (; g + 1 < g_end; g += 2) {
            group(tb, form, g, 0);
            group(tb, form, g + 1, 1);
        }
        if (g < g_end) group(tb, form, g, 0);
    };
    if (team_b)
        run(std::true_type{}, std::false_type{});
    else if (upper)
        run(std::false_type{}, std::false_type{});
    else
        run(std::false_type{}, std::true_type{});
    // The last (possibly partial) block of corrections.
    consume(((g_end - 1 - g_begin) >> 3) & 1);

    if (part) {
        float *dst = part + ((size_t)blockIdx.z * gridDim.x * gridDim.y + blockIdx.y * gridDim.x +
                             blockIdx.x) * L::tile;
#pragma unroll
        for (int pos = 0; pos < NBT; ++pos) {
            const int bt = (pos + CT * w) & (NBT - 1);
#pragma unroll
            for (int qv = 0; qv < 4; ++qv)
                *reinterpret_cast<float4 *>(dst + gw_part_offset(bt, qv, tid)) =
                    make_float4(acc[pos][4 * qv], acc[pos][4 * qv + 1], acc[pos][4 * qv + 2],
                                acc[pos][4 * qv + 3]);
        }
        return;
    }
#pragma unroll
    for (int pos = 0; pos < NBT; ++pos) {
        const int bt = (pos + CT * w) & (NBT - 1);
        gw_store_block(acc[pos], b0 + 32 * bt, h, nrow, n, batch, POST, y, ldy, ybf16);
    }
}

// Adds the S partial tiles of a split launch in the order z = 0..S-1 and
// stores Y.  grid: (gridX, gridY, 4 waves x NBT tiles); block 64: workgroup
// (x, y, w * NBT + bt) finishes tile bt of wave w of GEMM workgroup (x, y).
template <int NBT>
__global__ __launch_bounds__(64) void gemm_wide_reduce_kernel(const float *__restrict__ part, int S,
                                                              int batch, int n, float post,
                                                              float *__restrict__ y, int64_t ldy,
                                                              int ybf16) {
    using L = GwLayout<NBT>;
    const int lane = threadIdx.x;
    const int w = blockIdx.z / NBT, bt = blockIdx.z % NBT;
    const int tid = w * 64 + lane;
    const int ntiles = gridDim.x * gridDim.y;
    const float *src = part + (size_t)(blockIdx.y * gridDim.x + blockIdx.x) * L::tile;
    gw_f32x16_t tot;
#pragma unroll
    for (int v = 0; v < 16; ++v) tot[v] = 0.f;
    for (int z0 = 0; z0 < S; z0 += 4) {
        float4 v[4][4];
#pragma unroll
        for (int zz = 0; zz < 4; ++zz)
#pragma unroll
            for (int qv = 0; qv < 4; ++qv)
                v[zz][qv] = *reinterpret_cast<const float4 *>(
                    src + (size_t)min(z0 + zz, S - 1) * ntiles * L::tile + gw_part_offset(bt, qv, tid));
#pragma unroll
        for (int zz = 0; zz < 4; ++zz) {
            const bool live = z0 + zz < S;
#pragma unroll
            for (int qv = 0; qv < 4; ++qv) {
                tot[4 * qv] += live ? v[zz][qv].x : 0.f;
                tot[4 * qv + 1] += live ? v[zz][qv].y : 0.f;
                tot[4 * qv + 2] += live ? v[zz][qv].z : 0.f;
                tot[4 * qv + 3] += live ? v[zz][qv].w : 0.f;
            }
        }
    }
    const int nrow = blockIdx.x * GW_BN + 32 * w + (lane & 31);
    gw_store_block(tot, blockIdx.y * L::BM + 32 * bt, lane >> 5, nrow, n, batch, post, y, ldy, ybf16);
}

// ---------------------------------------------------------------- host side

static int gw_nbt(int64_t) { return 4; }

static int gw_tiles(const QgemmArgs &a) {
    const int bm = 32 * gw_nbt(a.batch);
    return (a.n + GW_BN - 1) / GW_BN * (int)((a.batch + bm - 1) / bm);
}

// Splits of k: as many as fill the compute units once, each with at least 4
// groups; 1 when the tiles alone fill them.
static int gw_splits(const QgemmArgs &a, int cu_count) {
    const int tiles = gw_tiles(a);
    const int G = a.k / 128;
    int s = cu_count / tiles;
    if (s > G / 4) s = G / 4;
    if (s < 1) s = 1;
    const int gps = (G + s - 1) / s;
    return (G + gps - 1) / gps;  // splits that hold at least one group
}

int64_t gemm_wide_workspace_bytes(const QgemmArgs &a, int cu_count) {
    const int s = gw_splits(a, cu_count);
    if (s <= 1) return 0;
    const int nbt = gw_nbt(a.batch);
    return (int64_t)s * gw_tiles(a) * GW_BN * 32 * nbt * 4;
}

template <int R, int NBT>
static void gw_launch(const QgemmArgs &a, int cu_count, hipStream_t stream) {
    const int G = a.k / 128;
    const int64_t need = gemm_wide_workspace_bytes(a, cu_count);
    const bool use_ws = need > 0 && a.ws && a.ws_bytes >= need;
    const int want = use_ws ? gw_splits(a, cu_count) : 1;
    const int gps = (G + want - 1) / want;
    const int splits = (G + gps - 1) / gps;
    float *part = use_ws ? static_cast<float *>(a.ws) : nullptr;
    const dim3 grid((a.n + GW_BN - 1) / GW_BN, (unsigned)((a.batch + 32 * NBT - 1) / (32 * NBT)),
                    splits);
    hipLaunchKernelGGL((gemm_wide_kernel<R, NBT>), grid, dim3(GW_THREADS), 0, stream, a.x, a.ldx,
                       (int)a.batch, a.planes, a.plane_bytes, a.scales, a.n, a.k, gps, a.y, a.ldy,
                       a.ybf16, part);
    if (part)
        hipLaunchKernelGGL(gemm_wide_reduce_kernel<NBT>, dim3(grid.x, grid.y, GW_WAVES * NBT),
                           dim3(64), 0, stream, part, splits, (int)a.batch, a.n,
                           R > 4 ? 1.0f : (float)(1 << (8 - R)), a.y, a.ldy, a.ybf16);
}

template <int R>
static void gw_launch_r(const QgemmArgs &a, int cu_count, hipStream_t stream) {
    gw_launch<R, 4>(a, cu_count, stream);
}

hipError_t launch_gemm_wide(int r, const QgemmArgs &a, int cu_count, hipStream_t stream) {
    switch (r) {
    case 1: gw_launch_r<1>(a, cu_count, stream); break;
    case 2: gw_launch_r<2>(a, cu_count, stream); break;
    case 3: gw_launch_r<3>(a, cu_count, stream); break;
    case 4: gw_launch_r<4>(a, cu_count, stream); break;
    case 5: gw_launch_r<5>(a, cu_count, stream); break;
    case 6: gw_launch_r<6>(a, cu_count, stream); break;
    case 7: gw_launch_r<7>(a, cu_count, stream); break;
    case 8: gw_launch_r<8>(a, cu_count, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

void gemm_wide_name(int r, const QgemmArgs &a, char *out, size_t len) {
    snprintf(out, len, "nbw::gemm_wide_kernel<%d, %d>", r, gw_nbt(a.batch));
}

}  // namespace nbw
