// gemm.hip -- large-batch dequant-GEMM on the matrix cores, gfx950.
//
// Y[b][i] = sum_j X[b][j] * s[i][j/128] * 2^(8-r) * (q_r[i][j] + 1/2 - 2^(r-1)),
// the r-bit child of a sliceable parent (MatGPTQ: Efficient and Accurate
// Inference over Nested Quantized Models, Abstract: kernels that support
// batch sizes beyond one; Figure 1: batch sweep against a dense matmul).  At
// large batch the product is a real dense contraction, bound by the MFMA
// rate, so the weights are decoded once per workgroup tile and feed
// v_mfma_f32_32x32x16_bf16 directly.
//
// Layout of the work (D = A.B with A = X rows, B = decoded weights):
//  - a workgroup owns 128 batch rows x 256 weight rows and a range of 128-wide
//    groups along k; its 8 waves (two per SIMD) each own one block of 32
//    weight rows and all 128 batch rows (four 32-row blocks): 4 accumulator
//    tiles of 32 x 32.
//  - B operands never touch LDS: lane (row l%32, half h = l/32) of a weight
//    block loads 8 bytes of each plane -- words 2h and 2h+1 of its row's
//    16-byte chunk -- and decodes them (decode.h) into the 32 bf16 pairs of
//    columns 64h .. 64h+63 of the group; MFMA j takes pairs 4j..4j+3, i.e.
//    columns 64h + 8j .. 64h + 8j + 7, in natural order.
//  - A operands come from an LDS copy of the group's X tile (double
//    buffered, rows padded against bank conflicts): lane (row l%32, half h)
//    reads the same 8 columns 64h + 8j .. +7, so the k order of both
//    operands agrees.
//  - every 8-MFMA chain covers one group and starts from zero; the group
//    scale, one per lane (lane = weight row), is folded in fp32 right after.
//    Two batch blocks run their chains interleaved, so no MFMA waits on the
//    one before it.
//  - the decode's constant offsets leave a per-group correction
//    sum_k x_k * (1/2 - 2^(r-1) - offset_k) (X only) times the group scale;
//    these enter as a small fp32 product over groups (v_mfma_f32_32x32x2_f32,
//    two groups per instruction) from a four-slot LDS ring.
//  - X is loaded one group ahead (thread (row, quarter) moves 32 columns
//    and forms their share of the row's correction), planes and scales one
//    group ahead too; one barrier per group hands the X buffers over.
#include <cstdio>

#include "decode.h"
#include "launch.h"

namespace nbw {

typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int GEMM_BM = 128;        // batch rows per workgroup
constexpr int GEMM_WAVES = 8;       // waves per workgroup, one 32-row weight block each
constexpr int GEMM_BN = 32 * GEMM_WAVES;  // weight rows per workgroup
constexpr int GEMM_XSTRIDE = 136;   // bf16 per LDS row of the X tile (128 + 8 padding)

__device__ __forceinline__ float gm_dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ f32x16_t gm_mfma(const u32x4_t &a, const u32x4_t &b, const f32x16_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int GEMM_THREADS = 64 * GEMM_WAVES;
constexpr int GEMM_TILE = GEMM_BM * GEMM_BN;  // fp32 values of one partial tile

// Stores one 32 x 32 accumulator block: the lane of half h and weight row
// nrow holds batch rows brow + 8(v/4) + 4h + v%4 (v = 0..15) of column nrow,
// each scaled by post (fp32 or bf16).
__device__ __forceinline__ void gemm_store_block(const f32x16_t &a, int brow, int h, int nrow,
                                                 int n, int batch, float post, float *y,
                                                 int64_t ldy, int ybf16) {
    if (nrow >= n) return;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int b = brow + 8 * (v >> 2) + 4 * h + (v & 3);
        if (b >= batch) continue;
        const int64_t idx = (int64_t)b * ldy + nrow;
        store_y(y, ybf16, idx, a[v] * post);
    }
}

// Offset (in floats) of thread tid's accumulators (bb, 4q .. 4q+3) within a
// partial tile: slice bb*4+q holds one float4 per thread, in thread order,
// so both the stores here and the reads of the reduction are contiguous
// across a wave.
__device__ __forceinline__ int gemm_part_offset(int bb, int q, int tid) {
    return ((bb * 4 + q) * GEMM_THREADS + tid) * 4;
}

// Sum over the four lanes of a quad (lanes 4i..4i+3), in every lane: two
// DPP quad permutes, no LDS round trip.
__device__ __forceinline__ float quad_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
    return v;
}

// Operand form per child width.  R <= 4: the one-phase magic-exponent
// decode, operand offset_m + q with the offsets removed by the correction,
// result scaled by 2^(8-R) at the end.  R = 5..8: the single-phase byte
// decode, operand q * 2^(8-R) (exact in bf16), one correction coefficient
// (1/2 - 2^(R-1)) * 2^(8-R) for every column, no final scaling.  Either way
// one MFMA per k-step.
template <int R> struct GemmOperand {
    static constexpr bool bytes = R > 4;
    static constexpr float post = bytes ? 1.0f : (float)(1 << (8 - R));
    static constexpr float byte_coef = (0.5f - (float)(1 << (R - 1))) * (float)(1 << (8 - R));
};

// grid: (ceil(n / 256), ceil(batch / 128), splits); block 512.  Groups
// [z * gps, min(G, (z + 1) * gps)) of k.  Split k (splits > 1) needs a
// workspace (part != null): each split stores its partial tile there for
// gemm_reduce_kernel to add in a fixed order.  ASYM:
// asymmetric children, zeros bf16 [n][k/128]: each weight gains
// s * (127.5 - z) over the symmetric child, i.e. the product gains
// s * (127.5 - z) * (group sum of the batch row's X), added through the same
// fp32 product as the corrections (in accumulator units: divided by the
// final scaling GemmOperand<R>::post).
template <int R, bool ASYM>
__global__ __launch_bounds__(64 * GEMM_WAVES) void gemm_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int batch, const uint8_t *__restrict__ planes,
    int64_t plane_bytes, const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    int n, int k, int gps, float *__restrict__ y, int64_t ldy, int ybf16,
    float *__restrict__ part) {
    __shared__ __align__(16) uint16_t xs[2][GEMM_BM * GEMM_XSTRIDE];
    // corrections (and group sums of X) of the last four groups, per batch row:
    // while group g runs, the pair (g-2, g-1) is read and g+1 is staged
    __shared__ __align__(16) float corr[4][GEMM_BM];
    __shared__ __align__(16) float xsum[ASYM ? 4 : 1][GEMM_BM];
    constexpr bool BYTES = GemmOperand<R>::bytes;
    constexpr float POST = GemmOperand<R>::post;

    const int G = k >> 7;
    const int g_begin = blockIdx.z * gps;
    const int g_end = min(G, g_begin + gps);
    if (g_begin >= g_end) return;  // uniform over the workgroup

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int b0 = blockIdx.y * GEMM_BM;
    const int npad = (n + 15) & ~15;

    // This lane's weight row and the base of its 8 bytes in plane 0, group 0.
    const int nrow = blockIdx.x * GEMM_BN + 32 * w + l32;
    const int rc = min(nrow, npad - 1);
    const uint8_t *pbase = planes + ((int64_t)(rc >> 4) * G * 16 + (rc & 15)) * 16 + 8 * h;
    const uint16_t *sbase = scales + (int64_t)min(nrow, n - 1) * G;
    const uint16_t *zbase = ASYM ? zeros + (int64_t)min(nrow, n - 1) * G : nullptr;

    // X staging: thread (xr, qq) moves columns 32qq .. 32qq+31 (word qq of the
    // group: bf16 pairs m = 0..15) of batch row b0 + xr.
    const int xr = tid >> 2, qq = tid & 3;
    const uint16_t *xrow = x + (int64_t)min(b0 + xr, batch - 1) * ldx + 32 * qq;
    u32x4_t xv[4];
    auto load_x = [&](int g) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            xv[c] = *reinterpret_cast<const u32x4_t *>(xrow + 128 * g + 8 * c);
    };
    auto stage_x = [&](int buf, int slot) {
        uint32_t xw[16];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            *reinterpret_cast<u32x4_t *>(&xs[buf][xr * GEMM_XSTRIDE + 32 * qq + 8 * c]) = xv[c];
            xw[4 * c] = xv[c].x;
            xw[4 * c + 1] = xv[c].y;
            xw[4 * c + 2] = xv[c].z;
            xw[4 * c + 3] = xv[c].w;
        }
        // This thread's share of the row's correction (pairs m = 0..15 of
        // word qq), then the sum over the row's four threads (one quad).
        float own;
        if constexpr (BYTES) {
            const uint32_t one = 0x3F803F80u;  // bf16 (1.0, 1.0)
            float c0 = 0.f, c1 = 0.f;
#pragma unroll
            for (int m = 0; m < 16; m += 2) {
                c0 = gm_dot2(one, xw[m], c0);
                c1 = gm_dot2(one, xw[m + 1], c1);
            }
            own = GemmOperand<R>::byte_coef * (c0 + c1);
        } else {
            own = correction<R, 16>(xw);
        }
        const float cpart = quad_sum(own);
        if (qq == 0) corr[slot][xr] = cpart;
        if constexpr (ASYM) {
            const uint32_t one = 0x3F803F80u;  // bf16 (1.0, 1.0)
            float sx0 = 0.f, sx1 = 0.f;
#pragma unroll
            for (int m = 0; m < 16; m += 2) {
                sx0 = gm_dot2(one, xw[m], sx0);
                sx1 = gm_dot2(one, xw[m + 1], sx1);
            }
            const float sx = quad_sum(sx0 + sx1);
            if (qq == 0) xsum[slot][xr] = sx;
        }
    };

    // Planes and scale of the next group to decode.  They are reloaded right
    // after each decode (one group ahead), so no register copy -- which
    // would wait for the load it copies -- is ever needed.
    u32x2_t pw[R];
    uint32_t sraw, zraw;
    auto load_w = [&](int g) {
        const uint8_t *c = pbase + (int64_t)g * 256;
#pragma unroll
        for (int p = 0; p < R; ++p)
            pw[p] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x2_t *>(c + (int64_t)p * plane_bytes));
        sraw = sbase[g];
        if constexpr (ASYM) zraw = zbase[g];
    };

    load_x(g_begin);
    load_w(g_begin);
    stage_x(0, 0);
    __syncthreads();

    f32x16_t acc[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[bb][v] = 0.f;

    // The corrections enter through the fp32 matrix path, not the chains:
    // sum_g s[n][g] * corr[b][g] (and, asymmetric, sum_g s*zc[n][g] * xsum[b][g])
    // is a product over groups, added into acc two groups at a time with
    // v_mfma_f32_32x32x2_f32 (A: corrections [batch row][group], B: scales
    // [group][weight row]); lane half h takes the pair's group h.
    // (all reads first, then the MFMAs: one wait for the four reads)
    auto correct = [&](int slot_h, float bv, float bv2) {
        float a[4], a2[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            a[bb] = corr[slot_h][32 * bb + l32];
            if constexpr (ASYM) a2[bb] = xsum[slot_h][32 * bb + l32];
        }
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            acc[bb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[bb], bv, acc[bb], 0, 0, 0);
            if constexpr (ASYM)
                acc[bb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a2[bb], bv2, acc[bb], 0, 0, 0);
        }
    };
    // scales (and scale * zc) of the last two groups, for their pair's correction
    float s_prev = 0.f, zs_prev = 0.f, s_prev2 = 0.f, zs_prev2 = 0.f;

    for (int g = g_begin; g < g_end; ++g) {
        const int buf = (g - g_begin) & 1;
        const int slot = (g - g_begin) & 3;
        // X of the next group first, ahead of everything else in the group:
        // it is staged at the group's end and should arrive well before.
        // Loads retire in order, so staging X then waits only for X (an L2
        // hit), not for the planes coming from HBM.  The loads are
        // unconditional (clamped to the last group), so the number in flight
        // behind X is static and the compiler's wait for X stays exact.
        const int gn = min(g + 1, g_end - 1);
        load_x(gn);
        __builtin_amdgcn_sched_barrier(0);

        // Decode this group's weight operands: Bop[pair].
        uint32_t Bop[32];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            uint32_t P[R];
#pragma unroll
            for (int p = 0; p < R; ++p) P[p] = q ? pw[p].y : pw[p].x;
            if constexpr (BYTES) {
                decode_word_bytes<R>(P, Bop + 16 * q);
            } else {
                uint32_t D1[16];
                decode_word<R>(P, Bop + 16 * q, D1);
            }
        }
        float s = nrow < n ? __uint_as_float(sraw << 16) : 0.f;
        float zc = ASYM ? (127.5f - __uint_as_float(zraw << 16)) *
                              (1.0f / POST)
                        : 0.f;
        // Materialise them here, before sraw / zraw are reloaded: computed
        // after the reload, the old values would need a register copy at the
        // loop's end, and a copy waits for every load in flight (the planes
        // from HBM included).
        asm volatile("" : "+v"(s));
        if constexpr (ASYM) asm volatile("" : "+v"(zc));
        // Groups g-2, g-1 form a finished pair: their corrections go in now,
        // next to this group's decode (their slots are not written again
        // before the barrier after group g+1).
        if (g - g_begin >= 2 && ((g - g_begin) & 1) == 0)
            correct(h ? (slot + 3) & 3 : (slot + 2) & 3, h ? s_prev : s_prev2, h ? zs_prev : zs_prev2);

        // The planes of the next group.
        load_w(gn);

#pragma unroll
        for (int bp = 0; bp < 2; ++bp) {
            // Two batch blocks, chains interleaved, each from zero.
            f32x16_t Pc[2];
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int v = 0; v < 16; ++v) Pc[e][v] = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int bb = 2 * bp + e;
                    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(
                        &xs[buf][(32 * bb + l32) * GEMM_XSTRIDE + 64 * h + 8 * j]);
                    const u32x4_t wv = {Bop[4 * j], Bop[4 * j + 1], Bop[4 * j + 2], Bop[4 * j + 3]};
                    Pc[e] = gm_mfma(a, wv, Pc[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[2 * bp + e][v] = fmaf(s, Pc[e][v], acc[2 * bp + e][v]);
        }

        s_prev2 = s_prev;
        zs_prev2 = zs_prev;
        s_prev = s;
        zs_prev = ASYM ? s * zc : 0.f;

        // (kept after the MFMAs: scheduled among them, the staging's reads
        // of X would stall the chains on the X loads)
        __builtin_amdgcn_sched_barrier(0);
        stage_x(buf ^ 1, (slot + 1) & 3);  // (past the end: a repeat of the last group, never read)
        __syncthreads();
    }
    // The last pair, or an unpaired last group through the h = 0 lanes (the
    // h = 1 lanes multiply a valid correction by zero).
    {
        const int ng = g_end - g_begin;
        const int last = (ng - 1) & 3;
        if (ng & 1)
            correct(last, h ? 0.f : s_prev, h ? 0.f : zs_prev);
        else
            correct(h ? last : (last + 3) & 3, h ? s_prev : s_prev2, h ? zs_prev : zs_prev2);
    }

    // Split k through the workspace: store the raw partial tile and leave
    // the sum and the output to gemm_reduce_kernel (a later launch, so no
    // fence or counter is needed between the splits).
    if (part) {
        float *dst = part + ((size_t)blockIdx.z * gridDim.x * gridDim.y +
                             blockIdx.y * gridDim.x + blockIdx.x) * GEMM_TILE;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<float4 *>(dst + gemm_part_offset(bb, q, tid)) =
                    make_float4(acc[bb][4 * q], acc[bb][4 * q + 1], acc[bb][4 * q + 2], acc[bb][4 * q + 3]);
        return;
    }

    // Epilogue: lane holds rows b0 + 32bb + 8(v/4) + 4h + v%4 of column nrow.
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
        gemm_store_block(acc[bb], b0 + 32 * bb, h, nrow, n, batch, POST, y, ldy, ybf16);
}

// Adds the S partial tiles of a split launch in the order z = 0..S-1 and
// stores y (deterministic: the same sum on every run, any output type).
// grid: (ceil(n / 256), ceil(batch / 128), 8 waves x 4 batch blocks); block
// 64: workgroup (x, y, 4w + bb) finishes accumulator block bb of wave w of
// the GEMM workgroup (x, y), with the GEMM's lane-to-element mapping.
__global__ __launch_bounds__(64) void gemm_reduce_kernel(const float *__restrict__ part, int S,
                                                         int batch, int n, float post,
                                                         float *__restrict__ y, int64_t ldy,
                                                         int ybf16) {
    const int lane = threadIdx.x;
    const int w = blockIdx.z >> 2, bb = blockIdx.z & 3;
    const int tid = w * 64 + lane;
    const int ntiles = gridDim.x * gridDim.y;
    const float *src = part + (size_t)(blockIdx.y * gridDim.x + blockIdx.x) * GEMM_TILE;
    f32x16_t tot;
#pragma unroll
    for (int v = 0; v < 16; ++v) tot[v] = 0.f;
    // Four splits per round: their 16 loads are all in flight before the
    // first add (clamped at the end, so the count is static), and the adds
    // keep the order z = 0, 1, ..., S-1.
    for (int z0 = 0; z0 < S; z0 += 4) {
        float4 v[4][4];
#pragma unroll
        for (int zz = 0; zz < 4; ++zz)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                v[zz][q] = *reinterpret_cast<const float4 *>(
                    src + (size_t)min(z0 + zz, S - 1) * ntiles * GEMM_TILE +
                    gemm_part_offset(bb, q, tid));
        // (a repeat past the last split adds zero: a select, not a branch,
        // so the loads stay ahead of every add)
#pragma unroll
        for (int zz = 0; zz < 4; ++zz) {
            const bool live = z0 + zz < S;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                tot[4 * q] += live ? v[zz][q].x : 0.f;
                tot[4 * q + 1] += live ? v[zz][q].y : 0.f;
                tot[4 * q + 2] += live ? v[zz][q].z : 0.f;
                tot[4 * q + 3] += live ? v[zz][q].w : 0.f;
            }
        }
    }
    const int nrow = blockIdx.x * GEMM_BN + 32 * w + (lane & 31);
    gemm_store_block(tot, blockIdx.y * GEMM_BM + 32 * bb, lane >> 5, nrow, n, batch, post, y, ldy,
                     ybf16);
}

// Split k only when the output tiles leave most CUs idle.  Each split keeps
// at least min_groups groups.
static int gemm_tiles(const QgemmArgs &a) {
    return (a.n + GEMM_BN - 1) / GEMM_BN * (int)((a.batch + GEMM_BM - 1) / GEMM_BM);
}

static int gemm_splits(const QgemmArgs &a, int cu_count, int min_groups) {
    const int tiles = gemm_tiles(a);
    const int G = a.k / 128;
    int s = 1;
    while (tiles * s * 2 <= cu_count && G / (2 * s) >= min_groups) s *= 2;
    return s;
}

constexpr int GEMM_WS_MIN_GROUPS = 4;

// Splits that hold at least one group when each takes ceil(G / splits).
static int gemm_live_splits(int G, int splits) {
    const int gps = (G + splits - 1) / splits;
    return (G + gps - 1) / gps;
}

// Workspace of the deterministic split (splits x tiles partial tiles of
// fp32) of this kernel, which takes asymmetric children.
static int64_t gemm_asym_workspace_bytes(const QgemmArgs &a, int cu_count) {
    const int splits = gemm_live_splits(a.k / 128, gemm_splits(a, cu_count, GEMM_WS_MIN_GROUPS));
    if (splits <= 1) return 0;
    return (int64_t)splits * gemm_tiles(a) * GEMM_TILE * 4;
}

// Workspace that covers either large-batch kernel (symmetric children take
// gemm_wide_kernel, asymmetric ones this file's kernel).
int64_t gemm_workspace_bytes(const QgemmArgs &a, int cu_count) {
    const int64_t sym = gemm_wide_workspace_bytes(a, cu_count);
    const int64_t asym = gemm_asym_workspace_bytes(a, cu_count);
    return sym > asym ? sym : asym;
}

template <int R>
static void launch_r(const QgemmArgs &a, int cu_count, hipStream_t stream) {
    const int G = a.k / 128;
    // The splits meet only in a large enough caller workspace (a fixed order,
    // so the result is deterministic); without one the launch runs unsplit.
    const int64_t need = gemm_asym_workspace_bytes(a, cu_count);
    const bool use_ws = need > 0 && a.ws && a.ws_bytes >= need;
    const int want = use_ws ? gemm_splits(a, cu_count, GEMM_WS_MIN_GROUPS) : 1;
    const int gps = (G + want - 1) / want;
    const int splits = gemm_live_splits(G, want);
    float *part = use_ws ? static_cast<float *>(a.ws) : nullptr;
    const dim3 grid((a.n + GEMM_BN - 1) / GEMM_BN, (unsigned)((a.batch + GEMM_BM - 1) / GEMM_BM),
                    splits);
    if (a.zeros)
        hipLaunchKernelGGL((gemm_kernel<R, true>), grid, dim3(GEMM_THREADS), 0, stream, a.x,
                           a.ldx, (int)a.batch, a.planes, a.plane_bytes, a.scales, a.zeros, a.n, a.k,
                           gps, a.y, a.ldy, a.ybf16, part);
    else
        hipLaunchKernelGGL((gemm_kernel<R, false>), grid, dim3(GEMM_THREADS), 0, stream, a.x,
                           a.ldx, (int)a.batch, a.planes, a.plane_bytes, a.scales, a.zeros, a.n, a.k,
                           gps, a.y, a.ldy, a.ybf16, part);
    if (part)
        hipLaunchKernelGGL(gemm_reduce_kernel, dim3(grid.x, grid.y, 4 * GEMM_WAVES), dim3(64), 0,
                           stream, part, splits, (int)a.batch, a.n, GemmOperand<R>::post, a.y,
                           a.ldy, a.ybf16);
}

hipError_t launch_gemm(int r, const QgemmArgs &a, int cu_count, hipStream_t stream) {
    if (!a.zeros) return launch_gemm_wide(r, a, cu_count, stream);
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

void gemm_name(int r, const QgemmArgs &a, int cu_count, char *out, size_t len) {
    (void)cu_count;
    if (!a.zeros)
        gemm_wide_name(r, a, out, len);
    else
        snprintf(out, len, "nbw::gemm_kernel<%d, true>", r);
}

}  // namespace nbw
