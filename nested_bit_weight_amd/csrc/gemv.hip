// gemv.hip -- small-batch dequant-GEMV (VALU), gfx950.
//
// Y[b][i] = sum_j X[b][j] * s[i][j/128] * 2^(8-r) * (q_r[i][j] + 1/2 - 2^(r-1)),
// the r-bit child of a sliceable parent (MatGPTQ: Efficient and Accurate
// Inference over Nested Quantized Models, Abstract: lower precisions read
// fewer bits of the weights; Figure 1: the kernels run at 2..8 bits).
//
// At batch 1 this product is bound by HBM: r/8 bytes of planes per weight,
// one multiply-add per weight.  The kernel streams the r planes once and
// spends its VALU budget on the decode:
//
//  - lane (i, gg) of a wave owns row i of a 16-row tile and group g = 4*set+gg
//    of a 4-group set.  The wave's four 16-lane quarters read 4 x 256 = 1 KB
//    of contiguous plane bytes per plane and tile (the layout puts the 16 rows
//    of one group next to each other), with 128-bit loads.
//  - the lane keeps its group's 128 activations in registers as 64 bf16 pairs
//    for the whole set, walking down the tiles of its workgroup, so X is read
//    once per set and every plane byte exactly once.
//  - decode: bit-plane transpose network + one shift/and-or per bf16 pair
//    (decode.h), then v_dot2_f32_bf16 with the activation pair.  The constant
//    offsets of the decoded operands are cancelled by a per-lane correction
//    computed once per set.
//  - the group scale is folded in fp32 once per (row, group).
//  - the four group partials of a row meet through two cross-lane exchanges,
//    the waves of the workgroup (which split k) through LDS.
#include <cstdio>

#include "decode.h"
#include "launch.h"

namespace nbw {

constexpr int GEMV_MAX_WAVES = 8;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// NB: batch rows handled per launch slice (1 or 2); TM: tiles per workgroup.
template <int R, int NB, int TM>
__global__ __launch_bounds__(512) void gemv_kernel(const uint16_t *__restrict__ x, int nbv,
                                                   const uint8_t *__restrict__ planes,
                                                   int64_t plane_bytes,
                                                   const uint16_t *__restrict__ scales, int n,
                                                   int k, int tiles_total,
                                                   float *__restrict__ y) {
    __shared__ float red[GEMV_MAX_WAVES][TM][NB][16];
    const int G = k >> 7;
    const int nsets = (G + 3) >> 2;
    const int W = blockDim.x >> 6;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int i = lane & 15, gg = lane >> 4;
    const int tile0 = blockIdx.x * TM;
    const int tcount = min(TM, tiles_total - tile0);

    float acc[TM][NB];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[t][b] = 0.f;

    for (int set = w; set < nsets; set += W) {
        const int g = 4 * set + gg;
        const bool gvalid = g < G;
        const int gc = gvalid ? g : G - 1;

        // Activations of this lane's group, as 64 bf16 pairs per batch row.
        uint32_t X2[NB][64];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const bool ok = gvalid && b < nbv;
            const int bc = b < nbv ? b : nbv - 1;  // clamped: never form an address past X
            const uint4 *src = reinterpret_cast<const uint4 *>(x + (int64_t)bc * k + 128 * gc);
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                uint4 v = ok ? src[q] : make_uint4(0u, 0u, 0u, 0u);
                X2[b][4 * q] = v.x; X2[b][4 * q + 1] = v.y;
                X2[b][4 * q + 2] = v.z; X2[b][4 * q + 3] = v.w;
            }
        }
        // corr = sum_k x_k * (1/2 - 2^(R-1) - offset_k): turns the decoded
        // operands (offset_k + q_k) into (q_k + 1/2 - 2^(R-1)).
        float corr[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float o = 0.f, sx = 0.f;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                o = offset_dot<R>(X2[b] + 16 * d, o);
                sx = pair_sum(X2[b] + 16 * d, sx);
            }
            corr[b] = fmaf(0.5f - (float)(1 << (R - 1)), sx, -o);
        }

        // Planes of this lane's (row, group) chunk for the workgroup's tiles.
        uint32_t pl[TM][R][4];
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const int tile = min(tile0 + t, tiles_total - 1);
            const uint8_t *base = planes + (((int64_t)tile * G + gc) * 16 + i) * 16;
#pragma unroll
            for (int p = 0; p < R; ++p) {
                const u32x4_t v = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4_t *>(base + p * plane_bytes));
                pl[t][p][0] = v.x; pl[t][p][1] = v.y; pl[t][p][2] = v.z; pl[t][p][3] = v.w;
            }
        }

#pragma unroll
        for (int t = 0; t < TM; ++t) {
            float P[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) P[b] = 0.f;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t Pw[R];
#pragma unroll
                for (int p = 0; p < R; ++p) Pw[p] = pl[t][p][d];
                uint32_t D0[16], D1[16];
                decode_word<R>(Pw, D0, D1);
#pragma unroll
                for (int m = 0; m < 16; ++m)
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        P[b] = dot2(D0[m], X2[b][16 * d + m], P[b]);
                        if constexpr (Phases<R>::count == 2)
                            P[b] = dot2(D1[m], X2[b][16 * d + m], P[b]);
                    }
            }
            const int row = 16 * (tile0 + t) + i;
            float s = 0.f;
            if (gvalid && t < tcount && row < n) s = bf16_bits_to_f32(scales[(int64_t)row * G + g]);
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[t][b] = fmaf(s, P[b] + corr[b], acc[t][b]);
        }
    }

    // The four lanes of a row (one per group of the set) -> one value.
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float v = acc[t][b];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            if (gg == 0) red[w][t][b][i] = v;
        }
    __syncthreads();
    const float post = (float)(1 << (8 - R));
    for (int e = threadIdx.x; e < TM * NB * 16; e += blockDim.x) {
        const int t = e / (NB * 16), b = (e / 16) % NB, ii = e & 15;
        float sum = 0.f;
        for (int ww = 0; ww < W; ++ww) sum += red[ww][t][b][ii];
        const int row = 16 * (tile0 + t) + ii;
        if (t < tcount && row < n && b < nbv) y[(int64_t)b * n + row] = sum * post;
    }
}

template <int R, int NB, int TM>
static void launch_one(const QgemmArgs &a, int64_t b0, int nbv, int waves, hipStream_t stream) {
    const int tiles = (a.n + 15) / 16;
    dim3 grid((unsigned)((tiles + TM - 1) / TM));
    hipLaunchKernelGGL((gemv_kernel<R, NB, TM>), grid, dim3(64 * waves), 0, stream,
                       a.x + b0 * a.k, nbv, a.planes, a.plane_bytes, a.scales, a.n, a.k, tiles,
                       a.y + b0 * a.n);
}

// Launch shape: waves per workgroup (they split k), tiles per workgroup.
struct GemvPlan {
    int waves, tm;
};

static GemvPlan gemv_plan(const QgemmArgs &a, int cu_count) {
    const int G = a.k / 128;
    const int nsets = (G + 3) / 4;
    const int tiles = (a.n + 15) / 16;
    GemvPlan p;
    p.waves = nsets < GEMV_MAX_WAVES ? nsets : GEMV_MAX_WAVES;
    p.tm = tiles >= 4 * cu_count ? 2 : 1;  // two tiles per workgroup only when >= 2 workgroups per CU remain
    return p;
}

template <int R>
static void launch_r(const QgemmArgs &a, int cu_count, hipStream_t stream) {
    const GemvPlan plan = gemv_plan(a, cu_count);
    for (int64_t b0 = 0; b0 < a.batch; b0 += 2) {
        const int nbv = (int)((a.batch - b0) < 2 ? (a.batch - b0) : 2);
        if (nbv == 1) {
            if (plan.tm == 2) launch_one<R, 1, 2>(a, b0, nbv, plan.waves, stream);
            else launch_one<R, 1, 1>(a, b0, nbv, plan.waves, stream);
        } else {
            if (plan.tm == 2) launch_one<R, 2, 2>(a, b0, nbv, plan.waves, stream);
            else launch_one<R, 2, 1>(a, b0, nbv, plan.waves, stream);
        }
    }
}

void gemv_name(int r, const QgemmArgs &a, int cu_count, char *out, size_t len) {
    const GemvPlan plan = gemv_plan(a, cu_count);
    snprintf(out, len, "nbw::gemv_kernel<%d, %d, %d>", r, a.batch >= 2 ? 2 : 1, plan.tm);
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

}  // namespace nbw
