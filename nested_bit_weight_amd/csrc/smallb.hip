// smallb.hip -- small-batch dequant-GEMM on MFMA, gfx950.
//
// Same product as gemv.hip (MatGPTQ: Efficient and Accurate Inference over
// Nested Quantized Models, Abstract: kernels supporting batch sizes beyond
// one; Figure 1: batch sweep), for 2..16 batch rows per launch slice.  Beyond
// one batch row the bf16 dot products would take more VALU issue slots than
// the plane decode itself, so the contraction moves to the matrix cores:
//
//  - one v_mfma_f32_16x16x32_bf16 multiplies a 16-row x 32-column weight
//    fragment by 32 columns of up to 16 batch rows.  Lane l supplies row l%16,
//    k-quarter l/16 of the weight fragment, and batch row l%16, k-quarter l/16
//    of the activations; the k-slot order inside a quarter only has to agree
//    between the two operands, so each lane feeds its decoded plane word in
//    the order the decoder produces it (pairs 4j..4j+3 -> MFMA j).
//  - lane (row c, quarter d) of a wave loads 32-bit word d of its row's
//    16-byte chunk of each plane: one wave load covers the 256 contiguous
//    bytes of a 16-row tile of one group.
//  - every MFMA chain covers one 128-wide group, so the group scale is folded
//    in fp32 right after it (one FMA per output); the chain starts from the
//    correction that removes the decoded operands' constant offsets.
//  - a wave keeps the activation operands of its 4-group set in registers
//    and walks the tiles of its workgroup; waves split k and meet in LDS.
#include <cstdio>

#include "decode.h"
#include "launch.h"

namespace nbw {

constexpr int SMALLB_MAX_WAVES = 8;

__device__ __forceinline__ float sb_bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

template <int R, int TM>
__global__ __launch_bounds__(512) void smallb_kernel(const uint16_t *__restrict__ x, int64_t batch,
                                                     int64_t ldx,
                                                     const uint8_t *__restrict__ planes,
                                                     int64_t plane_bytes,
                                                     const uint16_t *__restrict__ scales,
                                                     const uint16_t *__restrict__ zeros, int n,
                                                     int k, int tiles_total,
                                                     float *__restrict__ y, int64_t ldy,
                                                     int ybf16) {
    __shared__ float red[SMALLB_MAX_WAVES][TM][4][64];
    const int G = k >> 7;
    const int nsets = (G + 3) >> 2;
    const int W = blockDim.x >> 6;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, d = lane >> 4;
    const int tile0 = blockIdx.x * TM;
    const int tcount = min(TM, tiles_total - tile0);
    const int64_t bcol = (int64_t)blockIdx.y * 16 + c;
    const bool bvalid = bcol < batch;
    const int64_t bclamp = bvalid ? bcol : batch - 1;

    f32x4_t acc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int set = w; set < nsets; set += W) {
        // Activation operands of the 4 groups: XB[gi][4j+e] is the bf16 pair of
        // columns 128g + 32d + 8j + 2e (+1) of batch row bcol.
        uint32_t XB[4][16];
        f32x4_t init[4];
        float xsum[4];  // group sums of this batch row's X (asymmetric term)
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            const int g = 4 * set + gi;
            const bool ok = bvalid && g < G;
            const int gc = g < G ? g : G - 1;
            const u32x4_t *src =
                reinterpret_cast<const u32x4_t *>(x + bclamp * ldx + 128 * gc + 32 * d);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4_t v = ok ? src[j] : u32x4_t{0u, 0u, 0u, 0u};
                XB[gi][4 * j] = v.x; XB[gi][4 * j + 1] = v.y;
                XB[gi][4 * j + 2] = v.z; XB[gi][4 * j + 3] = v.w;
            }
            float corr = correction<R, 16>(XB[gi]);
            corr += __shfl_xor(corr, 16);
            corr += __shfl_xor(corr, 32);
            init[gi] = f32x4_t{corr, corr, corr, corr};
            xsum[gi] = 0.f;
            if (zeros) {
                const uint32_t one = 0x3F803F80u;
                float sx = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    sx = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, one),
                                                         __builtin_bit_cast(bf16x2_t, XB[gi][m]),
                                                         sx, false);
                sx += __shfl_xor(sx, 16);
                sx += __shfl_xor(sx, 32);
                xsum[gi] = sx;
            }
        }

        // Plane words: lane (c, d) reads word d of row c's chunk, per plane.
        uint32_t pl[TM][4][R];
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const int tile = min(tile0 + t, tiles_total - 1);
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int g = 4 * set + gi;
                const int gc = g < G ? g : G - 1;
                const uint8_t *base = planes + (((int64_t)tile * G + gc) * 16 + c) * 16 + 4 * d;
#pragma unroll
                for (int p = 0; p < R; ++p)
                    pl[t][gi][p] = __builtin_nontemporal_load(
                        reinterpret_cast<const uint32_t *>(base + p * plane_bytes));
            }
        }

#pragma unroll
        for (int t = 0; t < TM; ++t) {
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int g = 4 * set + gi;
                uint32_t D0[16], D1[16];
                decode_word<R>(pl[t][gi], D0, D1);
                f32x4_t P = init[gi];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32x4_t xb = {XB[gi][4 * j], XB[gi][4 * j + 1], XB[gi][4 * j + 2],
                                        XB[gi][4 * j + 3]};
                    const u32x4_t a0 = {D0[4 * j], D0[4 * j + 1], D0[4 * j + 2], D0[4 * j + 3]};
                    P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0),
                                                                __builtin_bit_cast(bf16x8_t, xb), P,
                                                                0, 0, 0);
                    if constexpr (Phases<R>::count == 2) {
                        const u32x4_t a1 = {D1[4 * j], D1[4 * j + 1], D1[4 * j + 2],
                                            D1[4 * j + 3]};
                        P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, a1), __builtin_bit_cast(bf16x8_t, xb), P,
                            0, 0, 0);
                    }
                }
                // Output layout: this lane holds rows 4d..4d+3 of the tile, batch bcol.
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = 16 * (tile0 + t) + 4 * d + v;
                    float s = 0.f, pv = P[v];
                    if (g < G && t < tcount && row < n) {
                        s = sb_bf16_to_f32(scales[(int64_t)row * G + g]);
                        if (zeros) {  // + (127.5 - z) * 2^(R-8) * group sum of X
                            const float z = sb_bf16_to_f32(zeros[(int64_t)row * G + g]);
                            pv = fmaf((127.5f - z) * (1.0f / (float)(1 << (8 - R))), xsum[gi], pv);
                        }
                    }
                    acc[t][v] = fmaf(s, pv, acc[t][v]);
                }
            }
        }
    }

#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[w][t][v][lane] = acc[t][v];
    __syncthreads();
    const float post = (float)(1 << (8 - R));
    for (int e = threadIdx.x; e < TM * 4 * 64; e += blockDim.x) {
        const int t = e / 256, v = (e / 64) & 3, l = e & 63;
        float sum = 0.f;
        for (int ww = 0; ww < W; ++ww) sum += red[ww][t][v][l];
        const int row = 16 * (tile0 + t) + 4 * (l >> 4) + v;
        const int64_t b = (int64_t)blockIdx.y * 16 + (l & 15);
        if (t < tcount && row < n && b < batch) store_y(y, ybf16, b * ldy + row, sum * post);
    }
}

template <int R, int TM>
static void launch_tm(const QgemmArgs &a, int waves, hipStream_t stream) {
    const int tiles = (a.n + 15) / 16;
    dim3 grid((unsigned)((tiles + TM - 1) / TM), (unsigned)((a.batch + 15) / 16));
    hipLaunchKernelGGL((smallb_kernel<R, TM>), grid, dim3(64 * waves), 0, stream, a.x, a.batch,
                       a.ldx, a.planes, a.plane_bytes, a.scales, a.zeros, a.n, a.k, tiles, a.y,
                       a.ldy, a.ybf16);
}

static int smallb_tm(const QgemmArgs &a, int cu_count) {
    const int tiles = (a.n + 15) / 16;
    return tiles >= 4 * cu_count ? 2 : 1;
}

template <int R>
static void launch_r(const QgemmArgs &a, int cu_count, hipStream_t stream) {
    const int G = a.k / 128;
    const int nsets = (G + 3) / 4;
    const int waves = nsets < SMALLB_MAX_WAVES ? nsets : SMALLB_MAX_WAVES;
    if (smallb_tm(a, cu_count) == 2) launch_tm<R, 2>(a, waves, stream);
    else launch_tm<R, 1>(a, waves, stream);
}

void smallb_name(int r, const QgemmArgs &a, int cu_count, char *out, size_t len) {
    snprintf(out, len, "nbw::smallb_kernel<%d, %d>", r, smallb_tm(a, cu_count));
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
