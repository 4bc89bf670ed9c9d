// gemv.hip -- batch-1 dequant-GEMV (VALU), gfx950, single and grouped launches.
//
// y[i] = sum_j x[j] * s[i][j/128] * 2^(8-r) * (q_r[i][j] + 1/2 - 2^(r-1)),
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
// rate of the decode.  The layout of the work:
//
//  - a workgroup owns a range of T 16-row tiles of one product and all of k;
//    its W waves split k into 4-group sets (wave w: sets w, w+W, ...).
//  - lane (i, gg) of a wave holds row i of the tile and group 4*set+gg: the
//    wave's four 16-lane quarters read 4 x 256 contiguous plane bytes per
//    plane and tile with 128-bit loads.
//  - each wave walks its (set, tile) steps as one stream with PD steps of
//    planes and scales in flight; all loads are unconditional (clamped at the
//    end), so the loads-in-flight count between a load and its use is static.
//  - the activations and the per-group offset corrections are staged in LDS
//    once per workgroup; a set switch reloads the lane's 64 bf16 activation
//    pairs from LDS without touching the memory pipeline.
//  - decode: bit-plane transpose network + one shift / and-or per bf16 pair
//    (decode.h), then v_dot2_f32_bf16; the group scale is folded in fp32 once
//    per (row, group); the four groups of a set meet through two cross-lane
//    exchanges and the waves in LDS, in a fixed order.
#include <cstdio>

#include "decode.h"
#include "launch.h"

namespace nbw {

constexpr int GEMV_WAVES = 4;       // waves per workgroup: two workgroups share a CU
constexpr int GEMV_MAX_TILES = 16;  // tiles per workgroup
constexpr int GEMV_MAX_GROUP = 32;  // products per grouped launch

// Steps of planes a wave keeps in flight: about 16 x 16-byte loads per lane.
__host__ __device__ constexpr int gemv_depth(int r) {
    return r <= 2 ? 8 : (r == 3 ? 5 : (r == 4 ? 4 : 2));
}

// Dynamic LDS: X bf16 [k] | corr fp32 [k/128] | per-lane partial sums fp32
// [W][GEMV_MAX_TILES][64].
__host__ __device__ constexpr size_t gemv_lds_bytes(int k, int waves) {
    return (size_t)k * 2 + (size_t)(k / 128) * 4 + (size_t)waves * GEMV_MAX_TILES * 64 * 4;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// One workgroup: tiles [t_begin, t_begin + T) of one product, all of k.
template <int R, int PD>
__device__ __forceinline__ void gemv_tiles(const uint16_t *__restrict__ x,
                                           const uint8_t *__restrict__ planes,
                                           int64_t plane_bytes,
                                           const uint16_t *__restrict__ scales, int n, int k,
                                           int t_begin, int T, float *__restrict__ y,
                                           unsigned char *lds) {
    const int G = k >> 7;
    const int nsets = (G + 3) >> 2;
    const int W = blockDim.x >> 6;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int i = lane & 15, gg = lane >> 4;
    uint32_t *xs = reinterpret_cast<uint32_t *>(lds);                  // [k/2] bf16 pairs
    float *corr = reinterpret_cast<float *>(lds + (size_t)k * 2);      // [G]
    float *red = corr + G;                                             // [W][GEMV_MAX_TILES][64]

    // This wave's (set, tile) steps: set ordinal s = 0 .. my_sets-1 is set
    // w + s*W, tile t = 0 .. T-1; step u = s*T + t.
    const int my_sets = nsets > w ? (nsets - w + W - 1) / W : 0;
    const int U = my_sets * T;

    // 1. Prefetch the first PD steps (planes + the scale word of each).
    u32x4_t buf[PD][R];
    uint32_t sbuf[PD];
    int ps = 0, pt = 0;  // next step to prefetch
    auto load_step = [&](int j) {
        // clamped to the last step: past the end the load repeats it (L2 hit)
        int s = ps, t = pt;
        if (s >= my_sets) {
            s = my_sets - 1;
            t = T - 1;
        }
        const int g = min(4 * (w + s * W) + gg, G - 1);
        const uint8_t *c = planes + (((int64_t)(t_begin + t) * G + g) * 16 + i) * 16;
#pragma unroll
        for (int p = 0; p < R; ++p)
            buf[j][p] =
                __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(c + p * plane_bytes));
        // The aligned 32-bit word holding this lane's bf16 scale (in bounds:
        // the host sends only even group counts here).  A 16-bit load would
        // need a zero-extension that the compiler may put where it waits for
        // every load in flight.
        const int row = min(16 * (t_begin + t) + i, n - 1);
        const int64_t idx = (int64_t)row * G + g;
        sbuf[j] = *reinterpret_cast<const uint32_t *>(scales + (idx & ~(int64_t)1));
        if (++pt == T) {
            pt = 0;
            ++ps;
        }
    };
    if (U > 0) {
#pragma unroll
        for (int j = 0; j < PD; ++j) load_step(j);
    }

    // 2. Stage X in LDS and compute the per-group corrections
    //    sum_k x_k * (1/2 - 2^(R-1) - offset_k); zero the partial sums.
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
        uint32_t X2[64];
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(x + 128 * g);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const u32x4_t v = src[q];
            X2[4 * q] = v.x; X2[4 * q + 1] = v.y; X2[4 * q + 2] = v.z; X2[4 * q + 3] = v.w;
            reinterpret_cast<u32x4_t *>(xs + 64 * g)[q] = v;
        }
        corr[g] = correction<R, 64>(X2);
    }
    for (int t = 0; t < T; ++t) red[(w * GEMV_MAX_TILES + t) * 64 + lane] = 0.f;
    __syncthreads();

    // 3. Stream the steps.
    uint32_t X2[64];
    float cg = 0.f;
    int cs = 0, ct = 0;  // step being computed
    auto compute = [&](int j) {
        const int g = 4 * (w + cs * W) + gg;
        const bool gvalid = g < G;
        if (ct == 0) {  // new set: this lane's activations and correction from LDS
            const int gc = gvalid ? g : G - 1;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const u32x4_t v = reinterpret_cast<const u32x4_t *>(xs + 64 * gc)[q];
                X2[4 * q] = v.x; X2[4 * q + 1] = v.y; X2[4 * q + 2] = v.z; X2[4 * q + 3] = v.w;
            }
            cg = corr[gc];
        }
        // four independent dot2 chains (one per 32-column word) keep a wave's
        // dependent-issue latency off the critical path
        float P4[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t Pw[R];
#pragma unroll
            for (int p = 0; p < R; ++p) Pw[p] = buf[j][p][d];
            uint32_t D0[16], D1[16];
            decode_word<R>(Pw, D0, D1);
            float Pd = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                Pd = dot2(D0[m], X2[16 * d + m], Pd);
                if constexpr (Phases<R>::count == 2) Pd = dot2(D1[m], X2[16 * d + m], Pd);
            }
            P4[d] = Pd;
        }
        const float P = (P4[0] + P4[1]) + (P4[2] + P4[3]);
        const int row = 16 * (t_begin + ct) + i;
        const uint32_t sbits = (g & 1) ? (sbuf[j] & 0xFFFF0000u) : (sbuf[j] << 16);
        const float s = (gvalid && row < n) ? __uint_as_float(sbits) : 0.f;
        return s * (P + cg);
    };
    // Accumulate into this lane's own LDS slot for the tile: an add that
    // returns nothing, so the wave does not wait for it.  Each slot has a
    // single writer, so the order of the additions is fixed.
    auto commit = [&](float v) {
        __hip_atomic_fetch_add(&red[(w * GEMV_MAX_TILES + ct) * 64 + lane], v,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
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

    // 4. Rows: add the four groups of each set and the waves, in a fixed order.
    __syncthreads();
    const float post = (float)(1 << (8 - R));
    for (int e = threadIdx.x; e < T * 16; e += blockDim.x) {
        const int t = e >> 4, ii = e & 15;
        float sum = 0.f;
        for (int ww = 0; ww < W; ++ww) {
            const float *slot = red + (ww * GEMV_MAX_TILES + t) * 64 + ii;
            sum += (slot[0] + slot[16]) + (slot[32] + slot[48]);
        }
        const int row = 16 * t_begin + e;
        if (row < n) y[row] = sum * post;
    }
}

// Odd group counts (k = 128 * odd) would need 16-bit scale loads, and very
// large k would not fit X in LDS; these rare shapes take this plain one-tile
// kernel: one workgroup per 16-row tile.
template <int R>
__global__ __launch_bounds__(256) void gemv_odd_kernel(const uint16_t *__restrict__ x,
                                                       const uint8_t *__restrict__ planes,
                                                       int64_t plane_bytes,
                                                       const uint16_t *__restrict__ scales,
                                                       int n, int k, float *__restrict__ y) {
    __shared__ float red[GEMV_WAVES][16];
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
        const uint32_t sb = (uint32_t)scales[(int64_t)min(row, n - 1) * G + gc] << 16;
        const float s = (gvalid && row < n) ? __uint_as_float(sb) : 0.f;
        acc = fmaf(s, P + correction<R, 64>(X2), acc);
    }
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    if (gg == 0) red[w][i] = acc;
    __syncthreads();
    if (threadIdx.x < 16) {
        float sum = 0.f;
        for (int ww = 0; ww < W; ++ww) sum += red[ww][threadIdx.x];
        if (16 * tile + (int)threadIdx.x < n)
            y[16 * tile + threadIdx.x] = sum * (float)(1 << (8 - R));
    }
}

template <int R>
__global__ __launch_bounds__(256) void gemv_kernel(const uint16_t *__restrict__ x,
                                                   const uint8_t *__restrict__ planes,
                                                   int64_t plane_bytes,
                                                   const uint16_t *__restrict__ scales, int n,
                                                   int k, int tiles_total, int tiles_per_wg,
                                                   float *__restrict__ y) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int t_begin = blockIdx.x * tiles_per_wg;
    const int T = min(tiles_per_wg, tiles_total - t_begin);
    gemv_tiles<R, gemv_depth(R)>(x, planes, plane_bytes, scales, n, k, t_begin, T, y, lds);
}

// ---------------------------------------------------------------- grouped launch

struct GemvJob {
    const uint16_t *x;
    const uint8_t *planes;
    int64_t plane_bytes;
    const uint16_t *scales;
    float *y;
    int n, k, r, tiles, tpw, item_begin;
};

struct GemvGroup {
    GemvJob job[GEMV_MAX_GROUP];
    int count;
};

// Workgroup b runs item b; items are numbered product by product.
__global__ __launch_bounds__(256) void gemv_group_kernel(GemvGroup grp) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int item = blockIdx.x;
    int jb = 0;
    while (jb + 1 < grp.count && item >= grp.job[jb + 1].item_begin) ++jb;
    const GemvJob &J = grp.job[jb];
    const int t_begin = (item - J.item_begin) * J.tpw;
    const int T = min(J.tpw, J.tiles - t_begin);
    switch (J.r) {
#define NBW_GEMV_CASE(RR)                                                                        \
    case RR:                                                                                     \
        gemv_tiles<RR, gemv_depth(RR)>(J.x, J.planes, J.plane_bytes, J.scales, J.n, J.k, t_begin, \
                                       T, J.y, lds);                                             \
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

// Tiles per workgroup: items of about `target` plane bytes (large enough to
// amortise a workgroup's start-up, small enough to spread over the CUs),
// at most GEMV_MAX_TILES, and never fewer workgroups than CUs when the
// matrix allows it.
static int gemv_tpw(int n, int k, int r, int cu_count, int64_t target) {
    const int tiles = (n + 15) / 16;
    const int64_t tile_bytes = (int64_t)2 * k * r;  // 16 rows x k/8 bytes x r planes
    int tpw = (int)((target + tile_bytes / 2) / tile_bytes);
    if (tpw < 1) tpw = 1;
    if (tpw > GEMV_MAX_TILES) tpw = GEMV_MAX_TILES;
    const int fill = (tiles + cu_count - 1) / cu_count;  // tiles per WG with one WG per CU
    if (tpw > fill) tpw = fill;
    return tpw;
}

constexpr int64_t GEMV_SINGLE_TARGET = 256 << 10;
constexpr int64_t GEMV_GROUP_TARGET = 256 << 10;

static bool gemv_streamable(int k);

template <int R>
static void launch_r(const QgemmArgs &a, int cu_count, hipStream_t stream) {
    const int tiles = (a.n + 15) / 16;
    for (int64_t b = 0; b < a.batch; ++b) {  // one batch row per launch
        if (!gemv_streamable(a.k)) {
            hipLaunchKernelGGL(gemv_odd_kernel<R>, dim3(tiles), dim3(64 * GEMV_WAVES), 0, stream,
                               a.x + b * a.k, a.planes, a.plane_bytes, a.scales, a.n, a.k,
                               a.y + b * a.n);
        } else {
            const int tpw = gemv_tpw(a.n, a.k, R, cu_count, GEMV_SINGLE_TARGET);
            hipLaunchKernelGGL(gemv_kernel<R>, dim3((tiles + tpw - 1) / tpw),
                               dim3(64 * GEMV_WAVES), gemv_lds_bytes(a.k, GEMV_WAVES), stream,
                               a.x + b * a.k, a.planes, a.plane_bytes, a.scales, a.n, a.k, tiles,
                               tpw, a.y + b * a.n);
        }
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
    (void)cu_count;
    if (!gemv_streamable(a.k))
        snprintf(out, len, "nbw::gemv_odd_kernel<%d>", r);
    else
        snprintf(out, len, "nbw::gemv_kernel<%d>", r);
}

int gemv_group_capacity() { return GEMV_MAX_GROUP; }

// The streaming kernel stages X in LDS and reads scales as aligned words:
// it takes even group counts whose X fits in 64 KB of LDS.
static bool gemv_streamable(int k) {
    return ((k / 128) & 1) == 0 && gemv_lds_bytes(k, GEMV_WAVES) <= 64 * 1024;
}

bool gemv_group_eligible(const QgemmArgs &a) { return a.batch == 1 && gemv_streamable(a.k); }

hipError_t launch_gemv_group(const QgemmArgs *probs, const int *rs, int count, int cu_count,
                             hipStream_t stream) {
    GemvGroup grp = {};
    grp.count = count;
    int items = 0, kmax = 128;
    for (int j = 0; j < count; ++j) {
        const QgemmArgs &a = probs[j];
        GemvJob &J = grp.job[j];
        J.x = a.x;
        J.planes = a.planes;
        J.plane_bytes = a.plane_bytes;
        J.scales = a.scales;
        J.y = a.y;
        J.n = a.n;
        J.k = a.k;
        J.r = rs[j];
        J.tiles = (a.n + 15) / 16;
        J.tpw = gemv_tpw(a.n, a.k, rs[j], cu_count, GEMV_GROUP_TARGET);
        J.item_begin = items;
        items += (J.tiles + J.tpw - 1) / J.tpw;
        if (a.k > kmax) kmax = a.k;
    }
    hipLaunchKernelGGL(gemv_group_kernel, dim3(items), dim3(64 * GEMV_WAVES),
                       gemv_lds_bytes(kmax, GEMV_WAVES), stream, grp);
    return hipGetLastError();
}

}  // namespace nbw
