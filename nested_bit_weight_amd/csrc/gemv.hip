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

constexpr int GEMV_MAX_WAVES = 8;   // waves per workgroup (the launch picks 4 or 8)
constexpr int GEMV_ODD_WAVES = 4;   // waves per workgroup of the odd-group-count kernel
constexpr int GEMV_MAX_TILES = 16;  // tiles per workgroup
constexpr int GEMV_MAX_GROUP = 32;  // products per grouped launch

// Steps a wave keeps in flight (prefetch depth).  Every wave of the grid
// prefetches this many steps at once, so the total in flight must stay near
// what HBM delivers in one memory latency, not a large share of the matrix:
// a deeper queue only delays each wave's first step.  Waves with only a few
// steps take depth 1 (a second buffer would hold repeats of the last step).
// (Measured on 70B- and Qwen3-8B-sized linears: depth 3 or 4 at r = 2, 3 is
// slower than 2; at r = 6 depth 2 beats 1 by 7%.)
constexpr int GEMV_DEPTH_SHORT = 1;
__host__ __device__ constexpr int gemv_depth(int r) { return r <= 6 ? 2 : 1; }

// Dynamic LDS: per wave, one set of X (4 groups x 128 bf16 = 1 KB), then the
// per-lane partial sums fp32 [W][slots][64], one slot per tile.
__host__ __device__ constexpr size_t gemv_lds_bytes(int waves, int slots) {
    return (size_t)waves * 1024 + (size_t)waves * slots * 64 * 4;
}

// Sum over each 16-lane row of the wave, in every lane of the row: DPP quad
// permutes [1,0,3,2] and [2,3,0,1], then row_half_mirror (lane i of each
// half-row reads lane 7-i: the other quad) and row_mirror (lane i reads
// lane 15-i: the other half).  VALU only, no LDS round trip.
__device__ __forceinline__ float row16_sum(float v) {
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

// One workgroup: tiles [t_begin, t_begin + T) of one product, all of k;
// `slots` partial-sum slots per wave in LDS (T <= slots).
//
// Waves are independent until the final reduction: a wave loads the X of its
// current set itself (one 16-byte load per lane, part of the step's load
// stream), stages it in its own 1 KB of LDS and reads back its lanes'
// groups, so no barrier -- and no wait for every load in flight -- stands
// between a wave's first loads and its first step.
template <int R, int PD, bool ASYM>
__device__ __forceinline__ void gemv_tiles(const uint16_t *__restrict__ x,
                                           const uint8_t *__restrict__ planes,
                                           int64_t plane_bytes,
                                           const uint16_t *__restrict__ scales,
                                           const uint16_t *__restrict__ zeros, int n, int k,
                                           int t_begin, int T, int slots, float *__restrict__ y,
                                           int ybf16, unsigned char *lds) {
    const int G = k >> 7;
    const int nsets = (G + 3) >> 2;
    const int W = blockDim.x >> 6;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int i = lane & 15, gg = lane >> 4;
    uint32_t *xw = reinterpret_cast<uint32_t *>(lds) + w * 256;          // this wave's set of X
    float *red = reinterpret_cast<float *>(lds + (size_t)W * 1024);      // [W][slots][64]

    // This wave's (set, tile) steps: set ordinal s = 0 .. my_sets-1 is set
    // w + s*W, tile t = 0 .. T-1; step u = s*T + t.
    const int my_sets = nsets > w ? (nsets - w + W - 1) / W : 0;
    const int U = my_sets * T;

    // Zero this wave's partial sums (only this wave writes them until the
    // final barrier).
    for (int t = 0; t < T; ++t) red[(w * slots + t) * 64 + lane] = 0.f;

    // Coefficient of this lane's pair sums in the group correction
    // sum_k x_k * (1/2 - 2^(R-1) - offset_k): lane (i, gg) takes the pairs
    // i, i+16, i+32, i+48 of its group, which share one offset.
    float my_coef = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m)
        if (i == m) my_coef = pair_coef<R>(m);

    // Step loads: R plane chunks, the aligned 32-bit scale word, and the
    // lane's 16 bytes of the set's X (the same chunk for every tile of a set;
    // reloading it keeps the number of loads per step fixed).  All loads are
    // unconditional (clamped at the end), so the loads-in-flight count between
    // a load and its use is static.
    u32x4_t buf[PD][R];
    u32x4_t xbuf[PD];
    uint32_t sbuf[PD];
    uint32_t zbuf[ASYM ? PD : 1];
    int ps = 0, pt = 0;  // next step to prefetch
    const int xchunks = k >> 3;
    auto load_step = [&](int j) {
        int s = ps, t = pt;
        if (s >= my_sets) {
            s = my_sets - 1;
            t = T - 1;
        }
        const int set = w + s * W;
        xbuf[j] = reinterpret_cast<const u32x4_t *>(x)[min(set * 64 + lane, xchunks - 1)];
        const int g = min(4 * set + gg, G - 1);
        const uint8_t *c = planes + (((int64_t)(t_begin + t) * G + g) * 16 + i) * 16;
#pragma unroll
        for (int p = 0; p < R; ++p)
            buf[j][p] =
                __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(c + p * plane_bytes));
        // (in bounds: the host sends only even group counts here; a 16-bit
        // load would need a zero-extension that the compiler may place where
        // it waits for every load in flight)
        const int row = min(16 * (t_begin + t) + i, n - 1);
        const int64_t idx = (int64_t)row * G + g;
        sbuf[j] = *reinterpret_cast<const uint32_t *>(scales + (idx & ~(int64_t)1));
        if constexpr (ASYM) zbuf[j] = *reinterpret_cast<const uint32_t *>(zeros + (idx & ~(int64_t)1));
        if (++pt == T) {
            pt = 0;
            ++ps;
        }
    };
    if (U > 0) {
#pragma unroll
        for (int j = 0; j < PD; ++j) load_step(j);
    }

    uint32_t X2[64];
    float cg = 0.f, sg = 0.f;  // group correction; group sum of X (asymmetric term)
    int cs = 0, ct = 0;  // step being computed
    auto compute = [&](int j) {
        const int g = 4 * (w + cs * W) + gg;
        const bool gvalid = g < G;
        if (ct == 0) {
            // New set: stage its X (LDS operations of one wave complete in
            // order, so the previous set's reads are done), read back this
            // lane's group, and form the group's correction over the quarter.
            reinterpret_cast<u32x4_t *>(xw)[lane] = xbuf[j];
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const u32x4_t v = reinterpret_cast<const u32x4_t *>(xw + 64 * gg)[q];
                X2[4 * q] = v.x; X2[4 * q + 1] = v.y; X2[4 * q + 2] = v.z; X2[4 * q + 3] = v.w;
            }
            const uint32_t one = 0x3F803F80u;  // bf16 (1.0, 1.0)
            float sx = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) sx = dot2(one, xw[64 * gg + i + 16 * q], sx);
            cg = row16_sum(my_coef * sx);
            if constexpr (ASYM) sg = row16_sum(sx);
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
        if constexpr (ASYM) {
            // asymmetric child = symmetric child + s * (127.5 - z) per weight;
            // in the units of P (which the epilogue scales by 2^(8-R)):
            const uint32_t zbits = (g & 1) ? (zbuf[j] & 0xFFFF0000u) : (zbuf[j] << 16);
            const float zc = (127.5f - __uint_as_float(zbits)) * (1.0f / (float)(1 << (8 - R)));
            return s * fmaf(zc, sg, P + cg);
        }
        return s * (P + cg);
    };
    // Accumulate into this lane's own LDS slot for the tile.  Each slot has a
    // single writer (this lane), so no atomic is needed and the order of the
    // additions is fixed: the wave's first set stores, later sets read, add
    // and store.  (LDS float atomics serialize across the CU: one wave-wide
    // ds_add_f32 per step cost about a microsecond per launch.)
    auto commit = [&](float v) {
        float *slot = &red[(w * slots + ct) * 64 + lane];
        if (cs == 0)
            *slot = v;
        else
            *slot += v;
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

    // Rows: add the four groups of each set and the waves, in a fixed order.
    __syncthreads();
    const float post = (float)(1 << (8 - R));
    for (int e = threadIdx.x; e < T * 16; e += blockDim.x) {
        const int t = e >> 4, ii = e & 15;
        float sum = 0.f;
        for (int ww = 0; ww < W; ++ww) {
            const float *slot = red + (ww * slots + t) * 64 + ii;
            sum += (slot[0] + slot[16]) + (slot[32] + slot[48]);
        }
        const int row = 16 * t_begin + e;
        if (row < n) store_y(y, ybf16, row, sum * post);
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

template <int R, int PD, bool ASYM>
__global__ __launch_bounds__(64 * GEMV_MAX_WAVES) void gemv_kernel(const uint16_t *__restrict__ x,
                                                                  const uint8_t *__restrict__ planes,
                                                                  int64_t plane_bytes,
                                                                  const uint16_t *__restrict__ scales,
                                                                  const uint16_t *__restrict__ zeros,
                                                                  int n, int k, int tiles_total,
                                                                  int tiles_per_wg,
                                                                  float *__restrict__ y, int ybf16) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int t_begin = blockIdx.x * tiles_per_wg;
    const int T = min(tiles_per_wg, tiles_total - t_begin);
    gemv_tiles<R, PD, ASYM>(x, planes, plane_bytes, scales, zeros, n, k, t_begin, T, tiles_per_wg,
                            y, ybf16, lds);
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
    int count, slots;
};

// Workgroup b runs item b; items are numbered product by product.  Every
// item has `slots` partial-sum slots per wave (the largest tpw of the group).
__global__ __launch_bounds__(64 * GEMV_MAX_WAVES) void gemv_group_kernel(GemvGroup grp) {
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
        gemv_tiles<RR, gemv_depth(RR), false>(J.x, J.planes, J.plane_bytes, J.scales, nullptr,   \
                                              J.n, J.k, t_begin, T, grp.slots, J.y, 0, lds);  \
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

// Launch shape of the streaming kernel.  Eight waves per workgroup (two per
// SIMD: one wave alone leaves the decode's dependent-issue gaps unfilled) and
// about one workgroup per CU, each owning a run of 16-row tiles.
struct GemvPlan {
    int waves, tpw;
    bool deep;  // prefetch depth gemv_depth(r), else GEMV_DEPTH_SHORT
};

static GemvPlan gemv_plan(int n, int k, int r, int cu_count) {
    const int tiles = (n + 15) / 16;
    GemvPlan p;
    p.waves = GEMV_MAX_WAVES;
    int tpw = (tiles + cu_count / 2) / cu_count;  // about one workgroup per CU
    if (tpw > GEMV_MAX_TILES) tpw = GEMV_MAX_TILES;
    if (tpw < 1) tpw = 1;
    p.tpw = tpw;
    const int nsets = (k / 128 + 3) / 4;
    const int steps = (nsets + p.waves - 1) / p.waves * tpw;  // per wave, at most
    p.deep = gemv_depth(r) > GEMV_DEPTH_SHORT && steps >= 4;
    return p;
}

static bool gemv_streamable(int k);

template <int R, bool ASYM>
static void launch_stream(const GemvPlan &p, int tiles, const QgemmArgs &a, const uint16_t *x,
                          float *y, hipStream_t stream) {
    const dim3 grid((tiles + p.tpw - 1) / p.tpw), block(64 * p.waves);
    const size_t lds = gemv_lds_bytes(p.waves, p.tpw);
    if (p.deep)
        hipLaunchKernelGGL((gemv_kernel<R, gemv_depth(R), ASYM>), grid, block, lds, stream, x, a.planes,
                           a.plane_bytes, a.scales, a.zeros, a.n, a.k, tiles, p.tpw, y, a.ybf16);
    else
        hipLaunchKernelGGL((gemv_kernel<R, GEMV_DEPTH_SHORT, ASYM>), grid, block, lds, stream, x,
                           a.planes, a.plane_bytes, a.scales, a.zeros, a.n, a.k, tiles, p.tpw, y,
                           a.ybf16);
}

template <int R>
static void launch_r(const QgemmArgs &a, int cu_count, hipStream_t stream) {
    const int tiles = (a.n + 15) / 16;
    for (int64_t b = 0; b < a.batch; ++b) {  // one batch row per launch
        const uint16_t *x = a.x + b * a.ldx;
        // (y advances by ldy elements of the output type)
        float *y = a.ybf16 ? reinterpret_cast<float *>(reinterpret_cast<uint16_t *>(a.y) + b * a.ldy)
                           : a.y + b * a.ldy;
        if (!gemv_streamable(a.k)) {
            hipLaunchKernelGGL(gemv_odd_kernel<R>, dim3(tiles), dim3(64 * GEMV_ODD_WAVES), 0, stream,
                               x, a.planes, a.plane_bytes, a.scales, a.zeros, a.n, a.k, y, a.ybf16);
        } else {
            const GemvPlan p = gemv_plan(a.n, a.k, R, cu_count);
            if (a.zeros)
                launch_stream<R, true>(p, tiles, a, x, y, stream);
            else
                launch_stream<R, false>(p, tiles, a, x, y, stream);
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
    if (!gemv_streamable(a.k)) {
        snprintf(out, len, "nbw::gemv_odd_kernel<%d>", r);
    } else {
        const GemvPlan p = gemv_plan(a.n, a.k, r, cu_count);
        snprintf(out, len, "nbw::gemv_kernel<%d, %d, %s>", r, p.deep ? gemv_depth(r) : GEMV_DEPTH_SHORT,
                 a.zeros ? "true" : "false");
    }
}

int gemv_group_capacity() { return GEMV_MAX_GROUP; }

// The streaming kernel reads scales as aligned 32-bit words: it takes even
// group counts (every other shape goes to the plain one-tile kernel).
static bool gemv_streamable(int k) { return ((k / 128) & 1) == 0; }

bool gemv_group_eligible(const QgemmArgs &a) {
    return a.batch == 1 && gemv_streamable(a.k) && !a.zeros && !a.ybf16;
}

hipError_t launch_gemv_group(const QgemmArgs *probs, const int *rs, int count, int cu_count,
                             hipStream_t stream) {
    GemvGroup grp = {};
    grp.count = count;
    int items = 0, slots = 1;
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
        J.tpw = gemv_plan(a.n, a.k, rs[j], cu_count).tpw;
        if (J.tpw > slots) slots = J.tpw;
        J.item_begin = items;
        items += (J.tiles + J.tpw - 1) / J.tpw;
    }
    grp.slots = slots;
    hipLaunchKernelGGL(gemv_group_kernel, dim3(items), dim3(64 * GEMV_MAX_WAVES),
                       gemv_lds_bytes(GEMV_MAX_WAVES, slots), stream, grp);
    return hipGetLastError();
}

}  // namespace nbw
