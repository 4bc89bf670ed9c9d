// pack.hip -- bit-plane packer and the unpack test hook (gfx950).
//
// Packing turns one 8-bit parent code per weight into eight MSB-first
// bit-planes, so that the r-bit child is the first r planes and reads exactly
// r bits (MatGPTQ: Efficient and Accurate Inference over Nested Quantized
// Models, Abstract; Table 1, "Exact r-bit loading").  Bit order inside a plane
// is the library layout (see nbw.h).
//
// pack_kernel: one workgroup per (16-row tile, run of up to 16 groups).
//   Phase 1 streams the codes of the region into LDS with coalesced 128-bit
//   loads (each row segment is contiguous in the codes).  Phase 2 gives each
//   thread one (row, group) chunk: it reads its 128 codes from LDS, runs the
//   bit-transpose network of decode.h backwards (every merge is its own
//   inverse) and writes eight 16-byte plane chunks; consecutive threads write
//   consecutive chunks, so the plane stores are coalesced too.
//   HBM traffic: 1 byte read + 1 byte written per weight.
#include "decode.h"
#include "launch.h"

namespace nbw {

constexpr int PACK_GROUPS = 16;                   // groups per workgroup region
constexpr int PACK_ROW_BYTES = PACK_GROUPS * 128; // LDS row pitch
// 16-byte chunk c of region row i sits at chunk c ^ pack_swz(i) of the row.
// The LDS serves a 16-byte-per-lane access half a wave at a time over 128
// four-byte banks (32 chunks); lanes of a half-wave that hit one bank at
// different addresses conflict.  Phase 1 writes 32 consecutive chunks of one
// row per half-wave: any XOR below 32 keeps them on 32 distinct banks.  Phase
// 2 has the 16 rows of two neighbouring groups in a half-wave, reading chunks
// 8 gl + e: the two groups differ in bit 3 of the chunk index, so the
// swizzles of the 16 rows must differ in bits 0..2 and 4 and leave bit 3
// clear -- (i & 7) | (i & 8) << 1 -- and all 32 reads land on distinct banks.
__device__ __forceinline__ int pack_swz(int i) { return (i & 7) | ((i & 8) << 1); }

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t *__restrict__ codes, int n, int k,
                                                   uint8_t *__restrict__ planes,
                                                   int64_t plane_bytes) {
    __shared__ __align__(16) uint8_t lds[16 * PACK_ROW_BYTES];
    const int G = k / 128;
    const int tile = blockIdx.x;
    const int g0 = blockIdx.y * PACK_GROUPS;
    const int gcount = min(PACK_GROUPS, G - g0);
    const int tid = threadIdx.x;

    // Phase 1: 16 rows x (gcount*128) bytes into LDS, 16 bytes per load.  A
    // full region is 8 loads per thread, all issued before the first LDS
    // write (a load-wait-write loop would pay the memory latency 8 times).
    const int vec_per_row = gcount * 8;
    auto load16 = [&](int u) {
        const int i = u / vec_per_row, v = u % vec_per_row;
        const int row = tile * 16 + i;
        u32x4_t val = {0u, 0u, 0u, 0u};
        if (row < n)
            val = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(
                codes + (int64_t)row * k + (int64_t)g0 * 128 + 16 * v));
        return val;
    };
    auto put16 = [&](int u, const u32x4_t &val) {
        const int i = u / vec_per_row, v = u % vec_per_row;
        *reinterpret_cast<u32x4_t *>(lds + i * PACK_ROW_BYTES + 16 * (v ^ pack_swz(i))) = val;
    };
    if (gcount == PACK_GROUPS) {
        constexpr int PER = 16 * PACK_GROUPS * 8 / 256;
        u32x4_t val[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) val[q] = load16(tid + 256 * q);
#pragma unroll
        for (int q = 0; q < PER; ++q) put16(tid + 256 * q, val[q]);
    } else {
        for (int u = tid; u < 16 * vec_per_row; u += 256) put16(u, load16(u));
    }
    __syncthreads();

    // Phase 2: thread -> (row i, group gl) chunk.
    const int i = tid & 15, gl = tid >> 4;
    if (gl >= gcount) return;
    const uint8_t *src = lds + i * PACK_ROW_BYTES;
    const int swz = pack_swz(i);
    uint32_t out[8][4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t W[8];
        const uint4 a = *reinterpret_cast<const uint4 *>(src + 16 * ((8 * gl + 2 * d) ^ swz));
        const uint4 b = *reinterpret_cast<const uint4 *>(src + 16 * ((8 * gl + 2 * d + 1) ^ swz));
        W[0] = a.x; W[1] = a.y; W[2] = a.z; W[3] = a.w;
        W[4] = b.x; W[5] = b.y; W[6] = b.z; W[7] = b.w;
        uint32_t P[8];
        pack_word32(W, P);
#pragma unroll
        for (int p = 0; p < 8; ++p) out[p][d] = P[p];
    }
    const int64_t chunk = ((int64_t)tile * G + g0 + gl) * 16 + i;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const u32x4_t v = {out[p][0], out[p][1], out[p][2], out[p][3]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(planes + p * plane_bytes + chunk * 16));
    }
}

// Unpack test hook: thread per (row, group) chunk; reads planes 0..R-1 only,
// decodes them with the same network and extraction plan as the qgemm
// kernels, and writes the 128 child codes of its chunk (row-major codes).
template <int R>
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t *__restrict__ planes,
                                                     int64_t plane_bytes, int n, int k,
                                                     uint8_t *__restrict__ codes) {
    const int G = k / 128;
    const int64_t ci = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t tiles = (n + 15) / 16;
    if (ci >= tiles * G * 16) return;
    const int i = (int)(ci % 16);
    const int g = (int)((ci / 16) % G);
    const int64_t tile = ci / (16 * G);
    const int64_t row = tile * 16 + i;
    if (row >= n) return;
    uint32_t pw[R][4];
#pragma unroll
    for (int p = 0; p < R; ++p) {
        const uint4 v = *reinterpret_cast<const uint4 *>(planes + p * plane_bytes + ci * 16);
        pw[p][0] = v.x; pw[p][1] = v.y; pw[p][2] = v.z; pw[p][3] = v.w;
    }
    uint32_t outw[32];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t P[R];
#pragma unroll
        for (int p = 0; p < R; ++p) P[p] = pw[p][d];
        constexpr int rp0 = Phases<R>::rp0, rp1 = Phases<R>::rp1;
        uint32_t Z0[NetWords<rp0>::value];
        network<rp0>(P, Z0);
        uint32_t Z1[NetWords<(rp1 > 0 ? rp1 : 1)>::value];
        if constexpr (rp1 > 0) network<rp1>(P + 4, Z1);
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            uint32_t v = extract_codes<rp0>(Z0, m);
            if constexpr (rp1 > 0) v = (v << rp1) | extract_codes<rp1>(Z1, m);
            // pair m = columns 32d+2m (low half) and 32d+2m+1 (high half)
            const uint32_t two = (v & 0xFFu) | ((v >> 8) & 0xFF00u);
            const int w = 8 * d + (m >> 1);
            if (m & 1)
                outw[w] |= two << 16;
            else
                outw[w] = two;
        }
    }
    uint8_t *dst = codes + row * k + (int64_t)g * 128;
#pragma unroll
    for (int q = 0; q < 8; ++q)
        *reinterpret_cast<uint4 *>(dst + 16 * q) =
            make_uint4(outw[4 * q], outw[4 * q + 1], outw[4 * q + 2], outw[4 * q + 3]);
}

hipError_t launch_pack(const uint8_t *codes, int n, int k, uint8_t *planes, int64_t plane_bytes,
                       hipStream_t stream) {
    const int G = k / 128;
    dim3 grid((unsigned)((n + 15) / 16), (unsigned)((G + PACK_GROUPS - 1) / PACK_GROUPS));
    hipLaunchKernelGGL(pack_kernel, grid, dim3(256), 0, stream, codes, n, k, planes, plane_bytes);
    return hipGetLastError();
}

template <int R>
static void launch_unpack_r(const uint8_t *planes, int64_t plane_bytes, int n, int k,
                            uint8_t *codes, hipStream_t stream) {
    const int64_t chunks = (int64_t)((n + 15) / 16) * (k / 128) * 16;
    dim3 grid((unsigned)((chunks + 255) / 256));
    hipLaunchKernelGGL(unpack_kernel<R>, grid, dim3(256), 0, stream, planes, plane_bytes, n, k,
                       codes);
}

hipError_t launch_unpack(int r, const uint8_t *planes, int64_t plane_bytes, int n, int k,
                         uint8_t *codes, hipStream_t stream) {
    switch (r) {
    case 1: launch_unpack_r<1>(planes, plane_bytes, n, k, codes, stream); break;
    case 2: launch_unpack_r<2>(planes, plane_bytes, n, k, codes, stream); break;
    case 3: launch_unpack_r<3>(planes, plane_bytes, n, k, codes, stream); break;
    case 4: launch_unpack_r<4>(planes, plane_bytes, n, k, codes, stream); break;
    case 5: launch_unpack_r<5>(planes, plane_bytes, n, k, codes, stream); break;
    case 6: launch_unpack_r<6>(planes, plane_bytes, n, k, codes, stream); break;
    case 7: launch_unpack_r<7>(planes, plane_bytes, n, k, codes, stream); break;
    case 8: launch_unpack_r<8>(planes, plane_bytes, n, k, codes, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace nbw
