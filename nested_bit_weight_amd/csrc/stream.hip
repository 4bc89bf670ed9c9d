// stream.hip -- the two reference launches of the measurements, gfx950.
//
// A plain streaming read: a batch-1 product reads each plane byte once
// (MatGPTQ: Efficient and Accurate Inference over Nested Quantized Models,
// Table 1: an r-bit child loads r/8 bytes per weight), so the fastest it can
// finish is the time one launch takes to read the same bytes and do nothing
// else.  This kernel is that launch: 16-byte non-temporal loads over the
// range, an XOR per wave so the loads cannot be dropped, one word per wave
// written out.  Launch shape: NBW_STREAM_BLOCKS workgroups of 4 waves (the
// fastest shape measured for 8..176 MB; many waves keep enough bytes in
// flight from the first cycle).
//
// A matrix-unit rate loop: the large-batch products are bound by
// v_mfma_f32_32x32x16_bf16 (the same paper, Abstract: kernels that serve
// batch sizes beyond one), and this kernel issues nothing else -- four
// independent accumulator chains per wave, two waves per SIMD on every
// compute unit, the operands cycling through 8 A and 8 B fragments held in
// registers, so the data the unit multiplies changes from one instruction to
// the next as it does in the products.  Its rate is the ceiling those
// products are measured against on the same chip and data; with random
// operands the chip runs this load at a lower clock than with constant ones.
#include "launch.h"

namespace nbw {

typedef uint32_t u32x4_s __attribute__((ext_vector_type(4)));

constexpr int STREAM_BLOCKS = 2048;
constexpr int STREAM_WAVES = 4;

__global__ __launch_bounds__(64 * STREAM_WAVES) void stream_read_kernel(const u32x4_s *__restrict__ p,
                                                                       int64_t n16, int64_t per_wave,
                                                                       uint32_t *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * STREAM_WAVES + (threadIdx.x >> 6);
    const int64_t base = wave * per_wave * 64;
    u32x4_s acc = {0u, 0u, 0u, 0u};
#pragma unroll 8
    for (int64_t i = 0; i < per_wave; ++i) {
        const int64_t idx = base + i * 64 + lane;
        if (idx < n16) acc ^= __builtin_nontemporal_load(p + idx);
    }
    uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    // XOR over the wave (butterfly), one word per wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) r ^= __shfl_xor(r, d);
    if (lane == 0) sink[wave] = r;
}

int stream_sink_words() { return STREAM_BLOCKS * STREAM_WAVES; }

typedef float f32x16_s __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_s __attribute__((ext_vector_type(8)));

constexpr int MFMA_RATE_WAVES = 8;  // two per SIMD

// ops: 16 fragments of 64 lanes x 16 bytes (fragment f of lane l at index
// f * 64 + l): f < 8 the A operands, f >= 8 the B operands.  Each round is 64
// MFMAs; MFMA s of a round takes A fragment s % 8, B fragment (s / 8) % 8 and
// accumulator s % 4.  sink[thread] = the sum of the thread's accumulators.
__global__ __launch_bounds__(64 * MFMA_RATE_WAVES) void mfma_rate_kernel(const u32x4_s *__restrict__ ops,
                                                                        int iters, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    u32x4_s a[8], b[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
        a[f] = ops[f * 64 + lane];
        b[f] = ops[(8 + f) * 64 + lane];
    }
    f32x16_s acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 64; ++s)
            acc[s & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_s, a[s & 7]),
                                                                 __builtin_bit_cast(bf16x8_s, b[(s >> 3) & 7]),
                                                                 acc[s & 3], 0, 0, 0);
    }
    float t = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) t += acc[c][v];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = t;
}

int mfma_rate_threads(int cu_count) { return cu_count * 64 * MFMA_RATE_WAVES; }

hipError_t launch_mfma_rate(const void *ops, int iters, float *sink, int cu_count, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(cu_count), dim3(64 * MFMA_RATE_WAVES), 0, stream,
                       (const u32x4_s *)ops, iters, sink);
    return hipGetLastError();
}


hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t waves = (int64_t)STREAM_BLOCKS * STREAM_WAVES;
    const int64_t per_wave = (n16 + waves * 64 - 1) / (waves * 64);
    hipLaunchKernelGGL(stream_read_kernel, dim3(STREAM_BLOCKS), dim3(64 * STREAM_WAVES), 0, stream,
                       (const u32x4_s *)src, n16, per_wave, sink);
    return hipGetLastError();
}

}  // namespace nbw
