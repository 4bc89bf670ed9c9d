// stream.hip -- a plain streaming read, gfx950: the bandwidth reference for
// the batch-1 products.
//
// A batch-1 product reads each plane byte once (MatGPTQ: Efficient and
// Accurate Inference over Nested Quantized Models, Table 1: an r-bit child
// loads r/8 bytes per weight), so the fastest it can finish is the time one
// launch takes to read the same bytes and do nothing else.  This kernel is
// that launch: 16-byte non-temporal loads over the range, an XOR per wave so
// the loads cannot be dropped, one word per wave written out.  Launch shape:
// NBW_STREAM_BLOCKS workgroups of 4 waves (the fastest shape measured for
// 8..176 MB; many waves keep enough bytes in flight from the first cycle).
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

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t waves = (int64_t)STREAM_BLOCKS * STREAM_WAVES;
    const int64_t per_wave = (n16 + waves * 64 - 1) / (waves * 64);
    hipLaunchKernelGGL(stream_read_kernel, dim3(STREAM_BLOCKS), dim3(64 * STREAM_WAVES), 0, stream,
                       (const u32x4_s *)src, n16, per_wave, sink);
    return hipGetLastError();
}

}  // namespace nbw
