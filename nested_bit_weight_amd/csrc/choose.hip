// choose.hip -- data-free choice of sliceable parent codes, gfx950.
//
// For each fp32 weight w with group scale s, pick the parent code c in 0..255
// minimising the weighted squared error of the children it serves (MatGPTQ:
// Accurate and Efficient Post-Training Matryoshka Quantization, abstract: one
// parent, several precisions by slicing the most significant bits; MatGPTQ:
// Efficient and Accurate Inference over Nested Quantized Models, captions of
// Tables 6 and 7: per-precision weights lambda_r):
//     loss(c) = sum_t lambda_t * (w - s * 2^(8-r_t) * ((c >> (8-r_t)) + 1/2 - 2^(r_t-1)))^2,
// the first code with the smallest loss winning.  The kernel tries every code
// (256 per weight, one weight per thread) in IEEE double, one rounded
// operation at a time and in a fixed order (difference, square, weight, then
// the widths left to right), so the chosen code is the same as that of any
// other evaluation that follows the same steps; fp64 has the headroom for the
// differences and squares to be exact or nearly so.
#include <cstdio>

#include "launch.h"

namespace nbw {

__global__ __launch_bounds__(256) void choose_kernel(const float *__restrict__ w, int64_t count,
                                                     int k, const uint16_t *__restrict__ scales,
                                                     ChooseSpec spec, uint8_t *__restrict__ codes) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= count) return;
    const int64_t i = e / k, j = e % k;
    const int G = k >> 7;
    const double wv = (double)w[e];
    const double s = (double)__uint_as_float((uint32_t)scales[i * G + (j >> 7)] << 16);
    // per-width constants: 2^(8-r) and 2^(r-1) (unrolled over the at most 8
    // widths, so the arrays stay in registers)
    double up[8], half_range[8];
    int shift[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int r = t < spec.nw ? spec.widths[t] : 8;
        shift[t] = 8 - r;
        up[t] = (double)(1 << shift[t]);
        half_range[t] = (double)(1 << (r - 1));
    }
    int best = 0;
    double best_loss = 0.0;
    for (int c = 0; c < 256; ++c) {
        double loss = 0.0;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t < spec.nw) {
                const double q = (double)(c >> shift[t]);
                // s * 2^(8-r) * (q + 1/2 - 2^(r-1)): every step exact
                const double d =
                    __dmul_rn(__dmul_rn(s, up[t]), __dsub_rn(__dadd_rn(q, 0.5), half_range[t]));
                const double err = __dsub_rn(wv, d);
                const double e2 = __dmul_rn(err, err);
                const double term = __dmul_rn(spec.lambdas[t], e2);
                loss = __dadd_rn(loss, term);
            }
        }
        if (c == 0 || loss < best_loss) {
            best = c;
            best_loss = loss;
        }
    }
    codes[e] = (uint8_t)best;
}

hipError_t launch_choose(const float *w, int64_t n, int k, const uint16_t *scales,
                         const ChooseSpec &spec, uint8_t *codes, hipStream_t stream) {
    const int64_t count = n * (int64_t)k;
    const int64_t blocks = (count + 255) / 256;
    hipLaunchKernelGGL(choose_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, count, k, scales,
                       spec, codes);
    return hipGetLastError();
}

}  // namespace nbw
