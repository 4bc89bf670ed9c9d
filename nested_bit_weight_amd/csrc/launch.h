// launch.h -- internal launchers shared by the C ABI (abi.cpp) and the kernel
// translation units.  Callers have validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nbw {

// Geometry shared by the qgemm launchers.
struct QgemmArgs {
    const uint16_t *x;       // bf16 [batch][ldx]
    int64_t batch;
    const uint8_t *planes;   // plane 0 of the child
    int64_t plane_bytes;
    const uint16_t *scales;  // bf16 [n][k/128]
    int n, k;
    float *y;                // fp32 [batch][ldy] (or bf16 when ybf16)
    int64_t ldx = 0, ldy = 0;          // row strides in elements (set by the caller: >= k, >= n)
    int ybf16 = 0;                     // store Y as bf16 (round to nearest even)
    const uint16_t *zeros = nullptr;   // asymmetric: bf16 [n][k/128] zero points, else null
    void *ws = nullptr;                // caller's workspace for split-k (zeroed before first use), or null
    int64_t ws_bytes = 0;
};

// Y element store shared by the kernels: fp32, or bf16 rounded to nearest even.
__device__ __forceinline__ void store_y(float *y, int ybf16, int64_t idx, float v) {
    if (ybf16) {
        uint32_t u = __float_as_uint(v);
        u += 0x7FFFu + ((u >> 16) & 1u);
        reinterpret_cast<uint16_t *>(y)[idx] = (uint16_t)(u >> 16);
    } else {
        y[idx] = v;
    }
}

// Widths and weights of the code-choice objective (at most 8 widths).
struct ChooseSpec {
    int widths[8];
    double lambdas[8];
    int nw;
};

hipError_t launch_pack(const uint8_t *codes, int n, int k, uint8_t *planes, int64_t plane_bytes,
                       hipStream_t stream);
hipError_t launch_choose(const float *w, int64_t n, int k, const uint16_t *scales,
                         const ChooseSpec &spec, uint8_t *codes, hipStream_t stream);
hipError_t launch_unpack(int r, const uint8_t *planes, int64_t plane_bytes, int n, int k,
                         uint8_t *codes, hipStream_t stream);
hipError_t launch_gemv(int r, const QgemmArgs &a, int cu_count, hipStream_t stream);
hipError_t launch_smallb(int r, const QgemmArgs &a, int cu_count, hipStream_t stream);
// Batch rows the small-batch kernel covers per pass over the planes (16 or 32).
int smallb_pass_rows(int r, int n, int cu_count);
hipError_t launch_gemm(int r, const QgemmArgs &a, int cu_count, hipStream_t stream);
// The large-batch kernel of symmetric children (gemm_wide.hip) and its split-k
// workspace bytes (0: the launch does not split).
hipError_t launch_gemm_wide(int r, const QgemmArgs &a, int cu_count, hipStream_t stream);
int64_t gemm_wide_workspace_bytes(const QgemmArgs &a, int cu_count);
void gemm_wide_name(int r, const QgemmArgs &a, char *out, size_t len);
// Workspace bytes the large-batch GEMM uses to split k deterministically (0:
// the launch does not split).
int64_t gemm_workspace_bytes(const QgemmArgs &a, int cu_count);

// Plain streaming read of [src, src + bytes) (bytes a multiple of 16), one
// XOR word per wave into sink (stream_sink_words() words).
int stream_sink_words();
hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream);
int mfma_rate_threads(int cu_count);
hipError_t launch_mfma_rate(const void *ops, int iters, float *sink, int cu_count, hipStream_t stream);

// Grouped batch-1 launch: several products (each with its own r) as one
// dispatch.  Eligible problems: batch 1, shapes the streaming kernel takes.
int gemv_group_capacity();
int gemv_max_batch();  // batch rows one streaming launch takes
bool gemv_group_eligible(const QgemmArgs &a);
hipError_t launch_gemv_group(const QgemmArgs *probs, const int *rs, int count, int cu_count,
                             hipStream_t stream);

// Grouped small-batch launch: several batch-2..16 products (each with its own
// r) as one dispatch, bit-identical to their single launches.
int smallb_group_capacity();
bool smallb_group_eligible(const QgemmArgs &a);
hipError_t launch_smallb_group(const QgemmArgs *probs, const int *rs, int count, int cu_count,
                               hipStream_t stream);

// Name of the kernel template instance the launcher above would use (as
// rocprofv3 prints it, without the parameter list).
void gemv_name(int r, const QgemmArgs &a, int cu_count, char *out, size_t len);
void smallb_name(int r, const QgemmArgs &a, int cu_count, char *out, size_t len);
void gemm_name(int r, const QgemmArgs &a, int cu_count, char *out, size_t len);

}  // namespace nbw
