// launch.h -- internal launchers shared by the C ABI (abi.cpp) and the kernel
// translation units.  Callers have validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nbw {

// Geometry shared by the qgemm launchers.
struct QgemmArgs {
    const uint16_t *x;       // bf16 [batch][k]
    int64_t batch;
    const uint8_t *planes;   // plane 0 of the child
    int64_t plane_bytes;
    const uint16_t *scales;  // bf16 [n][k/128]
    int n, k;
    float *y;                // fp32 [batch][n]
};

hipError_t launch_pack(const uint8_t *codes, int n, int k, uint8_t *planes, int64_t plane_bytes,
                       hipStream_t stream);
hipError_t launch_unpack(int r, const uint8_t *planes, int64_t plane_bytes, int n, int k,
                         uint8_t *codes, hipStream_t stream);
hipError_t launch_gemv(int r, const QgemmArgs &a, int cu_count, hipStream_t stream);
hipError_t launch_smallb(int r, const QgemmArgs &a, int cu_count, hipStream_t stream);
hipError_t launch_gemm(int r, const QgemmArgs &a, int cu_count, hipStream_t stream);

// Grouped batch-1 launch: several products (each with its own r) as one
// dispatch.  Eligible problems: batch 1, shapes the streaming kernel takes.
int gemv_group_capacity();
bool gemv_group_eligible(const QgemmArgs &a);
hipError_t launch_gemv_group(const QgemmArgs *probs, const int *rs, int count, int cu_count,
                             hipStream_t stream);

// Name of the kernel template instance the launcher above would use (as
// rocprofv3 prints it, without the parameter list).
void gemv_name(int r, const QgemmArgs &a, int cu_count, char *out, size_t len);
void smallb_name(int r, const QgemmArgs &a, int cu_count, char *out, size_t len);
void gemm_name(int r, const QgemmArgs &a, int cu_count, char *out, size_t len);

}  // namespace nbw
