// Two measurement aids: the streaming-read bandwidth and the bf16 MFMA rate
// that this device attains, so that the attention kernels' rates can be read
// against what the chip delivers as well as against its published peaks.
#include "rba_internal.h"

namespace rba {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Each workgroup reads 1024 consecutive 16-byte chunks per step (four loads
// per thread, 4 KiB apart) and strides over the buffer; n is a multiple of
// 1024, so every chunk is read exactly once.  The result is stored only when
// it equals a sentinel, which keeps the loads without writing anything.
__global__ __launch_bounds__(256) void calib_read_kernel(const u32x4 *__restrict__ a, int64_t n,
                                                         unsigned *__restrict__ sink) {
    u32x4 acc = {};
    const int64_t stride = (int64_t)gridDim.x * 1024;
    for (int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x; i < n; i += stride) {
        const u32x4 x0 = a[i], x1 = a[i + 256], x2 = a[i + 512], x3 = a[i + 768];
        acc ^= x0 ^ x1 ^ x2 ^ x3;
    }
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) sink[0] = 1u;
}

// Back-to-back v_mfma_f32_32x32x16_bf16 on four independent accumulators per
// wave; operands come from the lane id and a run-time seed.
__global__ __launch_bounds__(256) void calib_mfma_kernel(int iters, float seed, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * (float)(lane + i));
        b[i] = (__bf16)(seed * (float)(lane - i));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    if (s == 1234.5f) sink[0] = s;
}

}  // namespace

hipError_t launch_calib_read(const void *buf, int64_t bytes, void *sink, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL(calib_read_kernel, dim3(blocks), dim3(256), 0, stream, (const u32x4 *)buf, bytes / 16,
                       (unsigned *)sink);
    return hipGetLastError();
}

hipError_t launch_calib_mfma(int iters, int blocks, void *sink, hipStream_t stream) {
    hipLaunchKernelGGL(calib_mfma_kernel, dim3(blocks), dim3(256), 0, stream, iters, 0.001f, (float *)sink);
    return hipGetLastError();
}

}  // namespace rba
