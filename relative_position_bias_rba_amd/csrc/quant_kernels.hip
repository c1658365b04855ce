// MXFP8 encoding for the KV cache: OCP Microscaling (MX) v1.0 with FP8 E4M3
// elements.  Blocks of 32 consecutive entries share an E8M0 scale 2^e with
// e = floor(log2(max |x|)) - 8 (8 = the exponent of E4M3's largest normal,
// 448), clamped to [-127, 127] and -127 for an all-zero block; each entry is
// x / 2^e rounded to the nearest E4M3 value (ties to even) and saturated to
// +-448.  The attention pages run their kernel in an MXFP8 configuration
// ("SGLang と Miles が Inkling を初日からサポート", section "Relative
// Attention と FA4 経路") and name FP8 as the way to relieve the KV cache
// ("vLLM TML Inkling サポート").
//
// Four lanes encode one block (8 entries each, one 16-byte load of bf16):
// the block maximum is exchanged among them, each lane scales its entries
// exactly (ldexp), clamps them to +-448 and converts them with the
// hardware's round-to-nearest-even E4M3 conversion, then writes two dwords
// of codes; the block's first lane writes the scale byte.  Bound by HBM (2 or 4 bytes read, 1.03 written per
// entry).
#include "rba_internal.h"

#include <math.h>

namespace rba {
namespace {

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename TI>
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const TI *__restrict__ x, int64_t rows, int nblk,
                                                            int64_t xs, uint8_t *__restrict__ q, int64_t qs,
                                                            uint8_t *__restrict__ sc, int64_t ss) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = g >> 2;            // the 4 lanes of a block are adjacent and share validity
    const int sub = (int)(g & 3);
    const int64_t row = blk / nblk;
    if (row >= rows) return;
    const int bi = (int)(blk - row * nblk);
    const int e0 = 32 * bi + 8 * sub;
    float v[8];
    if constexpr (sizeof(TI) == 2) {
        const u32x4 w = *(const u32x4 *)(x + row * xs + e0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
            v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
        }
    } else {
        const f32x4 w0 = *(const f32x4 *)(x + row * xs + e0), w1 = *(const f32x4 *)(x + row * xs + e0 + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = w0[i];
            v[4 + i] = w1[i];
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    // floor(log2 amax) = frexp exponent - 1 (exact, subnormals included)
    int e = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 1 - 8 : -127;
    e = min(max(e, -127), 127);
    float s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = fminf(fmaxf(ldexpf(v[i], -e), -448.f), 448.f);
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(s[0], s[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(s[2], s[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(s[4], s[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(s[6], s[7], w1, true);
    unsigned *dst = (unsigned *)(q + row * qs + e0);
    dst[0] = (unsigned)w0;
    dst[1] = (unsigned)w1;
    if (sub == 0) sc[row * ss + bi] = (uint8_t)(e + 127);
}

}  // namespace

hipError_t launch_mxfp8_quantize(bool in_bf16, int64_t rows, int n, const void *x, int64_t x_stride, void *codes,
                                 int64_t codes_stride, void *scales, int64_t scales_stride, hipStream_t stream) {
    const int nblk = n / 32;
    const int64_t lanes = rows * nblk * 4;
    const int64_t grid = (lanes + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (in_bf16)
        hipLaunchKernelGGL(mxfp8_quantize_kernel<__bf16>, dim3((unsigned)grid), dim3(256), 0, stream,
                           (const __bf16 *)x, rows, nblk, x_stride, (uint8_t *)codes, codes_stride,
                           (uint8_t *)scales, scales_stride);
    else
        hipLaunchKernelGGL(mxfp8_quantize_kernel<float>, dim3((unsigned)grid), dim3(256), 0, stream,
                           (const float *)x, rows, nblk, x_stride, (uint8_t *)codes, codes_stride,
                           (uint8_t *)scales, scales_stride);
    return hipGetLastError();
}

}  // namespace rba
