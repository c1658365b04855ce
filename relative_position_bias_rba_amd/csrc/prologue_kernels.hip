// Attention prologue for gfx950: the K/V ShortConv, the Q/K RMSNorm and the
// KV-cache write of the new tokens in one pass ("SGLang と Miles が Inkling を
// 初日からサポート", sections "ShortConv：4カ所に現れる短距離因果畳み込み" and
// "ShortConv 最適化": a per-channel causal convolution over the current token
// and the W-1 before it, on the K stream before the Q/K normalisation and on
// the V stream; SGLang fuses the convolutions, the normalisation and the cache
// write into one prologue kernel).
//
// Per new token the kernel reads the q, k, v projections once and writes the
// normalised q and the cache rows once, so it is bound by HBM.  Half a wave
// (32 lanes x 4 channels) owns one 128-entry row: a q head (RMSNorm), a k head
// (convolution over the token and up to W-1 earlier rows - new rows of the
// same sequence or the conv state - then RMSNorm) or a v head (convolution).
// RMSNorm sums of squares are exchanged within the half wave.  The cache row
// goes to position seq_len - n_new + i of its sequence, dense or through the
// block table, as bf16 or as MXFP8 (the bf16 value encoded: eight lanes per
// 32-entry block share the block maximum).  A second small kernel then moves
// each sequence's last W-1 pre-convolution rows into its conv state.
#include "rba_internal.h"

#include <math.h>

namespace rba {
namespace {

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
constexpr int D = 128;

__device__ __forceinline__ void load4(const __bf16 *p, float x[4]) {
    const u32x2 w = *(const u32x2 *)p;
    x[0] = __builtin_bit_cast(float, w[0] << 16);
    x[1] = __builtin_bit_cast(float, w[0] & 0xffff0000u);
    x[2] = __builtin_bit_cast(float, w[1] << 16);
    x[3] = __builtin_bit_cast(float, w[1] & 0xffff0000u);
}

__device__ __forceinline__ u32x2 pack4(const float x[4]) {
    const unsigned a = __builtin_bit_cast(unsigned short, (__bf16)x[0]);
    const unsigned b = __builtin_bit_cast(unsigned short, (__bf16)x[1]);
    const unsigned c = __builtin_bit_cast(unsigned short, (__bf16)x[2]);
    const unsigned d = __builtin_bit_cast(unsigned short, (__bf16)x[3]);
    return u32x2{a | (b << 16), c | (d << 16)};
}

// x * g / sqrt(mean over the row's 128 entries of x^2 + eps), the row spread
// over the 32 lanes of this half wave
__device__ __forceinline__ void rms_norm4(float x[4], const float *g, int c0, float eps) {
    float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) ss += __shfl_xor(ss, m, 32);
    const float r = 1.f / sqrtf(ss * (1.f / D) + eps);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = x[e] * r * g[c0 + e];
}

template <bool F8, bool PG>
__global__ __launch_bounds__(256) void prologue_kernel(const PrologueParams p) {
    const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    const int lane = threadIdx.x & 31;
    const int HR = p.Hq + 2 * p.Hkv;
    if (row >= (int64_t)p.T * HR) return;   // the whole half wave leaves together
    const int t = (int)(row / HR);
    const int hr = (int)(row - (int64_t)t * HR);
    const int c0 = 4 * lane;

    if (hr < p.Hq) {                          // q: RMSNorm only
        float x[4];
        load4(p.q + (int64_t)t * p.qs0 + (int64_t)hr * p.qs1 + c0, x);
        rms_norm4(x, p.norm_q, c0, p.eps);
        *(u32x2 *)(p.q_out + (int64_t)t * p.qos0 + (int64_t)hr * p.qos1 + c0) = pack4(x);
        return;
    }
    const bool isk = hr < p.Hq + p.Hkv;
    const int g = hr - p.Hq - (isk ? 0 : p.Hkv);

    // the sequence owning token t: the last b with cu_new[b] <= t
    int lo = 0, hi = p.B;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.cu_new[mid] <= t) lo = mid; else hi = mid;
    }
    const int b = lo;
    // device values clamped so that every access stays in its tensor
    const int a0 = min(max(p.cu_new[b], 0), p.T);
    const int n = min(max(p.cu_new[b + 1], a0), p.T) - a0;
    const int i = t - a0;
    if (i < 0 || i >= n) return;              // token outside every sequence's range
    const int L = min(max(p.seq_lens[b], n), p.Skv);   // keys after the append
    const int pos = L - n + i;

    const __bf16 *src = isk ? p.k : p.v;
    const int64_t s0 = isk ? p.ks0 : p.vs0, s1 = isk ? p.ks1 : p.vs1;
    const __bf16 *state = isk ? p.state_k : p.state_v;
    const float *w = (isk ? p.conv_wk : p.conv_wv) + (int64_t)(g * D + c0) * p.W;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int l = 0; l < p.W; ++l) {
        if (pos - l < 0) break;               // before the sequence start: zero
        const __bf16 *rp = (i - l >= 0)
                               ? src + (int64_t)(t - l) * s0 + (int64_t)g * s1
                               : state + (((int64_t)b * (p.W - 1) + (p.W - 1 + i - l)) * p.Hkv + g) * D;
        float x[4];
        load4(rp + c0, x);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(w[e * p.W + l], x[e], acc[e]);
    }
    if (isk) rms_norm4(acc, p.norm_k, c0, p.eps);

    // destination row of the cache
    int64_t off;                              // element (= byte for MXFP8) offset of the row
    int64_t soff;                             // scale offset (MXFP8)
    const int64_t cs0 = isk ? p.cks0 : p.cvs0, cs1 = isk ? p.cks1 : p.cvs1, cs2 = isk ? p.cks2 : p.cvs2;
    const int64_t ss0 = isk ? p.sks0 : p.svs0, ss1 = isk ? p.sks1 : p.svs1, ss2 = isk ? p.sks2 : p.svs2;
    if constexpr (PG) {
        const int pg = pos / p.page_size;
        const int page = min(max(p.block_table[(int64_t)b * p.bt_stride + pg], 0), p.num_pages - 1);
        const int r = pos - pg * p.page_size;
        off = (int64_t)page * cs0 + (int64_t)r * cs1 + (int64_t)g * cs2;
        soff = (int64_t)page * ss0 + (int64_t)r * ss1 + (int64_t)g * ss2;
    } else {
        off = (int64_t)b * cs0 + (int64_t)pos * cs1 + (int64_t)g * cs2;
        soff = (int64_t)b * ss0 + (int64_t)pos * ss1 + (int64_t)g * ss2;
    }
    const u32x2 h = pack4(acc);
    if constexpr (!F8) {
        *(u32x2 *)((__bf16 *)(isk ? p.k_cache : p.v_cache) + off + c0) = h;
    } else {
        // encode the bf16 row: block = 8 lanes (32 entries)
        float x[4];
        x[0] = __builtin_bit_cast(float, h[0] << 16);
        x[1] = __builtin_bit_cast(float, h[0] & 0xffff0000u);
        x[2] = __builtin_bit_cast(float, h[1] << 16);
        x[3] = __builtin_bit_cast(float, h[1] & 0xffff0000u);
        float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        amax = fmaxf(amax, __shfl_xor(amax, 4));
        int e = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 1 - 8 : -127;
        e = min(max(e, -127), 127);
        float s[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) s[j] = fminf(fmaxf(ldexpf(x[j], -e), -448.f), 448.f);
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(s[0], s[1], 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(s[2], s[3], wd, true);
        *(unsigned *)((uint8_t *)(isk ? p.k_cache : p.v_cache) + off + c0) = (unsigned)wd;
        if ((lane & 7) == 0) ((uint8_t *)(isk ? p.k_scale : p.v_scale))[soff + (lane >> 3)] = (uint8_t)(e + 127);
    }
}

// conv state <- the pre-convolution rows of each sequence's last W-1
// positions.  One thread per (sequence, stream, kv head, 4 channels), rows in
// ascending order: row j reads old row j + n (not yet overwritten) or new row.
__global__ __launch_bounds__(256) void conv_state_kernel(const PrologueParams p) {
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)p.B * 2 * p.Hkv * (D / 4);
    if (id >= total) return;
    const int c0 = 4 * (int)(id % (D / 4));
    int64_t r = id / (D / 4);
    const int g = (int)(r % p.Hkv);
    r /= p.Hkv;
    const bool isk = (r & 1) == 0;
    const int b = (int)(r >> 1);
    const int a0 = min(max(p.cu_new[b], 0), p.T);
    const int n = min(max(p.cu_new[b + 1], a0), p.T) - a0;
    const __bf16 *src = isk ? p.k : p.v;
    const int64_t s0 = isk ? p.ks0 : p.vs0, s1 = isk ? p.ks1 : p.vs1;
    __bf16 *state = isk ? p.state_k : p.state_v;
    for (int j = 0; j < p.W - 1; ++j) {
        const int k = n + j;                  // index in [old state rows, new rows]
        u32x2 val;
        if (k < p.W - 1)
            val = *(const u32x2 *)(state + (((int64_t)b * (p.W - 1) + k) * p.Hkv + g) * D + c0);
        else
            val = *(const u32x2 *)(src + (int64_t)(a0 + k - (p.W - 1)) * s0 + (int64_t)g * s1 + c0);
        *(u32x2 *)(state + (((int64_t)b * (p.W - 1) + j) * p.Hkv + g) * D + c0) = val;
    }
}

}  // namespace

hipError_t launch_prologue(const PrologueParams &p, hipStream_t stream) {
    const int64_t rows = (int64_t)p.T * (p.Hq + 2 * p.Hkv);
    if (rows > 0) {
        const int64_t grid = (rows + 7) / 8;
        if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
        const bool f8 = p.k_scale != nullptr, pg = p.block_table != nullptr;
        if (f8 && pg)
            hipLaunchKernelGGL((prologue_kernel<true, true>), dim3((unsigned)grid), dim3(256), 0, stream, p);
        else if (f8)
            hipLaunchKernelGGL((prologue_kernel<true, false>), dim3((unsigned)grid), dim3(256), 0, stream, p);
        else if (pg)
            hipLaunchKernelGGL((prologue_kernel<false, true>), dim3((unsigned)grid), dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((prologue_kernel<false, false>), dim3((unsigned)grid), dim3(256), 0, stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (p.W > 1 && p.B > 0) {
        const int64_t total = (int64_t)p.B * 2 * p.Hkv * (D / 4);
        hipLaunchKernelGGL(conv_state_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace rba
