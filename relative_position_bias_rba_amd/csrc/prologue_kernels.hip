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
// (32 lanes x 4 channels of a 128-entry row) owns one head - a q head
// (RMSNorm), a k head (convolution over the token and the W-1 rows before it,
// then RMSNorm) or a v head (convolution) - for 8 consecutive tokens, keeping
// its taps and the previous rows in registers.
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

__device__ __forceinline__ void unpack4(u32x2 w, float x[4]) {
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
__device__ __forceinline__ void rms_norm4(float x[4], const float g[4], float eps) {
    float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) ss += __shfl_xor(ss, m, 32);
    const float r = 1.f / sqrtf(ss * (1.f / D) + eps);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = x[e] * r * g[e];
}

constexpr int TC = 8;          // consecutive tokens per half wave
constexpr int kMaxTaps = 8;    // largest tap count
constexpr int kSeqMaxNew = 32; // largest max_new served by the one-launch (per-sequence) kernel
constexpr int TCS = 16;        // new K/V rows per load batch of the one-launch kernel (a verify batch in one)

// The sequence owning token t: the last b with cu_new[b] <= t.
__device__ __forceinline__ int seq_of(const int *cu, int B, int t) {
    int lo = 0, hi = B;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

// Writes one convolved (and for K normalised) row: this lane's 4 channels of
// kv head g at cache position pos of sequence b, dense or through the block
// table, as bf16 or as MXFP8 (eight lanes per 32-entry block share the block
// maximum).
template <bool F8, bool PG>
__device__ __forceinline__ void write_cache_row(const PrologueParams &p, bool isk, int b, int pos, int g, int c0,
                                                int lane, const float acc[4]) {
    const int64_t cs0 = isk ? p.cks0 : p.cvs0, cs1 = isk ? p.cks1 : p.cvs1, cs2 = isk ? p.cks2 : p.cvs2;
    const int64_t ss0 = isk ? p.sks0 : p.svs0, ss1 = isk ? p.sks1 : p.svs1, ss2 = isk ? p.sks2 : p.svs2;
    int64_t off, soff;                    // element (= byte for MXFP8) and scale offsets of the row
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
        float y[4];
        y[0] = __builtin_bit_cast(float, h[0] << 16);
        y[1] = __builtin_bit_cast(float, h[0] & 0xffff0000u);
        y[2] = __builtin_bit_cast(float, h[1] << 16);
        y[3] = __builtin_bit_cast(float, h[1] & 0xffff0000u);
        float amax = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        amax = fmaxf(amax, __shfl_xor(amax, 4));
        int ex = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 1 - 8 : -127;
        ex = min(max(ex, -127), 127);
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[j] = fminf(fmaxf(ldexpf(y[j], -ex), -448.f), 448.f);
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(sc[0], sc[1], 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(sc[2], sc[3], wd, true);
        *(unsigned *)((uint8_t *)(isk ? p.k_cache : p.v_cache) + off + c0) = (unsigned)wd;
        if ((lane & 7) == 0)
            ((uint8_t *)(isk ? p.k_scale : p.v_scale))[soff + (lane >> 3)] = (uint8_t)(ex + 127);
    }
}

// Half a wave owns one head row kind (q head, k head or v head) for TC
// consecutive tokens; its 4 channels' taps and norm weights stay in
// registers, and so do the pre-convolution rows of the last W-1 positions of
// the current sequence (reloaded from the new rows, the conv state or zeros
// when a sequence starts inside the chunk).
// WMAX: taps held in registers (W <= WMAX).
template <bool F8, bool PG, int WMAX>
__global__ __launch_bounds__(256) void prologue_kernel(const PrologueParams p) {
    const int64_t item = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    const int lane = threadIdx.x & 31;
    const int HR = p.Hq + 2 * p.Hkv;
    const int nchunk = (p.T + TC - 1) / TC;
    if (item >= (int64_t)nchunk * HR) return;   // the whole half wave leaves together
    const int chunk = (int)(item / HR);
    const int hr = (int)(item - (int64_t)chunk * HR);
    const int t0 = chunk * TC, t1 = min(p.T, t0 + TC);
    const int c0 = 4 * lane;

    // the chunk's rows of this head, all loads in flight together
    const bool isq = hr < p.Hq;
    const bool isk = !isq && hr < p.Hq + p.Hkv;
    const int g = isq ? hr : hr - p.Hq - (isk ? 0 : p.Hkv);
    const __bf16 *src = isq ? p.q : isk ? p.k : p.v;
    const int64_t s0 = isq ? p.qs0 : isk ? p.ks0 : p.vs0, s1 = isq ? p.qs1 : isk ? p.ks1 : p.vs1;
    u32x2 raw[TC];
#pragma unroll
    for (int j = 0; j < TC; ++j)
        raw[j] = t0 + j < t1 ? *(const u32x2 *)(src + (int64_t)(t0 + j) * s0 + (int64_t)g * s1 + c0) : u32x2{0u, 0u};

    if (isq) {                                // q: RMSNorm only
        float gq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) gq[e] = p.norm_q[c0 + e];
#pragma unroll
        for (int j = 0; j < TC; ++j) {
            if (t0 + j >= t1) break;
            float x[4];
            unpack4(raw[j], x);
            rms_norm4(x, gq, p.eps);
            *(u32x2 *)(p.q_out + (int64_t)(t0 + j) * p.qos0 + (int64_t)hr * p.qos1 + c0) = pack4(x);
        }
        return;
    }
    const __bf16 *state = isk ? p.state_k : p.state_v;
    const int W = p.W;
    float w[4][WMAX], gk[4];
    {
        const float *wp = (isk ? p.conv_wk : p.conv_wv) + (int64_t)(g * D + c0) * W;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int l = 0; l < WMAX; ++l) w[e][l] = l < W ? wp[e * W + l] : 0.f;
            gk[e] = isk ? p.norm_k[c0 + e] : 1.f;
        }
    }
    float hist[WMAX - 1][4];                  // hist[l - 1] = pre-convolution row l positions back
    int b = -1, a0 = 0, a1 = 0, n = 0, L = 0;
#pragma unroll
    for (int j = 0; j < TC; ++j) {
        const int t = t0 + j;
        if (t >= t1) break;
        if (b < 0 || t >= a1) {
            // a new sequence: bounds (device values clamped so every access
            // stays in its tensor) and the rows before t
            b = seq_of(p.cu_new, p.B, t);
            a0 = min(max(p.cu_new[b], 0), p.T);
            a1 = min(max(p.cu_new[b + 1], a0), p.T);
            n = a1 - a0;
            L = min(max(p.seq_lens[b], n), p.Skv);
            const int i = t - a0;
#pragma unroll
            for (int l = 1; l < WMAX; ++l) {
#pragma unroll
                for (int e = 0; e < 4; ++e) hist[l - 1][e] = 0.f;
                if (l < W && L - n + i - l >= 0 && i >= 0) {
                    const __bf16 *rp = (i - l >= 0)
                                           ? src + (int64_t)(t - l) * s0 + (int64_t)g * s1
                                           : state + (((int64_t)b * (W - 1) + (W - 1 + i - l)) * p.Hkv + g) * D;
                    load4(rp + c0, hist[l - 1]);
                }
            }
        }
        const int i = t - a0;
        if (i < 0 || i >= n) continue;        // token outside every sequence's range
        const int pos = L - n + i;
        float x[4], acc[4];
        unpack4(raw[j], x);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[e] = w[e][0] * x[e];
#pragma unroll
            for (int l = 1; l < WMAX; ++l) acc[e] = fmaf(w[e][l], hist[l - 1][e], acc[e]);
        }
        // slide the window
#pragma unroll
        for (int l = WMAX - 2; l > 0; --l)
#pragma unroll
            for (int e = 0; e < 4; ++e) hist[l][e] = hist[l - 1][e];
#pragma unroll
        for (int e = 0; e < 4; ++e) hist[0][e] = x[e];
        if (isk) rms_norm4(acc, gk, p.eps);

        write_cache_row<F8, PG>(p, isk, b, pos, g, c0, lane, acc);
    }
}

// One launch for batches whose sequences each bring few new tokens (the
// caller's bound max_new: decode and MTP verify).  q rows are normalised per
// chunk of TC tokens as in prologue_kernel; for K and V, half a wave owns one
// stream and kv head of one sequence and takes all of that sequence's new
// tokens in order, TCS at a time.  It is then the only reader of the sequence's conv
// state for its stream and kv head, so it also advances that state itself
// (the rows of the sequence's last W-1 positions, old rows kept verbatim), and
// no second kernel is needed.  All of its loads except the rows of later
// chunks are issued together at the start.
template <bool F8, bool PG, int WMAX>
__global__ __launch_bounds__(256) void prologue_seq_kernel(const PrologueParams p) {
    const int64_t item = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    const int lane = threadIdx.x & 31;
    const int c0 = 4 * lane;
    // items: (chunk of TC tokens, q head) first, as in prologue_kernel, then
    // (sequence, k or v, kv head)
    const int64_t nq = (int64_t)((p.T + TC - 1) / TC) * p.Hq;
    if (item < nq) {                          // q: RMSNorm only
        const int chunk = (int)(item / p.Hq);
        const int hq = (int)(item - (int64_t)chunk * p.Hq);
        const int t0 = chunk * TC, t1 = min(p.T, t0 + TC);
        const __bf16 *srow = p.q + (int64_t)hq * p.qs1 + c0;
        u32x2 raw[TC];
#pragma unroll
        for (int j = 0; j < TC; ++j) raw[j] = t0 + j < t1 ? *(const u32x2 *)(srow + (int64_t)(t0 + j) * p.qs0) : u32x2{0u, 0u};
        float gq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) gq[e] = p.norm_q[c0 + e];
#pragma unroll
        for (int j = 0; j < TC; ++j) {
            if (t0 + j >= t1) break;
            float x[4];
            unpack4(raw[j], x);
            rms_norm4(x, gq, p.eps);
            *(u32x2 *)(p.q_out + (int64_t)(t0 + j) * p.qos0 + (int64_t)hq * p.qos1 + c0) = pack4(x);
        }
        return;
    }
    const int64_t kvi = item - nq;
    if (kvi >= (int64_t)p.B * 2 * p.Hkv) return;   // the whole half wave leaves together
    const int b = (int)(kvi / (2 * p.Hkv));
    const int hr = (int)(kvi - (int64_t)b * 2 * p.Hkv);
    const bool isk = hr < p.Hkv;
    const int g = isk ? hr : hr - p.Hkv;
    // device values clamped so that every access stays in its tensor
    const int a0 = min(max(p.cu_new[b], 0), p.T);
    const int a1 = min(max(p.cu_new[b + 1], a0), p.T);
    const int n = a1 - a0;
    const int L = min(max(p.seq_lens[b], n), p.Skv);
    const int64_t s0 = isk ? p.ks0 : p.vs0;
    const __bf16 *srow = (isk ? p.k : p.v) + (int64_t)g * (isk ? p.ks1 : p.vs1) + c0;

    if (n == 0) return;                       // no new rows: cache and state unchanged
    __bf16 *const state = isk ? p.state_k : p.state_v;
    const int W = p.W;
    const int64_t st_b = (int64_t)b * (W - 1);   // first state row of this sequence
    auto state_row = [&](int r) __attribute__((always_inline)) { return state + ((st_b + r) * p.Hkv + g) * D + c0; };

    // loads issued together: the old state rows (verbatim), the new rows that
    // end up in the advanced state, the taps and norm weight, the first chunk
    u32x2 old[WMAX - 1], keep[WMAX - 1];
#pragma unroll
    for (int r = 0; r < WMAX - 1; ++r) old[r] = r < W - 1 ? *(const u32x2 *)state_row(r) : u32x2{0u, 0u};
    // advanced state row j = pre-convolution row of position L - (W-1) + j:
    // old row n + j while n + j < W - 1, else new row a0 + n + j - (W - 1)
#pragma unroll
    for (int j = 0; j < WMAX - 1; ++j) {
        const int k = n + j;
        keep[j] = (j < W - 1 && k >= W - 1) ? *(const u32x2 *)(srow + (int64_t)(a0 + k - (W - 1)) * s0)
                                            : u32x2{0u, 0u};
    }
    float w[4][WMAX], gk[4];
    {
        const float *wp = (isk ? p.conv_wk : p.conv_wv) + (int64_t)(g * D + c0) * W;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int l = 0; l < WMAX; ++l) w[e][l] = l < W ? wp[e * W + l] : 0.f;
            gk[e] = isk ? p.norm_k[c0 + e] : 1.f;
        }
    }
    u32x2 raw[TCS];
#pragma unroll
    for (int j = 0; j < TCS; ++j) raw[j] = a0 + j < a1 ? *(const u32x2 *)(srow + (int64_t)(a0 + j) * s0) : u32x2{0u, 0u};

    // history of the first new token: row l positions back is old row
    // W - 1 - l, zero before the sequence's first position
    float hist[WMAX - 1][4];
#pragma unroll
    for (int l = 1; l < WMAX; ++l) {
        u32x2 v = u32x2{0u, 0u};
#pragma unroll
        for (int r = 0; r < WMAX - 1; ++r)
            if (r == W - 1 - l) v = old[r];
        if (!(l < W && L - n - l >= 0)) v = u32x2{0u, 0u};
        unpack4(v, hist[l - 1]);
    }

    for (int t0 = a0; t0 < a1; t0 += TCS) {
        if (t0 > a0) {
#pragma unroll
            for (int j = 0; j < TCS; ++j)
                raw[j] = t0 + j < a1 ? *(const u32x2 *)(srow + (int64_t)(t0 + j) * s0) : u32x2{0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < TCS; ++j) {
            const int t = t0 + j;
            if (t >= a1) break;
            const int pos = L - n + (t - a0);
            float x[4], acc[4];
            unpack4(raw[j], x);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] = w[e][0] * x[e];
#pragma unroll
                for (int l = 1; l < WMAX; ++l) acc[e] = fmaf(w[e][l], hist[l - 1][e], acc[e]);
            }
#pragma unroll
            for (int l = WMAX - 2; l > 0; --l)
#pragma unroll
                for (int e = 0; e < 4; ++e) hist[l][e] = hist[l - 1][e];
#pragma unroll
            for (int e = 0; e < 4; ++e) hist[0][e] = x[e];
            if (isk) rms_norm4(acc, gk, p.eps);
            write_cache_row<F8, PG>(p, isk, b, pos, g, c0, lane, acc);
        }
    }

    // advance the state (every read of the old rows is done above)
#pragma unroll
    for (int j = 0; j < WMAX - 1; ++j) {
        if (j >= W - 1) break;
        const int k = n + j;
        u32x2 v = keep[j];
        if (k < W - 1) {
#pragma unroll
            for (int r = 0; r < WMAX - 1; ++r)
                if (r == k) v = old[r];
        }
        *(u32x2 *)state_row(j) = v;
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
    if (p.max_new >= 1 && p.max_new <= kSeqMaxNew && p.B > 0) {
        // one launch: a half wave per (sequence, head row kind)
        const int64_t items = (int64_t)((p.T + TC - 1) / TC) * p.Hq + (int64_t)p.B * 2 * p.Hkv;
        const int64_t grid = (items + 7) / 8;
        if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
        const bool f8 = p.k_scale != nullptr, pg = p.block_table != nullptr, w4 = p.W <= 4;
#define RBA_PROS(F8, PG, WM) \
    hipLaunchKernelGGL((prologue_seq_kernel<F8, PG, WM>), dim3((unsigned)grid), dim3(256), 0, stream, p)
        if (f8 && pg) {
            if (w4) RBA_PROS(true, true, 4); else RBA_PROS(true, true, kMaxTaps);
        } else if (f8) {
            if (w4) RBA_PROS(true, false, 4); else RBA_PROS(true, false, kMaxTaps);
        } else if (pg) {
            if (w4) RBA_PROS(false, true, 4); else RBA_PROS(false, true, kMaxTaps);
        } else {
            if (w4) RBA_PROS(false, false, 4); else RBA_PROS(false, false, kMaxTaps);
        }
#undef RBA_PROS
        return hipGetLastError();
    }
    const int64_t items = (int64_t)((p.T + TC - 1) / TC) * (p.Hq + 2 * p.Hkv);
    if (items > 0) {
        const int64_t grid = (items + 7) / 8;
        if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
        const bool f8 = p.k_scale != nullptr, pg = p.block_table != nullptr, w4 = p.W <= 4;
#define RBA_PRO(F8, PG, WM) \
    hipLaunchKernelGGL((prologue_kernel<F8, PG, WM>), dim3((unsigned)grid), dim3(256), 0, stream, p)
        if (f8 && pg) {
            if (w4) RBA_PRO(true, true, 4); else RBA_PRO(true, true, kMaxTaps);
        } else if (f8) {
            if (w4) RBA_PRO(true, false, 4); else RBA_PRO(true, false, kMaxTaps);
        } else if (pg) {
            if (w4) RBA_PRO(false, true, 4); else RBA_PRO(false, true, kMaxTaps);
        } else {
            if (w4) RBA_PRO(false, false, 4); else RBA_PRO(false, false, kMaxTaps);
        }
#undef RBA_PRO
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
