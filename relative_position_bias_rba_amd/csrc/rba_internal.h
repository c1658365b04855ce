// Internal launch interface between the C ABI (rba_abi.cpp) and the gfx950
// kernels (attn_kernels.hip, relproj_kernels.hip).  Host-side only types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rba.h"

namespace rba {

// One attention launch.  Query rows are grouped into blocks of QB consecutive
// rows; a workgroup owns one (batch, kv head, query block, split) and all G
// query heads of that kv head, so every K/V tile it stages serves G*QB
// query columns.
struct AttnParams {
    const void *q, *k, *v, *R;
    void *o;
    float *lse;
    float *o_part, *lse_part;  // split partials (splits > 1), else null
    int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2, Rs0, Rs1, Rs2;
    int B, Sq, Skv, Hq, Hkv, G, E, window;
    float scale_log2e;   // scale * log2(e): the dot-product multiplier in the exp2 domain
    float inv_ln_base;   // 1/ln(base) for the log-scale factor, 0 = off
    int QB;              // query rows per block
    int nqb;             // query blocks per (batch, kv head)
    int splits;          // key-range splits per block
    int r_vec;           // R rows allow 16-byte chunk loads
    int kv32;            // K and V of one (batch, kv head) span less than 2^31 bytes
    // Paged K/V (block_table != null): k and v point to page pools, ks0/vs0
    // are page strides, and sequence b has seq_lens[b] keys stored in pages
    // block_table[b * bt_stride + i], page_size keys each (a multiple of the
    // key tile).  Null for contiguous K/V.
    const int *block_table;
    const int *seq_lens;
    int64_t bt_stride;
    int page_size;
    int num_pages;
    // MXFP8 K/V (k_scale != null): k and v hold E4M3 codes (one byte per
    // element, strides ks*/vs* in bytes) and k_scale / v_scale one E8M0 byte
    // per 32 head-dim entries, [.., key, head, 4] with strides kss* / vss*
    // (bytes) laid out like k and v (paged: page, key, head).
    const uint8_t *k_scale, *v_scale;
    int64_t kss0, kss1, kss2, vss0, vss1, vss2;
    int qk8;             // MXFP8 logits: q encoded too, S = QK^T on the scaled FP8 MFMA
    // Relative logits computed inside the prefill kernel (rf != null; then
    // R is null): relative features rf [B, Sq, (Hq,) r_dim] with strides
    // rfs0..2 (rfs2 = 0: shared by the heads), the projection packed by
    // launch_relproj_pack, and bias_ws, G*ceil(E/32)*QB*32 bf16 entries per
    // workgroup of the grid, where each block's rows of R are kept.
    const void *rf;
    int64_t rfs0, rfs1, rfs2;
    int r_dim;
    const void *PT;
    void *bias_ws;
};

// One attention-prologue launch (ShortConv, RMSNorm, cache write) for T new
// tokens of B sequences; bf16 projections, fp32 weights.
struct PrologueParams {
    int B, T, Hq, Hkv, W, Skv;
    float eps;
    const int *cu_new, *seq_lens;
    const __bf16 *q, *k, *v;
    int64_t qs0, qs1, ks0, ks1, vs0, vs1, qos0, qos1;
    const float *conv_wk, *conv_wv, *norm_q, *norm_k;
    __bf16 *state_k, *state_v, *q_out;
    void *k_cache, *v_cache;                   // bf16, or MXFP8 codes when k_scale != null
    int64_t cks0, cks1, cks2, cvs0, cvs1, cvs2;
    uint8_t *k_scale, *v_scale;
    int64_t sks0, sks1, sks2, svs0, svs1, svs2;
    const int *block_table;                    // paged cache when != null
    int64_t bt_stride;
    int page_size, num_pages;
    int max_new;                               // bound on any sequence's new tokens (0 = none given)
};

hipError_t launch_prologue(const PrologueParams &p, hipStream_t stream);

// Kernel variants.  WIDE: two 32-column tiles per wave (prefill, bf16).
enum class AttnVariant { BF16_WIDE, BF16_NARROW, FP32 };

// Largest G*QB one workgroup of the variant covers.
int attn_max_columns(AttnVariant v);

hipError_t launch_attention(const AttnParams &p, AttnVariant v, hipStream_t stream);

// The prefill kernel with the relative logits computed in place (p.rf set):
// `grid` workgroups, each owning bias_ws rows QB*G*E of its own; with
// bias_ws null (r_dim <= 64) each banded tile's logits are computed into LDS
// instead and `grid` is not used.
hipError_t launch_attention_fused(const AttnParams &p, int grid, hipStream_t stream);

// Workgroups the fused prefill kernel runs with for `items` work items on a
// device with `cus` compute units (the bias workspace holds one region each).
int fused_grid(int64_t items, int cus);

// The projection P [Hq, r_dim, E] (bf16, r_dim a multiple of 16) packed as
// MFMA A-operand fragments for the prefill kernel: Hq*ceil(E/32)*32*r_dim
// entries.
hipError_t launch_relproj_pack(int Hq, int r_dim, int E, const void *P, void *PT, hipStream_t stream);

hipError_t launch_combine(const float *o_part, const float *lse_part, int splits, int B, int Sq, int Hq,
                          void *o, bool o_bf16, int64_t os0, int64_t os1, int64_t os2, float *lse,
                          hipStream_t stream);

hipError_t launch_relproj(bool in_bf16, bool out_bf16, int64_t T, int Hq, int r_dim, int E, const void *r,
                          int64_t r_stride, int64_t r_stride_h, const void *P, void *R, hipStream_t stream);

hipError_t launch_mxfp8_quantize(bool in_bf16, int64_t rows, int n, const void *x, int64_t x_stride, void *codes,
                                 int64_t codes_stride, void *scales, int64_t scales_stride, hipStream_t stream);

hipError_t launch_calib_read(const void *buf, int64_t bytes, void *sink, int blocks, hipStream_t stream);

hipError_t launch_calib_mfma(int iters, int blocks, void *sink, hipStream_t stream);

// Device address of the library's split-KV scratch array on the current
// device (looked up on the first call per device).
hipError_t scratch_address(void **out);

}  // namespace rba
