/*
 * rba.h - C ABI of librba: causal grouped-query attention (head dim 128) with a
 * learned, query-conditioned relative-position bias, for AMD MI355X (gfx950).
 *
 * What is computed (sources are web pages, cited by title and section):
 *   [S-RPB]  "SGLang と Miles が Inkling を初日からサポート" (winzheng.jp), section
 *            "相対位置バイアス付き Attention": each token carries a relative
 *            feature r next to q, k, v; a learned matrix P per head maps r to
 *            relative logits indexed by causal distance; the logit of query i,
 *            key j, head h is the scaled dot product plus the entry for i-j;
 *            distances past the extent add nothing; future keys are masked;
 *            layers are sliding-window or full, and full layers may scale the
 *            logits by a length-dependent log factor.
 *   [V-ARCH] "vLLM TML Inkling サポート" (agentlenshq.com), section
 *            "TML Inkling モデルアーキテクチャ": every layer is GQA with head
 *            size 128; the relative term is added before softmax.
 *   [V-OPT]  same page, section "低レイテンシコレクティブとカーネル": the
 *            split-KV factor (num_splits) is chosen per batch size and KV length.
 *   [S-FA4]  "SGLang と Miles が Inkling を初日からサポート", section "Relative
 *            Attention と FA4 経路": the attention kernel runs with MXFP8 data
 *            together with the sheared bias; "vLLM TML Inkling サポート" lists
 *            FP8 global attention as the way to relieve compute and the KV
 *            cache.  MXFP8 is the OCP Microscaling Formats (MX) v1.0 format:
 *            32 consecutive entries share a power-of-two E8M0 scale, entries
 *            are FP8 E4M3 (OCP).
 *   [S-SC]   "SGLang と Miles が Inkling を初日からサポート", sections
 *            "ShortConv：4カ所に現れる短距離因果畳み込み" and "ShortConv 最適化": a
 *            per-channel causal convolution over the current token and the
 *            W-1 before it (W = 4) runs on the K stream before the Q/K
 *            normalisation and on the V stream; the convolutions, the Q/K
 *            RMSNorm and the KV-cache write are one prologue kernel.
 *   [V-KV]   same page, section "vLLM テクニカル最適化": the serving engine keeps
 *            the caches of all layers in one unified KV cache manager, and
 *            multi-token prediction re-runs its heads over the accepted
 *            tokens; read here as sequences of their own lengths whose keys
 *            are reached through a table of fixed-size pages.
 *
 * For batch b, query head h (kv head g = h / (Hq/Hkv)), query row t at
 * position p = Skv - Sq + t, and key j:
 *     visible(p, j) = j <= p  and  (window == 0  or  p - j < window)
 *     f(p)          = log_scale_base > 0 ? ln(p + 1) / ln(log_scale_base) : 1
 *     s(t, j)       = f(p) * ( scale * <q[b,t,h,:], k[b,j,g,:]> + bias )
 *     bias          = (R != NULL and p - j < E) ? R[b,t,h,p-j] : 0
 *     o[b,t,h,:]    = sum_j softmax_j(s(t, .))[j] * v[b,j,g,:]   (visible j only)
 *     lse[b,h,t]    = ln sum_j exp(s(t, j))                        (natural log)
 * and R itself comes from rba_relproj:  R[b,t,h,e] = sum_c r[b,t,c] * P[h,c,e].
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises; all work is enqueued on `stream`
 *     (a hipStream_t; NULL = the default stream) and runs asynchronously.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is launched and outputs are left untouched.  No C++
 *     exception crosses this boundary.
 *   - Strides are in ELEMENTS.  The innermost dimension (d, or E for R) must be
 *     contiguous.  Base pointers must be 16-byte aligned and the b/s/h strides
 *     of q, k, v and o multiples of 16 bytes.
 *   - dtype RBA_BF16: bf16 inputs, fp32 accumulation and softmax, bf16 output,
 *     fp32 lse.  RBA_FP32: fp32 everywhere.
 */
#ifndef RBA_H
#define RBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rba_status {
    RBA_OK = 0,
    RBA_E_INVALID = 1,     /* null pointer, bad shape/stride/alignment, Sq > Skv, window < 0 ... */
    RBA_E_UNSUPPORTED = 2, /* valid but not built: d != 128, dtype combination, r_dim > 128, G > 256 */
    RBA_E_WORKSPACE = 3,   /* decode workspace missing or smaller than rba_decode_workspace_bytes */
    RBA_E_LAUNCH = 4       /* the HIP runtime reported an error when enqueueing a kernel */
} rba_status;

typedef enum rba_dtype {
    RBA_FP32 = 0,
    RBA_BF16 = 1
} rba_dtype;

/* Storage of K and V ([S-FA4]). */
typedef enum rba_kv_format {
    RBA_KV_PLAIN = 0,   /* k, v have the element type dt */
    RBA_KV_MXFP8 = 1,   /* k, v hold OCP E4M3 codes (one byte each); k_scale, v_scale hold one
                           E8M0 code per 32 head-dim entries (value 2^(code-127); code 255 is NaN).
                           Attention then runs over the decoded values.  dt must be RBA_BF16. */
    RBA_KV_MXFP8_QK = 2 /* the cache of RBA_KV_MXFP8, and the logits in MXFP8 as well ([S-FA4]:
                           the attention kernel runs in an MXFP8 configuration; "vLLM TML Inkling
                           サポート" names FP8 attention against compute limits): q is encoded with
                           the cache's rule (blocks of 32 along d) and S = q.K^T is the dot product
                           of the decoded q and K, on the block-scaled FP8 matrix instruction; the
                           probabilities and V are as with RBA_KV_MXFP8.  The prologue writes the
                           same cache for both formats. */
} rba_kv_format;

/* Shapes, pointers and options of one attention call (prefill or decode).
 *   q, o : [B, Sq, Hq, d]    strides q_s / o_s = {b, s, h}
 *   k, v : [B, Skv, Hkv, d]  strides k_s / v_s = {b, s, h}
 *   R    : [B, Sq, Hq, E]    strides R_s = {b, t, h}; NULL = no bias (E ignored)
 *   lse  : [B, Hq, Sq] fp32, contiguous; NULL = not written
 *   kv_format = RBA_KV_MXFP8 or RBA_KV_MXFP8_QK: k_scale, v_scale : [B, Skv, Hkv, d/32] bytes,
 *          strides k_scale_s / v_scale_s = {b, s, h}, the d/32 codes of a row
 *          contiguous (paged: laid out like the pools, {page, key, head}).
 *          k_s / v_s are then byte strides and must be multiples of 16.
 *   A zero-initialised tail (kv_format 0, scales NULL) is the plain format. */
typedef struct rba_attn_args {
    rba_dtype dt;
    int B, Sq, Skv, Hq, Hkv, d, E;
    int window;            /* 0 = full causal; > 0: key visible iff 0 <= p - j < window */
    float scale;           /* multiplies q.k only; finite and > 0, usually 1/sqrt(d) */
    float log_scale_base;  /* 0 = off; > 1: logits multiplied by ln(p+1)/ln(base) */
    const void *q, *k, *v;
    const void *R;
    void *o;
    float *lse;
    int64_t q_s[3], k_s[3], v_s[3], o_s[3], R_s[3];
    int kv_format;         /* rba_kv_format */
    const void *k_scale, *v_scale;
    int64_t k_scale_s[3], v_scale_s[3];
} rba_attn_args;

/* R = r . P per head  ([S-RPB], the relative-logit projection):
 *     R[t, h, e] = sum_c r[t, (h,) c] * P[h, c, e]
 *   r : [T, r_dim] shared by all heads (r_stride_h = 0), or [T, Hq, r_dim]
 *       one feature per head (r_stride_h >= r_dim); token stride r_stride_t
 *       (>= r_dim, resp. >= Hq * r_stride_h) and head stride r_stride_h in
 *       elements, channel contiguous, in_dt
 *   P : [Hq, r_dim, E] (in_dt), contiguous
 *   R : [T, Hq, E] (out_dt), contiguous
 * in_dt/out_dt may each be RBA_BF16 or RBA_FP32 (fp32 accumulation always;
 * bf16 output is rounded to nearest even).  1 <= r_dim <= 128, E >= 1.
 * T = 0 is a no-op.                                                          */
rba_status rba_relproj(rba_dtype in_dt, rba_dtype out_dt, int64_t T, int Hq, int r_dim, int E,
                       const void *r, int64_t r_stride_t, int64_t r_stride_h, const void *P, void *R,
                       void *stream);

/* Attention over all keys for every query row ([S-RPB], [V-ARCH]); one pass,
 * no workspace.  Any 1 <= Sq <= Skv is accepted (rows bottom-right aligned);
 * Sq = 0 is a no-op.                                                         */
rba_status rba_attn_prefill(const rba_attn_args *args, void *stream);

/* The projection weights repacked for rba_attn_prefill_fused ([S-RPB]):
 * P [Hq, r_dim, E] bf16, contiguous, 16-byte aligned, is rewritten into PT,
 * rba_relproj_packed_bytes(Hq, r_dim, E) bytes (16-byte aligned), in the
 * order the fused kernel's matrix-core operands read it: for head h, tile
 * eb of 32 distances, k-step k of 16 channels and lane l of a 64-lane wave,
 * the 8 values P[h, 16k + 8(l/32) + x, 32 eb + m(l % 32)], x = 0..7, are
 * consecutive, with m(i) = 16((i/4) % 2) + 4(i/8) + i % 4; entries past E are
 * zero.  The layout is otherwise opaque.  r_dim a multiple of 16, at most 128
 * (else RBA_E_UNSUPPORTED).  A weight is packed once and reused.            */
size_t rba_relproj_packed_bytes(int Hq, int r_dim, int E);
rba_status rba_relproj_pack(int Hq, int r_dim, int E, const void *P, void *PT, void *stream);

/* Relative-feature operands of rba_attn_prefill_fused ([S-RPB]):
 *   r   : [B, Sq, r_dim] shared by the heads (r_s[2] = 0) or [B, Sq, Hq,
 *         r_dim] one feature per head; strides r_s = {b, t, h} in elements,
 *         channel contiguous, multiples of 8; bf16, 16-byte aligned
 *   PT  : the projection as packed by rba_relproj_pack, 16-byte aligned
 *   r_dim : a multiple of 16, 16 <= r_dim <= 128                            */
typedef struct rba_relbias {
    int r_dim;
    const void *r;
    int64_t r_s[3];
    const void *PT;
} rba_relbias;

/* Bytes of workspace rba_attn_prefill_fused needs for `args` on the current
 * device: one region of QB * (Hq/Hkv) * 32 ceil(E/32) bf16 entries per
 * workgroup (QB = query rows per block, at most 32), where a workgroup keeps
 * the rows of R of the query block it is working on.
 * 0 if the call is invalid or unsupported.                                  */
size_t rba_prefill_fused_workspace_bytes(const rba_attn_args *args);

/* rba_relproj and rba_attn_prefill in one launch ([S-RPB]): the same outputs,
 * bit for bit, as rba_relproj (bf16 out) into an R that rba_attn_prefill then
 * reads, with the relative logits computed inside the attention kernel on
 * MFMA, in one of two ways:
 *   workspace given: each workgroup computes the rows of R its query block
 *     needs (all E distances of its rows) into its region of `workspace` and
 *     reads them from there, so no R for the whole problem is materialised;
 *   workspace NULL (r_dim <= 64): each wave computes, for every key tile that
 *     meets distances below E, the logits of its query columns that the tile
 *     needs straight into LDS: no R is written to memory at all.
 * With r_dim > 64 the workspace is required.
 * args->R must be NULL (the bias comes from rb); args->E is the extent (>= 1).
 * Supported where rba_attn_prefill runs its two-group bf16 kernel: bf16,
 * plain K/V, (Hq/Hkv) * min(Sq, 32) > 128, K/V spans of one (batch, kv
 * head) under 2^31 bytes; otherwise RBA_E_UNSUPPORTED.  Returns
 * RBA_E_WORKSPACE if a workspace is given but unaligned (16 bytes) or smaller
 * than rba_prefill_fused_workspace_bytes(args), or if it is NULL with
 * r_dim > 64.  The workspace is scratch: its contents before and after the
 * call carry no meaning; two calls in flight at once need two workspaces.   */
rba_status rba_attn_prefill_fused(const rba_attn_args *args, const rba_relbias *rb, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Split-KV count the library picks for `args` on a device with `num_cus`
 * compute units ([V-OPT]: from batch, kv heads and KV length).  num_cus <= 0
 * queries the current device.  Returns >= 1, or 0 if args is invalid.      */
int rba_num_splits(const rba_attn_args *args, int num_cus);

/* Bytes of workspace rba_attn_decode needs for `num_splits` splits
 * (0 = the heuristic's choice on the current device; split-KV decode as in
 * [V-OPT], "vLLM TML Inkling サポート", section
 * "低レイテンシコレクティブとカーネル").  0 when one split is
 * used (no workspace needed).  Layout: fp32 partial outputs
 * [splits][B][Sq][Hq][d] followed by fp32 partial lse [splits][B][Sq][Hq].  */
size_t rba_decode_workspace_bytes(const rba_attn_args *args, int num_splits);

/* Split-KV attention for a few query rows against a long cache ([V-OPT]:
 * the attention splits the key range, with the split count chosen per batch
 * and KV length; "vLLM TML Inkling サポート", section
 * "低レイテンシコレクティブとカーネル"); the scores are those of
 * rba_attn_prefill ([S-RPB]).  Each split covers a contiguous range of key
 * tiles and writes its normalised partial
 * output and lse into `workspace`; rba_splitkv_combine then merges them on
 * the same stream.  num_splits = 0 uses rba_num_splits; 1 writes o directly.
 * Returns RBA_E_WORKSPACE if workspace is NULL or too small when needed.   */
rba_status rba_attn_decode(const rba_attn_args *args, int num_splits, void *workspace,
                           size_t workspace_bytes, void *stream);

/* rba_attn_decode without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the split partials go to a scratch array
 * of RBA_DECODE_SCRATCH_BYTES that the library holds in device memory, one per
 * device, for the life of the process.  The call itself allocates nothing.
 * Same arguments, results and errors as rba_attn_decode; returns
 * RBA_E_WORKSPACE before any launch when the partials of `num_splits` splits
 * (rba_decode_workspace_bytes) exceed RBA_DECODE_SCRATCH_BYTES, and
 * RBA_E_LAUNCH if the scratch array's address cannot be looked up.  Every
 * call on one device shares that device's array (each call overwrites all of
 * the part it reads): calls that overlap on one device, on different streams
 * or from different threads without ordering, race.                        */
#define RBA_DECODE_SCRATCH_BYTES (16u << 20)
rba_status rba_attn_decode_noalloc(const rba_attn_args *args, int num_splits, void *stream);

/* Paged, variable-length K/V for rba_attn_paged ([V-KV]).  The cache is a
 * pool of pages of page_size consecutive keys of every kv head:
 *   args->k, args->v : [num_pages][page_size][Hkv][d]  strides k_s / v_s =
 *                      {page, key, head} (elements)
 * Sequence b has seq_lens[b] keys; key j of it is row j % page_size of page
 * block_table[b * bt_stride + j / page_size].  Its Sq query rows are its last
 * Sq positions: query row t sits at position seq_lens[b] - Sq + t.
 *   block_table : device int32 [B][bt_stride]; entries outside [0, num_pages)
 *                 are clamped into it on the device (never read out of bounds)
 *   seq_lens    : device int32 [B]; a length outside [Sq, args->Skv] is
 *                 clamped into it on the device.  args->Skv is the longest
 *                 length the table covers and drives the split heuristic.
 *   page_size   : a positive multiple of 64 (a page holds whole key tiles)
 *   bt_stride   : >= ceil(args->Skv / page_size)
 * The host cannot check device-side values; a table that names pages the
 * caller did not fill yields their contents, not an error.                 */
typedef struct rba_paged_kv {
    const int32_t *block_table;
    const int32_t *seq_lens;
    int64_t bt_stride;
    int page_size;
    int num_pages;
} rba_paged_kv;

/* Attention of each sequence's last Sq query rows over its own paged keys
 * ([V-KV], [S-RPB]); the same logits, mask, bias and outputs as
 * rba_attn_decode (q, o, R and lse keep their [B, Sq, ...] layouts and the
 * same workspace rules and size, rba_decode_workspace_bytes(args, splits)).
 * num_splits = 0 uses rba_num_splits(args): splits then cover each
 * sequence's own key range.  Also serves chunked prefill and multi-token
 * verification (Sq > 1) over a paged cache.                                */
rba_status rba_attn_paged(const rba_attn_args *args, const rba_paged_kv *kv, int num_splits, void *workspace,
                          size_t workspace_bytes, void *stream);

/* MXFP8 encoding of `rows` vectors of n entries ([S-FA4]; the KV-cache
 * write of an MXFP8 cache):
 *   x      : [rows, n] in_dt (RBA_BF16 or RBA_FP32), row stride x_stride
 *            elements; 16-byte aligned rows (x and x_stride * size)
 *   codes  : [rows, n] bytes, row stride codes_stride (4-byte aligned rows)
 *   scales : [rows, n/32] bytes, row stride scales_stride
 * Block k of a row is entries [32k, 32k+32).  Its scale code is e + 127 with
 * e = floor(log2(max |x|)) - 8 clamped to [-127, 127] (-127 for an all-zero
 * block); each code is the E4M3 value nearest to x / 2^e, ties to even,
 * saturated to +-448.  n a multiple of 32, 32 <= n <= 65536.  Inputs must
 * be finite.  rows = 0 is a no-op.                                          */
rba_status rba_mxfp8_quantize(rba_dtype in_dt, int64_t rows, int n, const void *x, int64_t x_stride, void *codes,
                              int64_t codes_stride, void *scales, int64_t scales_stride, void *stream);

/* Attention prologue ([S-SC]): for T new tokens of B sequences, in one pass,
 *   q_out[t, h]            = RMSNorm(q[t, h]; norm_q)
 *   cache K row (b, pos, g) = RMSNorm(ShortConv_k(k)[t, g]; norm_k)
 *   cache V row (b, pos, g) = ShortConv_v(v)[t, g]
 * with ShortConv(x)[t, g, c] = sum_{i < conv_w} w[g*d + c][i] * x at the
 * position i before t of the same sequence (tap 0 = the token itself; rows
 * before the sequence start read zero; rows before this call's new tokens
 * come from the conv state) and RMSNorm(x; w) = x * w / sqrt(mean(x^2) + eps)
 * over the d entries of one head.  Sequence b owns token rows
 * cu_new[b] .. cu_new[b+1]-1 (n_b of them), which take cache positions
 * seq_lens[b] - n_b .. seq_lens[b] - 1.  Afterwards the conv state of each
 * sequence holds the pre-convolution k and v rows of its last conv_w - 1
 * positions.
 *   cu_new     : device int32 [B+1], non-decreasing, cu_new[0] = 0, cu_new[B] = T
 *   seq_lens   : device int32 [B], keys after this append (clamped on the
 *                device to [n_b, cache->Skv])
 *   q, k, v    : bf16 [T, Hq|Hkv, d], strides {token, head} (elements, multiples of 4)
 *   conv_wk/wv : fp32 [Hkv*d, conv_w] contiguous;  norm_q/norm_k : fp32 [d]
 *   state_k/v  : bf16 [B, conv_w - 1, Hkv, d] contiguous, read and updated
 *                (NULL allowed when conv_w = 1)
 *   q_out      : bf16 [T, Hq, d], strides {token, head}
 * The cache is described exactly as rba_attn_decode reads it: `cache` gives
 * k, v, k_s, v_s, Hkv, Skv, d, kv_format and (MXFP8) the scales; its other
 * fields are ignored.  MXFP8 caches receive the bf16 row encoded as by
 * rba_mxfp8_quantize.  `paged` (NULL = dense [B, Skv, Hkv, d]) selects a
 * block-table cache as for rba_attn_paged.  d = 128, 1 <= conv_w <= 8,
 * eps > 0.  T = 0 is a no-op.
 *   max_new    : 0, or a bound on every n_b.  With 1 <= max_new <= 32 the
 *                prologue is one launch in which each sequence's K and V rows
 *                are taken in order by one half wave per kv head, which also
 *                advances that sequence's conv state (decode and MTP verify
 *                batches); otherwise new tokens are taken in chunks of 8 and
 *                a second launch advances the states.  Both give the same
 *                bits; a bound that a sequence exceeds is not an error (its
 *                tokens are all still taken, only more slowly).  < 0 is
 *                RBA_E_INVALID.                                           */
typedef struct rba_prologue_args {
    int B, T, Hq, Hkv, d;
    int conv_w;
    float eps;
    const int32_t *cu_new;
    const int32_t *seq_lens;
    const void *q, *k, *v;
    int64_t q_s[2], k_s[2], v_s[2];
    const float *conv_wk, *conv_wv;
    const float *norm_q, *norm_k;
    void *state_k, *state_v;
    void *q_out;
    int64_t q_out_s[2];
    int max_new;
} rba_prologue_args;

rba_status rba_attn_prologue(const rba_prologue_args *args, const rba_attn_args *cache, const rba_paged_kv *paged,
                             void *stream);

/* Merge split partials into args->o (and args->lse if non-NULL); the
 * combine step of [V-OPT]'s split-KV decode ("vLLM TML Inkling サポート",
 * section "低レイテンシコレクティブとカーネル"), exact because each split's
 * softmax is renormalised by its lse:
 *   M = max_s lse_s;  w_s = exp(lse_s - M);  o = sum_s w_s o_s / sum_s w_s;
 *   lse = M + ln sum_s w_s.  Splits with lse = -inf get weight 0; a row whose
 *   splits are all empty gets o = 0, lse = -inf.
 *   o_part : [num_splits][B][Sq][Hq][d] fp32 contiguous
 *   lse_part : [num_splits][B][Sq][Hq] fp32 contiguous                      */
rba_status rba_splitkv_combine(const float *o_part, const float *lse_part, int num_splits,
                               const rba_attn_args *args, void *stream);

/* Measurement aids (not part of the attention path).  They report what this
 * device attains, so that the kernels' rates can be read against it as well
 * as against the published peaks.
 *   rba_calib_read : read `bytes` (a multiple of 16384) of device memory at
 *                    `buf` once with 16-byte loads from 2 workgroups per CU;
 *                    `sink` is 4 bytes of device memory that is (almost
 *                    surely) left unwritten.  Time it with events.
 *   rba_calib_mfma : 8 workgroups per CU of 4 waves each run `iters` x 4
 *                    back-to-back bf16 32x32x16 matrix instructions; *flops
 *                    (host, may be NULL) receives the flop count of the
 *                    launch.  Same sink rule.                                */
rba_status rba_calib_read(const void *buf, size_t bytes, void *sink, void *stream);
rba_status rba_calib_mfma(int iters, void *sink, double *flops, void *stream);

/* Static description of a status code. */
const char *rba_status_string(rba_status status);

/* Version of the library as an integer (major*10000 + minor*100 + patch). */
int rba_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RBA_H */
