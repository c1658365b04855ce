// C ABI of librba: argument validation, work planning (query-block size,
// split-KV count) and kernel dispatch.  Declarations and the meaning of every
// argument are in include/rba.h.
#include "rba.h"

#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "rba_internal.h"

namespace {

constexpr int kHeadDim = 128;
constexpr int kMaxSplits = 1024;
constexpr int kMinTilesPerSplit = 4;
constexpr int kPageQuantum = 64;   // paged K/V: a page holds whole 64-key tiles
constexpr size_t kCalibReadQuantum = 16384;
constexpr int kMaxConvTaps = 8;   // the read probe covers 1024 16-byte chunks per step

int elem_size(rba_dtype dt) { return dt == RBA_BF16 ? 2 : 4; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool strides_ok(const int64_t s[3], int64_t mult) {
    for (int i = 0; i < 3; ++i)
        if (s[i] < 0 || s[i] % mult != 0) return false;
    return true;
}

// Bytes per K/V element in memory.
bool kv_mx(const rba_attn_args *a) { return a->kv_format == RBA_KV_MXFP8 || a->kv_format == RBA_KV_MXFP8_QK; }
int kv_elem_size(const rba_attn_args *a) { return kv_mx(a) ? 1 : elem_size(a->dt); }

rba_status validate_attn(const rba_attn_args *a) {
    if (a == nullptr) return RBA_E_INVALID;
    if (a->dt != RBA_BF16 && a->dt != RBA_FP32) return RBA_E_UNSUPPORTED;
    if (a->kv_format != RBA_KV_PLAIN && !kv_mx(a)) return RBA_E_INVALID;
    if (kv_mx(a) && a->dt != RBA_BF16) return RBA_E_UNSUPPORTED;
    if (a->d <= 0) return RBA_E_INVALID;
    if (a->d != kHeadDim) return RBA_E_UNSUPPORTED;
    if (a->B < 0 || a->Sq < 0 || a->Skv < 0 || a->Hq < 1 || a->Hkv < 1) return RBA_E_INVALID;
    if (a->Hq % a->Hkv != 0) return RBA_E_INVALID;
    if (a->Sq > a->Skv) return RBA_E_INVALID;
    if (a->window < 0) return RBA_E_INVALID;
    if (!isfinite(a->scale) || !(a->scale > 0.f)) return RBA_E_INVALID;
    if (!(a->log_scale_base == 0.f || (isfinite(a->log_scale_base) && a->log_scale_base > 1.f)))
        return RBA_E_INVALID;
    if (a->R != nullptr && a->E < 1) return RBA_E_INVALID;
    const int G = a->Hq / a->Hkv;
    const int maxc = rba::attn_max_columns(a->dt == RBA_FP32 ? rba::AttnVariant::FP32 : rba::AttnVariant::BF16_WIDE);
    if (G > maxc) return RBA_E_UNSUPPORTED;
    if ((int64_t)a->B * a->Sq == 0) return RBA_OK;  // nothing to do, pointers unused
    if (a->q == nullptr || a->k == nullptr || a->v == nullptr || a->o == nullptr) return RBA_E_INVALID;
    if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->o, 16)) return RBA_E_INVALID;
    const int64_t ch = 16 / elem_size(a->dt);
    const int64_t kch = 16 / kv_elem_size(a);
    if (!strides_ok(a->q_s, ch) || !strides_ok(a->k_s, kch) || !strides_ok(a->v_s, kch) || !strides_ok(a->o_s, ch))
        return RBA_E_INVALID;
    if (kv_mx(a)) {
        if (a->k_scale == nullptr || a->v_scale == nullptr) return RBA_E_INVALID;
        if (!strides_ok(a->k_scale_s, 1) || !strides_ok(a->v_scale_s, 1)) return RBA_E_INVALID;
    }
    if (a->R != nullptr) {
        if (!aligned(a->R, elem_size(a->dt))) return RBA_E_INVALID;
        if (!strides_ok(a->R_s, 1)) return RBA_E_INVALID;
    }
    if (a->lse != nullptr && !aligned(a->lse, 4)) return RBA_E_INVALID;
    return RBA_OK;
}

struct Plan {
    rba::AttnVariant var;
    int QB, nqb, N;
};

// Query-block size: all G heads of a kv head share a workgroup, so G*QB
// columns must fit the variant; QB <= 32 keeps the staged bias slab small.
Plan make_plan(const rba_attn_args *a) {
    Plan pl;
    const int G = a->Hq / a->Hkv;
    const int rows = std::max(1, std::min(a->Sq, 32));
    if (a->dt == RBA_FP32)
        pl.var = rba::AttnVariant::FP32;
    else if (G * rows > 128)
        pl.var = rba::AttnVariant::BF16_WIDE;   // two 32-column tiles per wave
    else
        pl.var = rba::AttnVariant::BF16_NARROW;
    const int maxc = rba::attn_max_columns(pl.var);
    pl.QB = std::max(1, std::min(rows, maxc / G));
    pl.nqb = a->Sq > 0 ? (a->Sq + pl.QB - 1) / pl.QB : 0;
    pl.N = a->dt == RBA_FP32 ? 32 : 64;
    return pl;
}

int tiles_last_block(const rba_attn_args *a, const Plan &pl) {
    if (a->Sq == 0) return 0;
    const int p_max = a->Skv - 1;
    const int p_min = a->Skv - a->Sq + (pl.nqb - 1) * pl.QB;
    const int lo = a->window > 0 ? std::max(0, p_min - a->window + 1) : 0;
    return p_max / pl.N - lo / pl.N + 1;
}

int heuristic_splits(const rba_attn_args *a, const Plan &pl, int num_cus) {
    const int64_t base = (int64_t)a->B * a->Hkv * pl.nqb;
    if (base <= 0) return 1;
    const int64_t target = 2 * (int64_t)num_cus;  // work items to keep every CU busy
    int64_t s = (target + base - 1) / base;
    const int n_t = tiles_last_block(a, pl);
    s = std::min<int64_t>(s, std::max(1, n_t / kMinTilesPerSplit));
    s = std::max<int64_t>(1, std::min<int64_t>(s, kMaxSplits));
    return (int)s;
}

int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

rba::AttnParams make_params(const rba_attn_args *a, const Plan &pl, int splits) {
    rba::AttnParams p{};
    p.q = a->q;
    p.k = a->k;
    p.v = a->v;
    p.R = a->R;
    p.o = a->o;
    p.lse = a->lse;
    p.qs0 = a->q_s[0], p.qs1 = a->q_s[1], p.qs2 = a->q_s[2];
    p.ks0 = a->k_s[0], p.ks1 = a->k_s[1], p.ks2 = a->k_s[2];
    p.vs0 = a->v_s[0], p.vs1 = a->v_s[1], p.vs2 = a->v_s[2];
    p.os0 = a->o_s[0], p.os1 = a->o_s[1], p.os2 = a->o_s[2];
    p.Rs0 = a->R_s[0], p.Rs1 = a->R_s[1], p.Rs2 = a->R_s[2];
    p.B = a->B, p.Sq = a->Sq, p.Skv = a->Skv, p.Hq = a->Hq, p.Hkv = a->Hkv;
    p.G = a->Hq / a->Hkv;
    p.E = a->R != nullptr ? a->E : 0;
    p.window = a->window;
    p.scale_log2e = a->scale * 1.4426950408889634f;
    p.inv_ln_base = a->log_scale_base > 0.f ? (float)(1.0 / log((double)a->log_scale_base)) : 0.f;
    p.QB = pl.QB;
    p.nqb = pl.nqb;
    p.splits = splits;
    const int64_t ch = 16 / elem_size(a->dt);
    p.r_vec = a->R != nullptr && aligned(a->R, 16) && a->E % ch == 0 && a->R_s[0] % ch == 0 &&
              a->R_s[1] % ch == 0 && a->R_s[2] % ch == 0;
    const int64_t kv_row = std::max(a->k_s[1], a->v_s[1]);
    p.kv32 = ((int64_t)a->Skv * kv_row + kHeadDim) * elem_size(a->dt) < ((int64_t)1 << 31);
    if (kv_mx(a)) {
        p.kv32 = 0;   // the MXFP8 path is the register-staged kernel
        p.qk8 = a->kv_format == RBA_KV_MXFP8_QK;
        p.k_scale = (const uint8_t *)a->k_scale;
        p.v_scale = (const uint8_t *)a->v_scale;
        p.kss0 = a->k_scale_s[0], p.kss1 = a->k_scale_s[1], p.kss2 = a->k_scale_s[2];
        p.vss0 = a->v_scale_s[0], p.vss1 = a->v_scale_s[1], p.vss2 = a->v_scale_s[2];
    }
    return p;
}

// rba_attn_prefill_fused runs the two-group bf16 prefill kernel only.
rba_status fused_supported(const rba_attn_args *a) {
    const rba_status st = validate_attn(a);
    if (st != RBA_OK) return st;
    if (a->R != nullptr || a->E < 1) return RBA_E_INVALID;
    if (a->dt != RBA_BF16 || a->kv_format != RBA_KV_PLAIN) return RBA_E_UNSUPPORTED;
    if ((int64_t)a->B * a->Sq == 0) return RBA_OK;   // nothing to do
    const Plan pl = make_plan(a);
    if (pl.var != rba::AttnVariant::BF16_WIDE) return RBA_E_UNSUPPORTED;
    const int64_t kv_row = std::max(a->k_s[1], a->v_s[1]);
    if (((int64_t)a->Skv * kv_row + kHeadDim) * elem_size(a->dt) >= ((int64_t)1 << 31)) return RBA_E_UNSUPPORTED;
    return RBA_OK;
}

size_t fused_workspace(const rba_attn_args *a, const Plan &pl, int cus) {
    const int64_t items = (int64_t)a->B * a->Hkv * pl.nqb;
    const int G = a->Hq / a->Hkv;
    const int64_t tiles = (a->E + 31) / 32;   // the region holds whole tiles of 32 distances
    return (size_t)rba::fused_grid(items, cus) * pl.QB * G * tiles * 32 * sizeof(uint16_t);
}

size_t workspace_bytes(const rba_attn_args *a, int splits) {
    if (splits <= 1) return 0;
    const size_t rows = (size_t)a->B * a->Sq * a->Hq;
    return (size_t)splits * rows * (kHeadDim + 1) * sizeof(float);
}

}  // namespace

extern "C" {

rba_status rba_relproj(rba_dtype in_dt, rba_dtype out_dt, int64_t T, int Hq, int r_dim, int E, const void *r,
                       int64_t r_stride_t, int64_t r_stride_h, const void *P, void *R, void *stream) {
    if ((in_dt != RBA_BF16 && in_dt != RBA_FP32) || (out_dt != RBA_BF16 && out_dt != RBA_FP32))
        return RBA_E_UNSUPPORTED;
    if (T < 0 || Hq < 1 || r_dim < 1 || E < 1) return RBA_E_INVALID;
    if (r_dim > 128 || Hq > 65535) return RBA_E_UNSUPPORTED;
    if (T == 0) return RBA_OK;
    if (r == nullptr || P == nullptr || R == nullptr) return RBA_E_INVALID;
    if (!aligned(r, 16) || !aligned(P, 16) || !aligned(R, 16)) return RBA_E_INVALID;
    if (r_stride_h != 0 && r_stride_h < r_dim) return RBA_E_INVALID;
    if (r_stride_t < (r_stride_h == 0 ? (int64_t)r_dim : r_stride_h * Hq)) return RBA_E_INVALID;
    const hipError_t e = rba::launch_relproj(in_dt == RBA_BF16, out_dt == RBA_BF16, T, Hq, r_dim, E, r, r_stride_t,
                                             r_stride_h, P, R, (hipStream_t)stream);
    return e == hipSuccess ? RBA_OK : RBA_E_LAUNCH;
}

rba_status rba_attn_prefill(const rba_attn_args *args, void *stream) {
    const rba_status st = validate_attn(args);
    if (st != RBA_OK) return st;
    if ((int64_t)args->B * args->Sq == 0) return RBA_OK;
    const Plan pl = make_plan(args);
    const rba::AttnParams p = make_params(args, pl, 1);
    return rba::launch_attention(p, pl.var, (hipStream_t)stream) == hipSuccess ? RBA_OK : RBA_E_LAUNCH;
}

size_t rba_relproj_packed_bytes(int Hq, int r_dim, int E) {
    if (Hq < 1 || r_dim < 1 || E < 1 || r_dim % 16 != 0 || r_dim > 128) return 0;
    return (size_t)Hq * ((E + 31) / 32) * 32 * r_dim * sizeof(uint16_t);
}

rba_status rba_relproj_pack(int Hq, int r_dim, int E, const void *P, void *PT, void *stream) {
    if (Hq < 1 || r_dim < 1 || E < 1) return RBA_E_INVALID;
    if (r_dim % 16 != 0 || r_dim > 128) return RBA_E_UNSUPPORTED;
    if (P == nullptr || PT == nullptr || !aligned(P, 16) || !aligned(PT, 16)) return RBA_E_INVALID;
    if ((int64_t)Hq > 65535) return RBA_E_UNSUPPORTED;
    return rba::launch_relproj_pack(Hq, r_dim, E, P, PT, (hipStream_t)stream) == hipSuccess ? RBA_OK
                                                                                             : RBA_E_LAUNCH;
}

size_t rba_prefill_fused_workspace_bytes(const rba_attn_args *args) {
    if (fused_supported(args) != RBA_OK) return 0;
    const int cus = device_cus();
    if (cus <= 0) return 0;
    return fused_workspace(args, make_plan(args), cus);
}

rba_status rba_attn_prefill_fused(const rba_attn_args *args, const rba_relbias *rb, void *workspace,
                                  size_t workspace_bytes_, void *stream) {
    rba_status st = fused_supported(args);
    if (st != RBA_OK) return st;
    if (rb == nullptr) return RBA_E_INVALID;
    if (rb->r_dim < 1) return RBA_E_INVALID;
    if (rb->r_dim % 16 != 0 || rb->r_dim > 128) return RBA_E_UNSUPPORTED;
    if ((int64_t)args->B * args->Sq == 0) return RBA_OK;
    if (rb->r == nullptr || rb->PT == nullptr || !aligned(rb->r, 16) || !aligned(rb->PT, 16)) return RBA_E_INVALID;
    if (!strides_ok(rb->r_s, 8)) return RBA_E_INVALID;
    if (rb->r_s[2] != 0 && rb->r_s[2] < rb->r_dim) return RBA_E_INVALID;
    // no workspace: the logits of each banded key tile are computed into LDS
    // (features of at most 64 channels)
    const bool on_chip = workspace == nullptr;
    if (on_chip && rb->r_dim > 64) return RBA_E_WORKSPACE;
    const int cus = device_cus();
    if (cus <= 0) return RBA_E_LAUNCH;
    const Plan pl = make_plan(args);
    const size_t need = fused_workspace(args, pl, cus);
    if (!on_chip && (workspace_bytes_ < need || !aligned(workspace, 16))) return RBA_E_WORKSPACE;
    rba::AttnParams p = make_params(args, pl, 1);
    p.E = args->E;
    p.rf = rb->r;
    p.rfs0 = rb->r_s[0], p.rfs1 = rb->r_s[1], p.rfs2 = rb->r_s[2];
    p.r_dim = rb->r_dim;
    p.PT = rb->PT;
    p.bias_ws = workspace;
    const int64_t items = (int64_t)args->B * args->Hkv * pl.nqb;
    return rba::launch_attention_fused(p, rba::fused_grid(items, cus), (hipStream_t)stream) == hipSuccess
               ? RBA_OK
               : RBA_E_LAUNCH;
}

int rba_num_splits(const rba_attn_args *args, int num_cus) {
    if (validate_attn(args) != RBA_OK) return 0;
    if (num_cus <= 0) num_cus = device_cus();
    if (num_cus <= 0) return 0;
    const Plan pl = make_plan(args);
    return heuristic_splits(args, pl, num_cus);
}

size_t rba_decode_workspace_bytes(const rba_attn_args *args, int num_splits) {
    if (validate_attn(args) != RBA_OK || num_splits < 0 || num_splits > kMaxSplits) return 0;
    if (num_splits == 0) num_splits = rba_num_splits(args, 0);
    return workspace_bytes(args, num_splits);
}

// Shared by rba_attn_decode and rba_attn_decode_noalloc.  scratch: take the
// workspace from the library's device scratch array instead of the caller.
static rba_status decode_impl(const rba_attn_args *args, int num_splits, void *workspace, size_t workspace_bytes_,
                              bool scratch, void *stream) {
    const rba_status st = validate_attn(args);
    if (st != RBA_OK) return st;
    if (num_splits < 0 || num_splits > kMaxSplits) return RBA_E_INVALID;
    if ((int64_t)args->B * args->Sq == 0) return RBA_OK;
    const Plan pl = make_plan(args);
    if (num_splits == 0) {
        const int cus = device_cus();
        if (cus <= 0) return RBA_E_LAUNCH;
        num_splits = heuristic_splits(args, pl, cus);
    }
    hipStream_t s = (hipStream_t)stream;
    if (num_splits == 1) {
        const rba::AttnParams p = make_params(args, pl, 1);
        return rba::launch_attention(p, pl.var, s) == hipSuccess ? RBA_OK : RBA_E_LAUNCH;
    }
    const size_t need = workspace_bytes(args, num_splits);
    if (scratch) {
        if (need > RBA_DECODE_SCRATCH_BYTES) return RBA_E_WORKSPACE;
        if (rba::scratch_address(&workspace) != hipSuccess) return RBA_E_LAUNCH;
        workspace_bytes_ = RBA_DECODE_SCRATCH_BYTES;
    }
    if (workspace == nullptr || workspace_bytes_ < need || !aligned(workspace, 16)) return RBA_E_WORKSPACE;
    rba::AttnParams p = make_params(args, pl, num_splits);
    const size_t rows = (size_t)args->B * args->Sq * args->Hq;
    p.o_part = (float *)workspace;
    p.lse_part = p.o_part + (size_t)num_splits * rows * kHeadDim;
    if (rba::launch_attention(p, pl.var, s) != hipSuccess) return RBA_E_LAUNCH;
    return rba_splitkv_combine(p.o_part, p.lse_part, num_splits, args, stream);
}

rba_status rba_attn_decode(const rba_attn_args *args, int num_splits, void *workspace, size_t workspace_bytes_,
                           void *stream) {
    return decode_impl(args, num_splits, workspace, workspace_bytes_, false, stream);
}

rba_status rba_attn_decode_noalloc(const rba_attn_args *args, int num_splits, void *stream) {
    return decode_impl(args, num_splits, nullptr, 0, true, stream);
}

rba_status rba_attn_paged(const rba_attn_args *args, const rba_paged_kv *kv, int num_splits, void *workspace,
                          size_t workspace_bytes_, void *stream) {
    const rba_status st = validate_attn(args);
    if (st != RBA_OK) return st;
    if (kv == nullptr) return RBA_E_INVALID;
    if (num_splits < 0 || num_splits > kMaxSplits) return RBA_E_INVALID;
    if (kv->page_size < kPageQuantum || kv->page_size % kPageQuantum != 0 || kv->num_pages < 1)
        return RBA_E_INVALID;
    if (kv->bt_stride < ((int64_t)args->Skv + kv->page_size - 1) / kv->page_size) return RBA_E_INVALID;
    if ((int64_t)args->B * args->Sq == 0) return RBA_OK;
    if (kv->block_table == nullptr || kv->seq_lens == nullptr || !aligned(kv->block_table, 4) ||
        !aligned(kv->seq_lens, 4))
        return RBA_E_INVALID;
    // one page of K or V must lie within a 32-bit buffer range
    const int64_t kv_row = std::max(args->k_s[1], args->v_s[1]);
    if (((int64_t)(kv->page_size - 1) * kv_row + kHeadDim) * kv_elem_size(args) >= ((int64_t)1 << 31))
        return RBA_E_UNSUPPORTED;
    const Plan pl = make_plan(args);
    if (num_splits == 0) {
        const int cus = device_cus();
        if (cus <= 0) return RBA_E_LAUNCH;
        num_splits = heuristic_splits(args, pl, cus);
    }
    rba::AttnParams p = make_params(args, pl, num_splits);
    p.kv32 = 0;
    p.block_table = kv->block_table;
    p.seq_lens = kv->seq_lens;
    p.bt_stride = kv->bt_stride;
    p.page_size = kv->page_size;
    p.num_pages = kv->num_pages;
    hipStream_t s = (hipStream_t)stream;
    if (num_splits == 1) return rba::launch_attention(p, pl.var, s) == hipSuccess ? RBA_OK : RBA_E_LAUNCH;
    const size_t need = workspace_bytes(args, num_splits);
    if (workspace == nullptr || workspace_bytes_ < need || !aligned(workspace, 16)) return RBA_E_WORKSPACE;
    const size_t rows = (size_t)args->B * args->Sq * args->Hq;
    p.o_part = (float *)workspace;
    p.lse_part = p.o_part + (size_t)num_splits * rows * kHeadDim;
    if (rba::launch_attention(p, pl.var, s) != hipSuccess) return RBA_E_LAUNCH;
    return rba_splitkv_combine(p.o_part, p.lse_part, num_splits, args, stream);
}

rba_status rba_attn_prologue(const rba_prologue_args *a, const rba_attn_args *c, const rba_paged_kv *kv,
                             void *stream) {
    if (a == nullptr || c == nullptr) return RBA_E_INVALID;
    if (c->dt != RBA_BF16) return RBA_E_UNSUPPORTED;
    if (c->kv_format != RBA_KV_PLAIN && !kv_mx(c)) return RBA_E_INVALID;
    if (a->d != kHeadDim || c->d != kHeadDim) return a->d <= 0 ? RBA_E_INVALID : RBA_E_UNSUPPORTED;
    if (a->B < 0 || a->T < 0 || a->Hq < 1 || a->Hkv < 1 || a->Hkv != c->Hkv || c->Skv < 1) return RBA_E_INVALID;
    if (a->conv_w < 1 || a->conv_w > kMaxConvTaps) return RBA_E_INVALID;
    if (!isfinite(a->eps) || !(a->eps > 0.f)) return RBA_E_INVALID;
    if (a->max_new < 0) return RBA_E_INVALID;
    if (a->T == 0) return RBA_OK;
    if (a->B < 1) return RBA_E_INVALID;
    if (a->cu_new == nullptr || a->seq_lens == nullptr || a->q == nullptr || a->k == nullptr || a->v == nullptr ||
        a->conv_wk == nullptr || a->conv_wv == nullptr || a->norm_q == nullptr || a->norm_k == nullptr ||
        a->q_out == nullptr || c->k == nullptr || c->v == nullptr)
        return RBA_E_INVALID;
    if (a->conv_w > 1 && (a->state_k == nullptr || a->state_v == nullptr)) return RBA_E_INVALID;
    // 8-byte pieces of bf16 rows
    auto rows_ok = [](const void *p, const int64_t *s, int n) {
        if (!aligned(p, 8)) return false;
        for (int i = 0; i < n; ++i)
            if (s[i] < 0 || s[i] % 4 != 0) return false;
        return true;
    };
    if (!rows_ok(a->q, a->q_s, 2) || !rows_ok(a->k, a->k_s, 2) || !rows_ok(a->v, a->v_s, 2) ||
        !rows_ok(a->q_out, a->q_out_s, 2) || !rows_ok(c->k, c->k_s, 3) || !rows_ok(c->v, c->v_s, 3))
        return RBA_E_INVALID;
    if (a->conv_w > 1 && (!aligned(a->state_k, 8) || !aligned(a->state_v, 8))) return RBA_E_INVALID;
    if (!aligned(a->cu_new, 4) || !aligned(a->seq_lens, 4) || !aligned(a->conv_wk, 4) || !aligned(a->conv_wv, 4) ||
        !aligned(a->norm_q, 4) || !aligned(a->norm_k, 4))
        return RBA_E_INVALID;
    const bool f8 = kv_mx(c);
    if (f8 && (c->k_scale == nullptr || c->v_scale == nullptr || !strides_ok(c->k_scale_s, 1) ||
               !strides_ok(c->v_scale_s, 1)))
        return RBA_E_INVALID;
    if (kv != nullptr) {
        if (kv->page_size < kPageQuantum || kv->page_size % kPageQuantum != 0 || kv->num_pages < 1)
            return RBA_E_INVALID;
        if (kv->bt_stride < ((int64_t)c->Skv + kv->page_size - 1) / kv->page_size) return RBA_E_INVALID;
        if (kv->block_table == nullptr || !aligned(kv->block_table, 4)) return RBA_E_INVALID;
    }
    rba::PrologueParams p{};
    p.B = a->B, p.T = a->T, p.Hq = a->Hq, p.Hkv = a->Hkv, p.W = a->conv_w, p.Skv = c->Skv;
    p.eps = a->eps;
    p.max_new = a->max_new;
    p.cu_new = a->cu_new, p.seq_lens = a->seq_lens;
    p.q = (const __bf16 *)a->q, p.k = (const __bf16 *)a->k, p.v = (const __bf16 *)a->v;
    p.qs0 = a->q_s[0], p.qs1 = a->q_s[1], p.ks0 = a->k_s[0], p.ks1 = a->k_s[1];
    p.vs0 = a->v_s[0], p.vs1 = a->v_s[1], p.qos0 = a->q_out_s[0], p.qos1 = a->q_out_s[1];
    p.conv_wk = a->conv_wk, p.conv_wv = a->conv_wv, p.norm_q = a->norm_q, p.norm_k = a->norm_k;
    p.state_k = (__bf16 *)a->state_k, p.state_v = (__bf16 *)a->state_v, p.q_out = (__bf16 *)a->q_out;
    p.k_cache = const_cast<void *>(c->k), p.v_cache = const_cast<void *>(c->v);
    p.cks0 = c->k_s[0], p.cks1 = c->k_s[1], p.cks2 = c->k_s[2];
    p.cvs0 = c->v_s[0], p.cvs1 = c->v_s[1], p.cvs2 = c->v_s[2];
    if (f8) {
        p.k_scale = (uint8_t *)const_cast<void *>(c->k_scale);
        p.v_scale = (uint8_t *)const_cast<void *>(c->v_scale);
        p.sks0 = c->k_scale_s[0], p.sks1 = c->k_scale_s[1], p.sks2 = c->k_scale_s[2];
        p.svs0 = c->v_scale_s[0], p.svs1 = c->v_scale_s[1], p.svs2 = c->v_scale_s[2];
    }
    if (kv != nullptr) {
        p.block_table = kv->block_table, p.bt_stride = kv->bt_stride;
        p.page_size = kv->page_size, p.num_pages = kv->num_pages;
    }
    return rba::launch_prologue(p, (hipStream_t)stream) == hipSuccess ? RBA_OK : RBA_E_LAUNCH;
}

rba_status rba_splitkv_combine(const float *o_part, const float *lse_part, int num_splits,
                               const rba_attn_args *args, void *stream) {
    const rba_status st = validate_attn(args);
    if (st != RBA_OK) return st;
    if (num_splits < 1 || num_splits > kMaxSplits) return RBA_E_INVALID;
    if ((int64_t)args->B * args->Sq == 0) return RBA_OK;
    if (o_part == nullptr || lse_part == nullptr || !aligned(o_part, 16) || !aligned(lse_part, 4))
        return RBA_E_INVALID;
    const hipError_t e =
        rba::launch_combine(o_part, lse_part, num_splits, args->B, args->Sq, args->Hq, args->o, args->dt == RBA_BF16,
                            args->o_s[0], args->o_s[1], args->o_s[2], args->lse, (hipStream_t)stream);
    return e == hipSuccess ? RBA_OK : RBA_E_LAUNCH;
}

rba_status rba_mxfp8_quantize(rba_dtype in_dt, int64_t rows, int n, const void *x, int64_t x_stride, void *codes,
                              int64_t codes_stride, void *scales, int64_t scales_stride, void *stream) {
    if (in_dt != RBA_BF16 && in_dt != RBA_FP32) return RBA_E_UNSUPPORTED;
    if (rows < 0 || n < 32 || n % 32 != 0 || n > 65536) return RBA_E_INVALID;
    if (rows == 0) return RBA_OK;
    if (x == nullptr || codes == nullptr || scales == nullptr) return RBA_E_INVALID;
    const int es = elem_size(in_dt);
    if (!aligned(x, 16) || (x_stride * es) % 16 != 0 || x_stride < n) return RBA_E_INVALID;
    if (!aligned(codes, 4) || codes_stride % 4 != 0 || codes_stride < n) return RBA_E_INVALID;
    if (scales_stride < n / 32) return RBA_E_INVALID;
    const hipError_t e = rba::launch_mxfp8_quantize(in_dt == RBA_BF16, rows, n, x, x_stride, codes, codes_stride,
                                                    scales, scales_stride, (hipStream_t)stream);
    return e == hipSuccess ? RBA_OK : RBA_E_LAUNCH;
}

rba_status rba_calib_read(const void *buf, size_t bytes, void *sink, void *stream) {
    if (bytes == 0) return RBA_OK;
    if (buf == nullptr || sink == nullptr || !aligned(buf, 16) || !aligned(sink, 4)) return RBA_E_INVALID;
    if (bytes % kCalibReadQuantum != 0 || bytes > ((size_t)1 << 40)) return RBA_E_INVALID;
    const int cus = device_cus();
    if (cus <= 0) return RBA_E_LAUNCH;
    return rba::launch_calib_read(buf, (int64_t)bytes, sink, 2 * cus, (hipStream_t)stream) == hipSuccess
               ? RBA_OK
               : RBA_E_LAUNCH;
}

rba_status rba_calib_mfma(int iters, void *sink, double *flops, void *stream) {
    if (iters < 1 || sink == nullptr || !aligned(sink, 4)) return RBA_E_INVALID;
    const int cus = device_cus();
    if (cus <= 0) return RBA_E_LAUNCH;
    const int blocks = 8 * cus;   // 32 waves per CU: eight per SIMD
    if (flops != nullptr) *flops = (double)blocks * 4 /*waves*/ * iters * 4 /*MFMAs*/ * (2.0 * 32 * 32 * 16);
    return rba::launch_calib_mfma(iters, blocks, sink, (hipStream_t)stream) == hipSuccess ? RBA_OK : RBA_E_LAUNCH;
}

const char *rba_status_string(rba_status status) {
    switch (status) {
        case RBA_OK: return "ok";
        case RBA_E_INVALID: return "invalid argument";
        case RBA_E_UNSUPPORTED: return "unsupported shape or dtype";
        case RBA_E_WORKSPACE: return "workspace missing or too small";
        case RBA_E_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

int rba_version(void) { return 200; }

}  // extern "C"
