// Relative-position-bias attention forward for gfx950 (MI355X).
//
// Computes, per batch b, query head h (kv head g = h / G) and query row t at
// position p = Skv - Sq + t:
//     s(t, j) = f(p) * (scale * q.k_j + [p - j < E] R[b,t,h,p-j]),  j visible
// followed by a softmax over the visible keys and the weighted sum of v
// ("SGLang と Miles が Inkling を初日からサポート", section
// "相対位置バイアス付き Attention"; GQA with head size 128 from "vLLM TML
// Inkling サポート", section "TML Inkling モデルアーキテクチャ").
//
// Two kernels share the arithmetic below: attn_fwd_kernel (split-KV decode,
// paged and MXFP8 K/V, narrow and fp32 shapes) and attn_prefill_pp_kernel
// (bf16 prefill: two groups of four waves alternate between matrix and vector
// phases, one persistent workgroup per CU; its FK > 0 instances compute the
// block's rows of R themselves from r and the packed projection).
//
// Design:
//  * A workgroup of NW waves owns one (batch, kv head, block of QB query rows,
//    key-range split) and all G query heads of that kv head.  Its G*QB query
//    columns form 32-column tiles, one per wave, and all of them read the K/V
//    tiles staged in LDS once (the GQA group loop).
//  * Scores are computed transposed, S^T = K . Q^T, with
//    v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator a lane owns one query
//    column and 16 of the 32 keys; the A-operand rows are permuted so those 16
//    keys are consecutive.  Row max/sum need one cross-half exchange, the bias
//    for 16 consecutive keys is 16 consecutive (reversed) entries of one R row,
//    and the probabilities feed the PV product (O^T = V^T . P^T) as the
//    B operand straight from registers.
//  * K tiles and, for key tiles whose smallest distance is below E, the R rows
//    of the block's columns (the entries that tile can touch) are copied
//    global -> LDS with direct-to-LDS loads, double-buffered: tile kt+1 streams
//    in while tile kt is computed.  V goes through registers because it is
//    stored transposed.  Each lane gathers its bias by diagonal offset p - j.
//  * Tiles outside the causal/window band are never visited, interior tiles
//    skip the mask, tiles past the extent skip the bias.
//  * Online softmax in the exp2 domain with fp32 state.  The reference max is
//    only raised when a tile exceeds it by more than 2^8, so O is rarely
//    rescaled.  bf16 P feeds PV.
//  * Work items are ordered longest-first and laid out so that each of the 8
//    XCDs processes contiguous (batch, kv head) ranges, keeping their K/V in
//    that XCD's L2.
#include "rba_internal.h"

#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

namespace rba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int D = 128;                // head size
constexpr int NT = 256;               // threads per workgroup of the combine kernel
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;  // log2 growth of the running max tolerated before O is rescaled
constexpr float kRescaleLimit = 256.f;   // 2^kRescaleSlack
constexpr int kPrioPeriod = 16;          // decode: key tiles per wave-priority phase

template <typename T>
struct Tile;

// bf16: 64-key tiles; V stored transposed so PV A-operands are 16-byte reads.
template <>
struct Tile<__bf16> {
    static constexpr int N = 64;              // keys per tile
    static constexpr int CH = 8;              // elements per 16-byte chunk
    static constexpr int VROWS = D;           // V^T rows (head dim)
    static constexpr int VS = N + 8;          // V^T row stride: 36 dwords
    static constexpr int SW = N + CH;         // slab row: the N entries a row needs, chunk-aligned
};

// fp32: 32-key tiles; V kept row-major (fp32 MFMA takes one element per lane).
template <>
struct Tile<float> {
    static constexpr int N = 32;
    static constexpr int CH = 4;
    static constexpr int VROWS = 32;
    static constexpr int VS = D + 4;
    static constexpr int SW = N + CH;
};

// A-operand row i of a 32x32 MFMA -> key offset inside a 32-key sub-tile.  With
// this order the accumulator register r of lane half hh holds key 16*hh + r.
__device__ __forceinline__ int mfma_row_key(int i) { return ((i >> 2) & 1) * 16 + (i >> 3) * 4 + (i & 3); }

// LDS row of key j inside a K tile (an involution).  K rows are padded by one
// 16-byte chunk, so row R starts at bank 4R mod 64; the permutation gives the
// 16 rows of one A-operand read pass distinct R mod 16.
__device__ __forceinline__ int lds_key_row(int j) { return j ^ (((j >> 4) & 1) * 12); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier after this wave's LDS accesses have completed.  The
// compiler-level memory fences keep LDS accesses from moving across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;   // raw buffer, 32-bit data format

// Buffer descriptor over [base, base + bytes).  Loads at offsets >= bytes
// return zero (the hardware range check), which pads K/V rows past the
// sequence end and R chunks outside a block.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0xffffffffll ? 0xffffffffll : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)(unsigned)n, kRsrcFlags);
}

// One 16-byte buffer -> LDS load per lane: lane i of the wave writes bytes
// [16 i, 16 i + 16) after the wave-uniform LDS address `lds_wave`.
__device__ __forceinline__ void dma16(rsrc_t r, unsigned voff, void *lds_wave) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_wave, 16, voff, 0, 0,
                                             0);
}

// Maximum of a lane's value and that of lane ^ 32, without the LDS pipeline:
// v_permlane32_swap exchanges the upper 32 lanes of one register with the
// lower 32 lanes of the other, so with both holding x every lane ends up
// with its own value in one register and its partner's in the other.
__device__ __forceinline__ float max_across_halves(float x) {
    float a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return fmaxf(a, b);
}

// A wave-uniform 32-bit read through the scalar data cache (a read-only
// use of that cache: the kernel never writes the table it reads).
__device__ __forceinline__ int load_scalar(const int *ptr) {
    return *(const __attribute__((address_space(4))) int *)ptr;
}

// Buffer descriptor words for dma16_untracked (same layout as make_rsrc).
__device__ __forceinline__ u32x4 make_rsrc_words(const void *base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0xffffffffll ? 0xffffffffll : bytes);
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return u32x4{(unsigned)a, (unsigned)(a >> 32) & 0xffffu, (unsigned)n, (unsigned)kRsrcFlags};
}

// dma16 written as inline assembly.  The compiler does not see this load, so
// it never makes later LDS reads wait for it (it cannot tell which LDS bytes
// a direct-to-LDS load writes and would otherwise wait for all of them);
// the caller waits (vmcnt(0)) before the barrier that hands the data over.
// The LDS address is an operand bound to m0, so the compiler writes m0 itself
// (m0 is reserved to it: the assembly must not write it); the s_nop is the
// wait state an LDS DMA needs after an m0 write.
__device__ __forceinline__ void dma16_untracked(u32x4 rsrc, unsigned voff, const void *lds_wave) {
    const unsigned m0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void *)lds_wave;
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(m0)
                 : "memory");
}

// E8M0 scale code -> its power of two (code 0 is 2^-127, an fp32 subnormal).
__device__ __forceinline__ float e8m0_scale(unsigned code) {
    return __builtin_bit_cast(float, code == 0 ? 0x00400000u : code << 23);
}

// Four OCP E4M3 codes (bytes of w, lowest first) times 2^scale -> four bf16
// in two dwords, lowest element in the low half.  Exact: an E4M3 value times
// a power of two fits bf16 unless it leaves bf16's exponent range.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(unsigned w, float sc) {
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, true);
    return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// PG: K and V live in a pool of fixed-size pages; key tile kt of sequence b
// is read from page block_table[b][kt * N / page_size] (a page holds whole
// tiles), and sequence b has its own length seq_lens[b].
// F8: K and V are MXFP8 (E4M3 codes, one E8M0 scale per 32 head-dim entries);
// both go through registers, are decoded to bf16 exactly and stored in the
// same LDS layouts as bf16 K and V, so the compute is the bf16 one.
// FQ (with F8): the logits run in MXFP8 too.  q is encoded once with the
// cache's rule (blocks of 32 along d), K stays as codes and scales in LDS,
// and S^T = K . Q^T runs on v_mfma_scale_f32_32x32x64_f8f6f4, which applies
// the E8M0 scales of both operands itself; V is decoded for PV as with F8.
// VD (4 waves, at most 96 query columns): K and V in two buffers each beside
// a 96-row bias slab, one barrier per tile.  bf16: V goes global -> LDS by
// direct-to-LDS loads like K, row-major, and is read transposed.  MXFP8
// cache (bf16 logits): the last wave, which has no columns, loads and decodes
// the next tile's K and V while the others compute.
template <typename T, int NW, bool SLAB2, bool PG, bool F8, bool FQ = false, bool VD = false>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_fwd_kernel(const AttnParams p) {
    using TL = Tile<T>;
    constexpr bool BF = sizeof(T) == 2;
    static_assert(!F8 || BF, "MXFP8 K/V is decoded to bf16");
    static_assert(!FQ || F8, "MXFP8 logits need an MXFP8 cache");
    static_assert(!VD || (BF && !FQ && NW == 4 && !SLAB2), "VD is the 4-wave decode of bf16 or MXFP8 K/V");
    constexpr int ES = (int)sizeof(T);
    constexpr int KES = F8 ? 1 : ES;             // bytes per K/V element in memory
    constexpr int NTH = 64 * NW;                 // threads per workgroup
    constexpr int N = TL::N;
    constexpr int KT = N / 32;                   // 32-key sub-tiles per tile
    constexpr int CH = TL::CH;
    constexpr int VS = TL::VS;
    constexpr int SW = TL::SW;
    constexpr int NCH = SW / CH;                 // chunks per slab row
    constexpr int SROWS = VD ? 96 : NW * 32;     // slab rows = max columns per workgroup
    constexpr int SCH = SROWS * NCH;             // slab chunks
    constexpr int NSI = (SCH + NTH - 1) / NTH;   // slab DMA instructions per thread
    constexpr int CPR = D * ES / 16;             // 16-byte chunks per K/V row
    constexpr int CPRP = CPR + 1;                // with the padding chunk
    constexpr int KS = CPRP * CH;                // K row stride in LDS (elements)
    constexpr int KCH = N * CPRP;                // K chunks per tile incl. padding
    constexpr int NKI = (KCH + NTH - 1) / NTH;   // K DMA instructions per thread
    constexpr int NVI = BF ? N * D / (NTH * 4) : N * CPR / NTH;  // V loads per thread
    static_assert(NVI * NTH * (BF ? 4 : CH) == N * D, "V tile must split evenly over threads");

    // FQ: K stays MXFP8 in LDS: row r of codes at byte K8R * r (DMA chunk
    // 8 of a row repeats chunk 0), the four scale bytes of row r at K8S + 4 r.
    constexpr int K8R = D + 16;                 // padded code row (bytes)
    constexpr int K8S = N * K8R;
    // FQ2 (MXFP8 logits, 4 waves): K codes and decoded V in two buffers each,
    // one bias buffer; the next tile's V is decoded right after this tile's
    // compute, so a tile takes one barrier.
    constexpr bool FQ2 = FQ && NW == 4;
    // F8 otherwise: one K and one V buffer (registers carry the tiles in
    // flight).  V is row-major with 16-byte chunks XOR-swizzled by row and
    // read transposed.
    constexpr int NKB = F8 ? ((FQ2 || VD) ? 2 : 1) : 2;
    constexpr int KBE = FQ2 ? (K8S + 4 * N) / (int)sizeof(T) : N * KS;   // elements of one K buffer
    constexpr int NVB = (FQ2 || VD) ? 2 : 1;
    constexpr int VSZ = (F8 || VD) ? N * D : TL::VROWS * VS;
    constexpr int NSB = (FQ2 || VD) ? 1 : ((SLAB2 || F8) ? 2 : 1);
    __shared__ __attribute__((aligned(16))) T sK[NKB][KBE];
    __shared__ __attribute__((aligned(16))) T sV[NVB * VSZ];
    __shared__ __attribute__((aligned(16))) T sR[NSB][SROWS * SW];
    static_assert(!FQ || K8S + 4 * N <= KBE * (int)sizeof(T), "K codes and scales fit a K buffer");
    constexpr int KBB = KBE * (int)sizeof(T);   // bytes of one K buffer
    unsigned char *const sK8 = (unsigned char *)&sK[0][0];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int hh = lane >> 5;     // lane half
    const int lc = lane & 31;     // lane column

    // ------------------------------------------------------------ work item
    const int per_bh = p.nqb * p.splits;
    const int total = p.B * p.Hkv * per_bh;
    int item = blockIdx.x;
    if ((total & 7) == 0) item = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    const int bh = item / per_bh;
    const int rem = item - bh * per_bh;
    const int qb = p.nqb - 1 - rem / p.splits;   // longest blocks first
    const int sp = rem % p.splits;
    const int b = bh / p.Hkv;
    const int hkv = bh - b * p.Hkv;
    const int t0 = qb * p.QB;
    const int nrows = min(p.QB, p.Sq - t0);
    // keys of this sequence; a paged length outside [Sq, Skv] is clamped
    const int Skv = PG ? min(max(p.seq_lens[b], p.Sq), p.Skv) : p.Skv;
    const int pos0 = Skv - p.Sq;
    const int p_min = pos0 + t0;
    const int p_max = p_min + nrows - 1;
    const int W = p.window;
    const int lo_key = W > 0 ? max(0, p_min - W + 1) : 0;
    const int kt_lo = lo_key / N;
    const int n_t = p_max / N - kt_lo + 1;
    const int kb = kt_lo + (int)((int64_t)sp * n_t / p.splits);
    const int ke = kt_lo + (int)((int64_t)(sp + 1) * n_t / p.splits);
    const int ncols = p.G * p.QB;
    const bool has_bias = p.R != nullptr && p.E > 0;

    // byte addresses of this (batch, kv head)'s K/V rows; paged: the page
    // offset is added per tile
    const char *__restrict__ gk = (const char *)p.k + ((PG ? 0 : (int64_t)b * p.ks0) + (int64_t)hkv * p.ks2) * KES;
    const char *__restrict__ gv = (const char *)p.v + ((PG ? 0 : (int64_t)b * p.vs0) + (int64_t)hkv * p.vs2) * KES;
    const char *__restrict__ gks = F8 ? (const char *)p.k_scale + (PG ? 0 : (int64_t)b * p.kss0) + (int64_t)hkv * p.kss2
                                      : nullptr;
    const char *__restrict__ gvs = F8 ? (const char *)p.v_scale + (PG ? 0 : (int64_t)b * p.vss0) + (int64_t)hkv * p.vss2
                                      : nullptr;

    // ------------------------------------------------------------ this lane's query column
    const int col = wave * 32 + lc;
    const int hl = col / p.QB;
    const int qi = col - hl * p.QB;
    const bool cvalid = col < ncols && qi < nrows;
    const int tq = t0 + qi;
    const int hq = hkv * p.G + min(hl, p.G - 1);
    const int prow = p_min + qi;
    // log-scale factor; kept > 0 (row p = 0 has one visible key, so its
    // output does not depend on the factor) so that masked -inf logits stay
    // -inf through the scale.
    const float fls = p.inv_ln_base > 0.f ? fmaxf(logf((float)prow + 1.f) * p.inv_ln_base, 1e-30f) : 1.f;
    const float amul = p.scale_log2e * fls;     // > 0
    const float bmul = kLog2e * fls;
    const bool wave_active = wave * 32 < ncols;
    // This column's slab row holds R entries [rb - j0, rb - j0 + SW) for key
    // tile j0: the N distances p - j of the tile, from a chunk boundary.
    const int rb = (prow - N + 1) & ~(CH - 1);

    // Q fragment (B operand of S^T = K Q^T), loaded once.
    constexpr int QREGS = FQ ? 1 : (BF ? 8 : 64);
    typedef typename std::conditional<BF, bf16x8, float>::type QFrag;
    QFrag qf[QREGS];
    {
        const T *qp = (const T *)p.q + (int64_t)b * p.qs0 + (int64_t)tq * p.qs1 + (int64_t)hq * p.qs2;
        if constexpr (FQ) {
            qf[0] = bf16x8{};
        } else if constexpr (BF) {
#pragma unroll
            for (int k = 0; k < 8; ++k) qf[k] = cvalid ? *(const bf16x8 *)(qp + 16 * k + 8 * hh) : bf16x8{};
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const f32x4 x = cvalid ? *(const f32x4 *)(qp + 64 * hh + 4 * k) : f32x4{};
                qf[4 * k + 0] = x[0];
                qf[4 * k + 1] = x[1];
                qf[4 * k + 2] = x[2];
                qf[4 * k + 3] = x[3];
            }
        }
        // Settle the loads here.  vmcnt counts in order, so a wait for them
        // left inside the tile loop would also wait for the next tile's V loads
        // (the wait there is then for the K tile only, the one the compiler
        // keeps ahead of the LDS reads).
#pragma unroll
        for (int k = 0; k < QREGS; ++k) asm volatile("" : "+v"(qf[k]));
    }
    // FQ: q encoded to MXFP8 as the B operand of the scaled MFMA.  For k-step
    // ks (64 head-dim entries), lane (column, half hh) holds the codes of
    // entries 64ks + 16hh + [0, 16) in bytes 0-15 and 64ks + 32 + 16hh +
    // [0, 16) in bytes 16-31; the instruction takes the scale of the block of
    // bytes 0-15 (entries 64ks .. 64ks+31) from the lower-half lane and that
    // of bytes 16-31 from the upper-half lane (lane layout checked on the
    // device).  So each block of 32 is split over the two halves of a
    // column, which exchange their maxima; encoding as the cache encoder
    // does: exponent floor(log2 max) - 8 clamped to [-127, 127] (-127 for a
    // zero block), exact scaling, saturation to 448, hardware RNE conversion.
    i32x8 q8[FQ ? 2 : 1] = {};
    int qsc[FQ ? 2 : 1] = {};
    if constexpr (FQ) {
        const T *qp = (const T *)p.q + (int64_t)b * p.qs0 + (int64_t)tq * p.qs1 + (int64_t)hq * p.qs2;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const int d0 = 32 * blk + 16 * hh;
            const bf16x8 x0 = cvalid ? *(const bf16x8 *)(qp + d0) : bf16x8{};
            const bf16x8 x1 = cvalid ? *(const bf16x8 *)(qp + d0 + 8) : bf16x8{};
            float v[16];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v[i] = (float)x0[i];
                v[8 + i] = (float)x1[i];
            }
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            int e = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 1 - 8 : -127;
            e = min(max(e, -127), 127);
            int w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float s0 = fminf(fmaxf(ldexpf(v[4 * i], -e), -448.f), 448.f);
                const float s1 = fminf(fmaxf(ldexpf(v[4 * i + 1], -e), -448.f), 448.f);
                const float s2 = fminf(fmaxf(ldexpf(v[4 * i + 2], -e), -448.f), 448.f);
                const float s3 = fminf(fmaxf(ldexpf(v[4 * i + 3], -e), -448.f), 448.f);
                w[i] = __builtin_amdgcn_cvt_pk_fp8_f32(s2, s3, __builtin_amdgcn_cvt_pk_fp8_f32(s0, s1, 0, false), true);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) q8[blk >> 1][4 * (blk & 1) + i] = w[i];
            qsc[blk >> 1] = (blk & 1) == hh ? e + 127 : qsc[blk >> 1];
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) asm volatile("" : "+v"(q8[ks]), "+v"(qsc[ks]));
    }

    f32x16 O[4];
    float m = -INFINITY, l = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) O[dt] = f32x16{};

    // ------------------------------------------------------------ staging offsets (per lane, fixed)
    // K: LDS chunk L of a tile holds chunk pc of LDS row L / CPRP, i.e. key
    // row lds_key_row(L / CPRP); the padding chunk reloads chunk 0.
    unsigned kvo[NKI];
#pragma unroll
    for (int i = 0; i < NKI; ++i) {
        const int L = (i * NW + wave) * 64 + lane;
        const int R = L / CPRP, pc = L - R * CPRP;
        kvo[i] = (unsigned)(((int64_t)lds_key_row(R) * p.ks1 + (pc < CPR ? pc : 0) * CH) * ES);
    }
    // V: bf16 lanes load 4 head-dim entries of NVI consecutive keys and store
    // them transposed; fp32 lanes copy 16-byte chunks row-major.
    constexpr int NKQ = BF ? N / NVI : 1;        // key groups (bf16)
    const int v_kq = (tid >> 2) & (NKQ - 1);
    const int v_dq = (tid & 3) | ((tid / (4 * NKQ)) << 2);
    unsigned vvo[F8 ? 1 : NVI];
#pragma unroll
    for (int i = 0; i < (F8 ? 0 : NVI); ++i) {
        if constexpr (BF) {
            vvo[i] = (unsigned)(((int64_t)(NVI * v_kq + i) * p.vs1 + 4 * v_dq) * ES);
        } else {
            const int ci = tid + NTH * i;
            const int row = ci / CPR, cc = ci - row * CPR;
            vvo[i] = (unsigned)(((int64_t)row * p.vs1 + cc * CH) * ES);
        }
    }
    // Slab: chunk L is chunk L % NCH of row L / NCH (a query column, at
    // position p_min + its row index within its head); -j0 is added per tile.
    const bool r_dma = has_bias && p.r_vec;
    unsigned svo[NSI];
    rsrc_t rR;
    u32x4 rR4;
    {
        const int64_t rbase = (int64_t)b * p.Rs0 + (int64_t)t0 * p.Rs1 + (int64_t)hkv * p.G * p.Rs2;
        const int64_t rspan = ((int64_t)(nrows - 1) * p.Rs1 + (int64_t)(p.G - 1) * p.Rs2 + p.E) * ES;
        rR = make_rsrc(has_bias ? (const T *)p.R + rbase : (const T *)p.q, has_bias ? rspan : 0);
        rR4 = make_rsrc_words(has_bias ? (const T *)p.R + rbase : (const T *)p.q, has_bias ? rspan : 0);
#pragma unroll
        for (int i = 0; i < NSI; ++i) {
            const int L = (i * NW + wave) * 64 + lane;
            const int row = L / NCH, ch = L - row * NCH;
            const int rhl = row / p.QB, rqi = row - rhl * p.QB;
            const bool live = row < ncols && rqi < nrows;
            const int rrb = (p_min + rqi - N + 1) & ~(CH - 1);
            // dead rows point far past the span: they read zeros
            svo[i] = live ? (unsigned)(((int64_t)rqi * p.Rs1 + (int64_t)rhl * p.Rs2 + rrb + ch * CH) * ES)
                          : 0x80000000u;
        }
    }

    typedef typename std::conditional<BF, u32x2, u32x4>::type VChunk;
    VChunk vreg[NVI];
    // F8 staging: each thread moves NP8 16-byte pieces (16 codes of one key
    // row, under one scale) of K and of V per tile.  Piece L is piece L % 8 of
    // key row L / 8.  Two register sets carry the next two tiles.
    constexpr int NP8 = F8 ? N * D / 16 / NTH : 1;
    struct F8Set {
        u32x4 k[NP8], v[NP8];
        unsigned char ks[NP8], vs[NP8];   // E8M0 codes, widened where used
    };
    // Offsets of piece 0; piece i is NTH / 8 rows further (the row
    // permutation and the chunk swizzle do not change over 32 rows).
    constexpr int RSTEP = NTH / 8;
    unsigned k8o = 0, k8s = 0, k8d = 0, v8o = 0, v8s = 0, v8d = 0;
    if constexpr (F8) {
        const int row = tid >> 3, c = tid & 7;
        k8o = (unsigned)((int64_t)row * p.ks1 + 16 * c);
        k8s = (unsigned)((int64_t)row * p.kss1 + (c >> 1));
        k8d = (unsigned)(lds_key_row(row) * KS + 16 * c);
        v8o = (unsigned)((int64_t)row * p.vs1 + 16 * c);
        v8s = (unsigned)((int64_t)row * p.vss1 + (c >> 1));
        // bf16 chunks 2c, 2c+1 of row r sit at chunks (2c) ^ 4(r % 4) and the next
        v8d = (unsigned)(row * D + 8 * ((2 * c) ^ ((row & 3) << 2)));
    }

    auto banded = [&](int kt) { return has_bias && (p_min - (kt * N + N - 1) < p.E); };

    // Rows j0 .. of K or V; rows past the sequence (or the page) read zeros.
    // Rows j0 .. of a per-key tensor at byte address g (strides in elements
    // of esz bytes, rowbytes bytes per row); rows past the sequence (or the
    // page) read zeros.
    auto kv_rsrc = [&](const char *g, int64_t pstride, int64_t stride, int j0, int esz, int rowbytes) {
        if constexpr (PG) {
            const int pg = __builtin_amdgcn_readfirstlane(j0 / p.page_size);   // wave-uniform
            const int off = j0 - pg * p.page_size;
            // through the scalar cache: a vector load would sit in the in-order
            // vector-memory queue and make the tile's staging wait for it
            const int page = min(max(load_scalar(p.block_table + (int64_t)b * p.bt_stride + pg), 0), p.num_pages - 1);
            const int rows = min(p.page_size - off, Skv - j0);
            return make_rsrc(g + ((int64_t)page * pstride + (int64_t)off * stride) * esz,
                             (int64_t)(rows - 1) * stride * esz + rowbytes);
        } else {
            return make_rsrc(g + (int64_t)j0 * stride * esz, (int64_t)(Skv - 1 - j0) * stride * esz + rowbytes);
        }
    };

    // The same rows as descriptor words, for dma16_untracked.
    auto kv_rsrc_words = [&](const char *g, int64_t pstride, int64_t stride, int j0, int esz, int rowbytes) {
        if constexpr (PG) {
            const int pg = __builtin_amdgcn_readfirstlane(j0 / p.page_size);
            const int off = j0 - pg * p.page_size;
            const int page = min(max(load_scalar(p.block_table + (int64_t)b * p.bt_stride + pg), 0), p.num_pages - 1);
            const int rows = min(p.page_size - off, Skv - j0);
            return make_rsrc_words(g + ((int64_t)page * pstride + (int64_t)off * stride) * esz,
                                   (int64_t)(rows - 1) * stride * esz + rowbytes);
        } else {
            return make_rsrc_words(g + (int64_t)j0 * stride * esz, (int64_t)(Skv - 1 - j0) * stride * esz + rowbytes);
        }
    };

    // FQ2: K codes of tile kt into K buffer buf by direct-to-LDS loads: LDS
    // chunk L (16 bytes) holds chunk L % 9 of code row L / 9, the ninth
    // (padding) chunk a repeat of chunk 0.  Untracked: the caller's counted
    // wait lands them before the barrier that hands them over.
    constexpr int K8CH = N * (K8R / 16);                 // 576 chunks
    constexpr int NK8I = (K8CH + NTH - 1) / NTH;
    unsigned k8vo[FQ2 ? NK8I : 1] = {};
    if constexpr (FQ2) {
#pragma unroll
        for (int i = 0; i < NK8I; ++i) {
            const int L = (i * NW + wave) * 64 + lane;
            const int row = L / (K8R / 16), c = L - row * (K8R / 16);
            k8vo[i] = (unsigned)((int64_t)min(row, N - 1) * p.ks1 + 16 * (c < D / 16 ? c : 0));
        }
    }
    auto stage_k8 = [&](int kt, int buf) __attribute__((always_inline)) {
        if constexpr (FQ2) {
            const u32x4 rk = kv_rsrc_words(gk, p.ks0, p.ks1, kt * N, 1, D);
#pragma unroll
            for (int i = 0; i < NK8I; ++i) {
                const int wc = (i * NW + wave) * 64;        // wave-uniform: whole waves in or out
                if (wc < K8CH) dma16_untracked(rk, k8vo[i], sK8 + buf * KBB + wc * 16);
            }
        }
    };

    // F8: codes and scales of tile kt's K and V into register set X
    auto load8 = [&](int kt, F8Set &X) __attribute__((always_inline)) {
        const rsrc_t rk = kv_rsrc(gk, p.ks0, p.ks1, kt * N, 1, D);
        const rsrc_t rks = kv_rsrc(gks, p.kss0, p.kss1, kt * N, 1, D / 32);
        const rsrc_t rv = kv_rsrc(gv, p.vs0, p.vs1, kt * N, 1, D);
        const rsrc_t rvs = kv_rsrc(gvs, p.vss0, p.vss1, kt * N, 1, D / 32);
#pragma unroll
        for (int i = 0; i < NP8; ++i) {
            const unsigned r = (unsigned)(i * RSTEP);
            if constexpr (!FQ2) X.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, k8o + r * (unsigned)p.ks1, 0, 0);
            X.ks[i] = __builtin_amdgcn_raw_buffer_load_b8(rks, k8s + r * (unsigned)p.kss1, 0, 0);
            X.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, v8o + r * (unsigned)p.vs1, 0, 0);
            X.vs[i] = __builtin_amdgcn_raw_buffer_load_b8(rvs, v8s + r * (unsigned)p.vss1, 0, 0);
        }
    };
    // vector-memory instructions one load8 issues (FQ2: K codes go by DMA)
    constexpr int kLoad8Ops = (FQ2 ? 3 : 4) * NP8;

    // F8: decode register set X into the K and V buffers (bf16)
    auto store8 = [&](const F8Set &X, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NP8; ++i) {
            const float sk = e8m0_scale(X.ks[i]), sv = e8m0_scale(X.vs[i]);
            if constexpr (FQ) {
                const int row = (tid >> 3) + i * RSTEP, c = tid & 7;
                if constexpr (!FQ2) *(u32x4 *)&sK8[row * K8R + 16 * c] = X.k[i];
                if ((c & 1) == 0) sK8[buf * KBB + K8S + 4 * row + (c >> 1)] = (unsigned char)X.ks[i];
            } else {
                u32x2 a = e4m3x4_to_bf16(X.k[i][0], sk), b2 = e4m3x4_to_bf16(X.k[i][1], sk);
                u32x2 c = e4m3x4_to_bf16(X.k[i][2], sk), d = e4m3x4_to_bf16(X.k[i][3], sk);
                T *dst = &sK[0][k8d + i * RSTEP * KS];
                *(u32x4 *)dst = u32x4{a[0], a[1], b2[0], b2[1]};
                *(u32x4 *)(dst + 8) = u32x4{c[0], c[1], d[0], d[1]};
            }
            u32x2 a = e4m3x4_to_bf16(X.v[i][0], sv), b2 = e4m3x4_to_bf16(X.v[i][1], sv);
            u32x2 c = e4m3x4_to_bf16(X.v[i][2], sv), d = e4m3x4_to_bf16(X.v[i][3], sv);
            T *dst = &sV[buf * VSZ + v8d + i * RSTEP * D];
            *(u32x4 *)dst = u32x4{a[0], a[1], b2[0], b2[1]};
            *(u32x4 *)(dst + 8) = u32x4{c[0], c[1], d[0], d[1]};
        }
    };

    // FQ2 with a wave that has no columns: that wave alone moves V and the
    // scales of a tile through its registers (8 pieces a lane: piece i of
    // lane l is row 8 i + l / 8, 16-code piece l % 8) and decodes them, while
    // the other waves compute.
    // (MXFP8 cache with bf16 logits, VD: K codes too, decoded into the bf16
    // K layout.)
    constexpr bool PK = F8 && VD;
    struct F8SetP {
        u32x4 v[8], k[PK ? 8 : 1];
        unsigned char ks[8], vs[8];
    };
    const int pc8 = lane & 7, pr8 = lane >> 3;
    const unsigned k8oP = (unsigned)((int64_t)pr8 * p.ks1 + 16 * pc8);
    const unsigned k8sP = (unsigned)((int64_t)pr8 * p.kss1 + (pc8 >> 1));
    const unsigned v8oP = (unsigned)((int64_t)pr8 * p.vs1 + 16 * pc8);
    const unsigned v8sP = (unsigned)((int64_t)pr8 * p.vss1 + (pc8 >> 1));
    auto load8P = [&](int kt, F8SetP &X, auto role_c) __attribute__((always_inline)) {
        constexpr int ROLE = decltype(role_c)::value;     // 0: K and V, 1: K only, 2: V only
        const rsrc_t rk = kv_rsrc(gk, p.ks0, p.ks1, kt * N, 1, D);
        const rsrc_t rks = kv_rsrc(gks, p.kss0, p.kss1, kt * N, 1, D / 32);
        const rsrc_t rv = kv_rsrc(gv, p.vs0, p.vs1, kt * N, 1, D);
        const rsrc_t rvs = kv_rsrc(gvs, p.vss0, p.vss1, kt * N, 1, D / 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const unsigned r = (unsigned)(8 * i);
            if constexpr (ROLE != 2) {
                if constexpr (PK) X.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, k8oP + r * (unsigned)p.ks1, 0, 0);
                X.ks[i] = __builtin_amdgcn_raw_buffer_load_b8(rks, k8sP + r * (unsigned)p.kss1, 0, 0);
            }
            if constexpr (ROLE != 1) {
                X.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, v8oP + r * (unsigned)p.vs1, 0, 0);
                X.vs[i] = __builtin_amdgcn_raw_buffer_load_b8(rvs, v8sP + r * (unsigned)p.vss1, 0, 0);
            }
        }
    };
    // vector-memory instructions one load8P of a role issues
    auto load8P_ops = [](int role) constexpr { return role == 0 ? (PK ? 32 : 24) : (role == 1 ? (PK ? 16 : 8) : 16); };
    auto store8P = [&](const F8SetP &X, int buf, auto role_c) __attribute__((always_inline)) {
        constexpr int ROLE = decltype(role_c)::value;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = 8 * i + pr8;
            if constexpr (ROLE == 2) {
            } else if constexpr (PK) {
                const float sk = e8m0_scale(X.ks[i]);
                const u32x2 a = e4m3x4_to_bf16(X.k[i][0], sk), b2 = e4m3x4_to_bf16(X.k[i][1], sk);
                const u32x2 c = e4m3x4_to_bf16(X.k[i][2], sk), d = e4m3x4_to_bf16(X.k[i][3], sk);
                T *dst = &sK[buf][lds_key_row(row) * KS + 16 * pc8];
                *(u32x4 *)dst = u32x4{a[0], a[1], b2[0], b2[1]};
                *(u32x4 *)(dst + 8) = u32x4{c[0], c[1], d[0], d[1]};
            } else if ((pc8 & 1) == 0) {
                sK8[buf * KBB + K8S + 4 * row + (pc8 >> 1)] = X.ks[i];
            }
            if constexpr (ROLE == 1) continue;
            const float sv = e8m0_scale(X.vs[i]);
            const u32x2 a = e4m3x4_to_bf16(X.v[i][0], sv), b2 = e4m3x4_to_bf16(X.v[i][1], sv);
            const u32x2 c = e4m3x4_to_bf16(X.v[i][2], sv), d = e4m3x4_to_bf16(X.v[i][3], sv);
            T *dst = &sV[buf * VSZ + row * D + 8 * ((2 * pc8) ^ ((row & 3) << 2))];
            *(u32x4 *)dst = u32x4{a[0], a[1], b2[0], b2[1]};
            *(u32x4 *)(dst + 8) = u32x4{c[0], c[1], d[0], d[1]};
        }
    };

    // VD: V tile kt into V buffer buf.  LDS chunk L (16 bytes) holds chunk
    // (L % 16) ^ 4 (r % 4) of key row r = L / 16, the layout the transposed
    // reads of PV expect.
    constexpr int NVDI = N * D * ES / 16 / NTH;
    unsigned vdo[(VD && !F8) ? NVDI : 1] = {};
    if constexpr (VD && !F8) {
#pragma unroll
        for (int i = 0; i < NVDI; ++i) {
            const int L = (i * NW + wave) * 64 + lane;
            const int r = L >> 4, c = (L & 15) ^ ((r & 3) << 2);
            vdo[i] = (unsigned)(((int64_t)r * p.vs1 + c * CH) * ES);
        }
    }
    auto stage_vd = [&](int kt, int buf) __attribute__((always_inline)) {
        if constexpr (VD && !F8) {
            const u32x4 rv = kv_rsrc_words(gv, p.vs0, p.vs1, kt * N, ES, D * ES);
#pragma unroll
            for (int i = 0; i < NVDI; ++i) dma16_untracked(rv, vdo[i], &sV[buf * VSZ + (i * NW + wave) * 64 * CH]);
        }
    };

    auto stage_k = [&](int kt, int buf) {
        const rsrc_t rk = kv_rsrc(gk, p.ks0, p.ks1, kt * N, ES, D * ES);
        const u32x4 rkw = kv_rsrc_words(gk, p.ks0, p.ks1, kt * N, ES, D * ES);
#pragma unroll
        for (int i = 0; i < NKI; ++i) {
            const int wc = (i * NW + wave) * 64;
            if (i < NKI - 1 || wc + lane < KCH) {
                if constexpr (VD)
                    dma16_untracked(rkw, kvo[i], &sK[buf][wc * CH]);
                else
                    dma16(rk, kvo[i], &sK[buf][wc * CH]);
            }
        }
    };

    auto load_v = [&](int kt) {
        const rsrc_t rv = kv_rsrc(gv, p.vs0, p.vs1, kt * N, ES, D * ES);
#pragma unroll
        for (int i = 0; i < NVI; ++i) {
            if constexpr (BF)
                vreg[i] = __builtin_amdgcn_raw_buffer_load_b64(rv, vvo[i], 0, 0);
            else
                vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, vvo[i], 0, 0);
        }
    };

    auto store_v = [&]() {
        if constexpr (BF) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int w = e >> 1;
                unsigned out[NVI / 2];
#pragma unroll
                for (int mm = 0; mm < NVI / 2; ++mm) {
                    const unsigned lo = vreg[2 * mm][w], hi = vreg[2 * mm + 1][w];
                    out[mm] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                }
                T *dst = &sV[(4 * v_dq + e) * VS + NVI * v_kq];
                if constexpr (NVI == 8)
                    *(u32x4 *)dst = u32x4{out[0], out[1], out[2], out[3]};
                else
                    *(u32x2 *)dst = u32x2{out[0], out[1]};
            }
        } else {
#pragma unroll
            for (int i = 0; i < NVI; ++i) {
                const int ci = tid + NTH * i;
                const int row = ci / CPR, cc = ci - row * CPR;
                *(u32x4 *)&sV[row * VS + cc * CH] = vreg[i];
            }
        }
    };

    // Each column's R window for tile kt.  Entries outside [0, E) hold
    // neighbouring rows or zeros; the gather never uses them (future keys
    // are masked; distances >= E are tested).
    auto stage_slab = [&](int kt, int buf) {
        const int eoff = -kt * N * ES;
        if (r_dma) {
#pragma unroll
            for (int i = 0; i < NSI; ++i) {
                const int wc = (i * NW + wave) * 64;
                if (i < NSI - 1 || wc + lane < SCH) dma16(rR, svo[i] + (unsigned)eoff, &sR[buf][wc * CH]);
            }
        } else {
            // rows not 16-byte aligned: element loads through registers
#pragma unroll
            for (int i = 0; i < NSI; ++i) {
                const int L = (i * NW + wave) * 64 + lane;
                if (L < SCH) {
                    u32x4 val = u32x4{};
#pragma unroll
                    for (int x = 0; x < CH; ++x) {
                        const unsigned off = svo[i] + (unsigned)eoff + (unsigned)(x * ES);
                        if constexpr (BF)
                            val[x >> 1] |= (unsigned)__builtin_amdgcn_raw_buffer_load_b16(rR, off, 0, 0) << (16 * (x & 1));
                        else
                            val[x] = __builtin_amdgcn_raw_buffer_load_b32(rR, off, 0, 0);
                    }
                    *(u32x4 *)&sR[buf][L * CH] = val;
                }
            }
        }
    };

    // The single bias buffer (SLAB2 false) for key tile kt, issued while the
    // tile before it is computed (that tile then carries no bias, so the
    // buffer is free).  Untracked so that the compiler does not hold the LDS
    // reads of that compute until it lands; the end-of-iteration wait does.
    auto stage_slab_ahead = [&](int kt, int buf) {
        const unsigned eoff = (unsigned)(-kt * N * ES);
#pragma unroll
        for (int i = 0; i < NSI; ++i) {
            const int wc = (i * NW + wave) * 64;
            if (i < NSI - 1 || wc + lane < SCH) dma16_untracked(rR4, svo[i] + eoff, &sR[buf][wc * CH]);
        }
    };

    // ------------------------------------------------------------ one key tile
    const int kr0 = lds_key_row(mfma_row_key(lc));   // LDS row of this lane's A-operand key (+32: sub-tile 1)
    const T *k_lane = &sK[0][kr0 * KS];
    const T *v_lane = BF ? &sV[lc * VS + 16 * hh] : &sV[16 * hh * VS + lc];
    // F8 (row-major V): V^T fragment of PV step (u, h2, dt) by two transpose
    // reads of 4 keys each.  Lane (g = lane / 16, a = lane % 4, i = lane / 4 % 4)
    // addresses key row 32u + 16(g / 2) + 8h2 + 4x + i and head-dim entries
    // 32dt + 16(g % 2) + 4a, and receives key rows of one head-dim entry back.
    const int tr_i = (lane >> 2) & 3;
    const int vt_base = (16 * hh + tr_i) * D + CH * ((((lane >> 4) & 1) << 1) | ((lane >> 1) & 1)) + 4 * (lane & 1);
    auto vt_off = [&](int dt) __attribute__((always_inline)) { return vt_base + CH * (((dt ^ tr_i) << 2)); };
    const int s_lane = col * SW + (prow - rb) - 16 * hh;   // slab entry of key offset 16*hh

    auto compute_tile = [&](int kt, int buf, int sbuf) __attribute__((always_inline)) {
        const int j0 = kt * N;
        f32x16 S[KT];
#pragma unroll
        for (int u = 0; u < KT; ++u) S[u] = f32x16{};

        // S^T = K . Q^T
        const T *kb_ = k_lane + buf * (N * KS);
        if constexpr (FQ) {
            // A operand: key row 32u + mfma_row_key(lc), entries 64ks + 16hh
            // + [0, 16) and 64ks + 32 + 16hh + [0, 16); its scale is the
            // row's block 2ks + hh (see the q encoding above)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int u = 0; u < KT; ++u) {
                    const int kr = 32 * u + mfma_row_key(lc);
                    const unsigned char *src = sK8 + buf * KBB + kr * K8R + 64 * ks + 16 * hh;
                    const u32x4 lo = *(const u32x4 *)src, hi = *(const u32x4 *)(src + 32);
                    const i32x8 a = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    const int sa = sK8[buf * KBB + K8S + 4 * kr + 2 * ks + hh];
                    S[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, q8[ks], S[u], 0, 0, 0, sa, 0, qsc[ks]);
                }
            }
        } else if constexpr (BF) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
#pragma unroll
                for (int u = 0; u < KT; ++u) {
                    const bf16x8 a = *(const bf16x8 *)(kb_ + u * 32 * KS + 16 * k + 8 * hh);
                    S[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[k], S[u], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const f32x4 a = *(const f32x4 *)(kb_ + 64 * hh + 4 * k);
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    S[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[x], qf[4 * k + x], S[0], 0, 0, 0);
            }
        }

        const bool band = banded(kt);
        const bool edge = !((j0 + N - 1 <= p_min) && (W == 0 || p_max - j0 < W));

        if (band) {
            // x = scale f q.k + f bias, in log2 units
            const T *sr = &sR[sbuf][s_lane];
            const bool partial = p_max - j0 >= p.E;      // some entries lie past the extent
            const int elim = prow - j0 - 16 * hh - p.E;  // key offset r (within the half) has e < E iff r > elim
#pragma unroll
            for (int u = 0; u < KT; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float bias;
                    if constexpr (BF)
                        bias = __builtin_bit_cast(float, (unsigned)__builtin_bit_cast(unsigned short, sr[-(32 * u + r)]) << 16);
                    else
                        bias = sr[-(32 * u + r)];
                    if (partial) bias = (32 * u + r > elim) ? bias : 0.f;
                    S[u][r] = fmaf(bias, bmul, S[u][r] * amul);
                }
        }
        if (edge) {
#pragma unroll
            for (int u = 0; u < KT; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int dist = prow - (j0 + 32 * u + 16 * hh + r);
                    const bool vis = dist >= 0 && (W == 0 || dist < W);
                    S[u][r] = vis ? S[u][r] : -INFINITY;
                }
        }
        // multiplier still to apply to S (interior tiles hold raw dot products)
        const float sa = band ? 1.f : amul;

        if constexpr (BF) {
            // Probabilities against the current reference max m (exp2 domain),
            // rounded to bf16 for PV; the row sum adds the fp32 values in two
            // chains (a v_dot2c sum over the bf16 values stalls beside the
            // other workgroup's MFMAs on the same SIMD).  The reference only
            // moves when the tile max exceeds it by more than kRescaleSlack.
            // While this lane's probabilities sum to at most 2^kRescaleSlack
            // none of them exceeds that bound, so the tile max is not needed;
            // otherwise, and at a column's first visible tile, it is taken and,
            // if m moves, O and l are rescaled and P recomputed.  Decisions
            // are wave-uniform, so both halves of a column decide alike.
            bf16x8 P[2 * KT];
            float sum = 0.f;
            auto exps = [&](float mu) __attribute__((always_inline)) {
                float sm[2] = {0.f, 0.f};
#pragma unroll
                for (int u = 0; u < KT; ++u)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        bf16x8 pb;
#pragma unroll
                        for (int x = 0; x < 8; ++x) {
                            const float e = fast_exp2(fmaf(S[u][8 * h2 + x], sa, -mu));
                            pb[x] = (__bf16)e;
                            sm[x & 1] += e;
                        }
                        P[2 * u + h2] = pb;
                    }
                sum = sm[0] + sm[1];
            };
            exps(m == -INFINITY ? 0.f : m);
            const bool slow = !(sum <= kRescaleLimit) || m == -INFINITY;
            if (__builtin_amdgcn_ballot_w64(slow) != 0) {
                float mt = -INFINITY;
#pragma unroll
                for (int u = 0; u < KT; ++u)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, S[u][r]);
                mt = max_across_halves(mt * sa);
                const bool grow = mt > m + kRescaleSlack;
                if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                    const float mn = grow ? mt : m;
                    const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mn);
                    m = mn;
                    l *= alpha;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) O[dt] *= alpha;
                    exps(m == -INFINITY ? 0.f : m);
                }
            }
            l += sum;

            // O^T += V^T . P^T
#pragma unroll
            for (int u = 0; u < KT; ++u) {
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) {
                        bf16x8 a;
                        if constexpr (F8 || VD) {
                            typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
                            const T *base = &sV[((FQ2 || VD) ? buf * VSZ : 0) + vt_off(dt) + (32 * u + 8 * h2) * D];
                            const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                (__attribute__((address_space(3))) bf16x4_t *)base);
                            const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                (__attribute__((address_space(3))) bf16x4_t *)(base + 4 * D));
                            a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                        } else {
                            a = *(const bf16x8 *)(v_lane + 32 * dt * VS + 32 * u + 8 * h2);
                        }
                        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[2 * u + h2], O[dt], 0, 0, 0);
                    }
                }
            }
        } else {
            // fp32: max first, then the exponentials in place
            float mt = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, S[0][r]);
            mt = max_across_halves(mt * sa);
            const bool grow = mt > m + kRescaleSlack;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                const float mn = grow ? mt : m;
                const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mn);
                m = mn;
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) O[dt] *= alpha;
            }
            const float mu = m == -INFINITY ? 0.f : m;
#pragma unroll
            for (int r = 0; r < 16; ++r) S[0][r] = fast_exp2(fmaf(S[0][r], sa, -mu));
            float sum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sum += S[0][r];
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const float a = v_lane[r * VS + 32 * dt];
                    O[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, S[0][r], O[dt], 0, 0, 0);
                }
            }
            l += sum;
        }
    };

    // ------------------------------------------------------------ main loop
    // Banded tiles (the suffix [kband, ke)) read R from HBM; they are spread
    // evenly through the tile sequence so that all workgroups do not demand
    // R at the same time.  Online softmax does not depend on the order.
    const int n_it = ke - kb;
    int kband = ke;
    if (has_bias) {
        // banded(kt)  <=>  kt * N > p_min - N + 1 - E
        const int x = p_min - N + 1 - p.E;
        const int first = x < 0 ? 0 : x / N + 1;
        kband = min(max(first, kb), ke);
    }
    const int n_band = ke - kband;
    // iteration i is banded iff floor((i+1) nb / n) > floor(i nb / n); scalar,
    // incremental
    int g_rem = 0, g_cnt = 0, g_idx = 0;
    auto next_tile = [&]() {
        const bool bnd = g_rem + n_band >= n_it;
        const int kt = bnd ? kband + g_cnt : kb + g_idx - g_cnt;
        g_rem += n_band;
        if (g_rem >= n_it) {
            g_rem -= n_it;
            ++g_cnt;
        }
        ++g_idx;
        return kt;
    };

    // Two workgroups share a CU and the older one's waves win issue ties, so
    // with equal work the younger one finishes last and the launch waits for
    // it.  The wave priority therefore alternates every kPrioPeriod tiles, in
    // opposite phase for the two halves of the grid (the halves that were
    // dispatched as first and second workgroup of a CU), so both progress
    // alike on average.
    auto fair_prio = [&](int it) __attribute__((always_inline)) {
        if constexpr (NW == 4) {
            if ((((it / kPrioPeriod) + (blockIdx.x >= gridDim.x / 2)) & 1) != 0)
                __builtin_amdgcn_s_setprio(1);
            else
                __builtin_amdgcn_s_setprio(0);
        }
    };
    int kt = n_it > 0 ? next_tile() : 0;
    // exactly one of the tile loops below runs for a configuration
    static_assert((int)(FQ2 || PK) + (int)(F8 && !FQ2 && !PK) + (int)(VD && !F8) + (int)(!VD && !F8) == 1,
                  "one tile loop per kernel configuration");
    if constexpr (FQ2 || PK) {
        // (PK: the MXFP8 cache with bf16 logits; its K codes travel with V
        // through the staging wave, which decodes both, and the launch picks
        // this variant only when the last wave has no columns.)
        // K codes by DMA one tile ahead into alternating buffers; V codes and
        // the scales of both two tiles ahead through registers.  The next
        // tile's V is decoded into the other buffers while this tile is
        // computed, and one barrier per tile hands both over.  With a wave
        // that has no columns, that wave (the last) does all of the decoding;
        // otherwise every thread decodes its share right after its compute.
        // The single bias buffer is loaded ahead when the tile being computed
        // carries no bias, else after the barrier (then a second one).
        const bool split = (NW - 1) * 32 >= ncols;          // the last wave has no columns
        // MXFP8 cache with two waves without columns: the last decodes V, the
        // one before it K; otherwise the last wave decodes both
        const bool split2 = PK && (NW - 2) * 32 >= ncols;
        const bool producer = split && (wave == NW - 1 || (split2 && wave == NW - 2));
        int kn = n_it > 1 ? next_tile() : kt;
        // the barriers of one tile, common to both roles; returns kn's successor
        auto tile_end = [&](int it, bool sahead, int kn2) __attribute__((always_inline)) {
            const bool nxt = it + 1 < n_it;
            __syncthreads();
            if (nxt && banded(kn) && !sahead) {
                stage_slab(kn, 0);
                wait_vmem();
                __syncthreads();
            }
            kt = kn;
            kn = kn2;
        };
        auto tile_begin = [&](int it, bool &sahead) __attribute__((always_inline)) {
            fair_prio(it);
            const bool nxt = it + 1 < n_it, nxt2 = it + 2 < n_it;
            const int kn2 = nxt2 ? next_tile() : kn;
            sahead = nxt && r_dma && banded(kn) && !banded(kt);
            if constexpr (FQ2) {
                if (nxt) stage_k8(kn, (it & 1) ^ 1);    // last read by the previous tile's compute
            }
            if (sahead) stage_slab_ahead(kn, 0);
            return kn2;
        };
        if (split) {
            if (producer) {
                auto stage = [&](auto role_c) __attribute__((always_inline)) {
                    constexpr int ROLE = decltype(role_c)::value;
                    constexpr int OPS = load8P_ops(ROLE);
                    F8SetP A, B;
                    if (n_it > 0) {
                        if constexpr (FQ2) stage_k8(kt, 0);
                        load8P(kt, A, role_c);
                        load8P(kn, B, role_c);
                        if (banded(kt)) stage_slab(kt, 0);
                        store8P(A, 0, role_c);
                        wait_vmem();
                    }
                    __syncthreads();
                    auto body = [&](int it, F8SetP &X, F8SetP &Y) __attribute__((always_inline)) {
                        bool sahead;
                        const int kn2 = tile_begin(it, sahead);
                        // issued on every tile (the last two repeat a tile and are
                        // never stored), so that every path carries the same count
                        load8P(kn2, Y, role_c);
                        if (it + 1 < n_it) store8P(X, (it & 1) ^ 1, role_c);
                        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(OPS) : "memory");
                        tile_end(it, sahead, kn2);
                    };
                    for (int it = 0; it < n_it; it += 2) {
                        body(it, B, A);
                        if (it + 1 < n_it) body(it + 1, A, B);
                    }
                    wait_vmem();
                };
                if (!split2)
                    stage(std::integral_constant<int, 0>{});
                else if (wave == NW - 1)
                    stage(std::integral_constant<int, 2>{});
                else
                    stage(std::integral_constant<int, 1>{});
                // no columns: nothing to write.  Leaving here makes q and O dead
                // on this path, which the K decode's registers need.
                if constexpr (PK) return;
            } else {
                if (n_it > 0) {
                    if constexpr (FQ2) stage_k8(kt, 0);
                    if (banded(kt)) stage_slab(kt, 0);
                    wait_vmem();
                }
                __syncthreads();
                for (int it = 0; it < n_it; ++it) {
                    bool sahead;
                    const int kn2 = tile_begin(it, sahead);
                    if (wave_active) compute_tile(kt, it & 1, 0);
                    wait_vmem();
                    tile_end(it, sahead, kn2);
                }
            }
        } else if constexpr (FQ2) {
            F8Set A, B;
            if (n_it > 0) {
                stage_k8(kt, 0);
                load8(kt, A);
                load8(kn, B);
                if (banded(kt)) stage_slab(kt, 0);
                store8(A, 0);
                wait_vmem();
            }
            __syncthreads();
            auto body = [&](int it, F8Set &X, F8Set &Y) __attribute__((always_inline)) {
                bool sahead;
                const int kn2 = tile_begin(it, sahead);
                // issued on every tile (the last two repeat a tile and are never
                // stored), so that the compiler's wait for X before the stores
                // below counts Y's loads on every path and leaves them in flight
                load8(kn2, Y);
                if (wave_active) compute_tile(kt, it & 1, 0);
                if (it + 1 < n_it) store8(X, (it & 1) ^ 1);
                // K codes and bias of kn landed (issued before Y's loads)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoad8Ops) : "memory");
                tile_end(it, sahead, kn2);
            };
            for (int it = 0; it < n_it; it += 2) {
                body(it, B, A);
                if (it + 1 < n_it) body(it + 1, A, B);
            }
            wait_vmem();
        }
    }
    if constexpr (F8 && !FQ2 && !PK) {
        // Two tiles in flight: while tile kt is computed from LDS, the codes of
        // tile kn wait in one register set and those of the tile after it load
        // into the other; each iteration decodes kn into the (single) K and V
        // buffers between two barriers.  Bias windows are double-buffered and
        // go by direct-to-LDS loads issued before the next codes, so a counted
        // wait lands them without waiting for the codes.
        F8Set A, B;
        int kn = n_it > 1 ? next_tile() : kt;
        if (n_it > 0) {
            load8(kt, A);
            if (n_it > 1) load8(kn, B);
            if (banded(kt)) stage_slab(kt, 0);
            store8(A, 0);
            wait_vmem();
        }
        __syncthreads();
        auto body = [&](int it, F8Set &X, F8Set &Y) __attribute__((always_inline)) {
            fair_prio(it);
            const bool nxt = it + 1 < n_it, nxt2 = it + 2 < n_it;
            const int kn2 = nxt2 ? next_tile() : kn;
            const int sb = it & 1;                       // bias buffer of kt; kn's is sb ^ 1
            const bool sdma = nxt && r_dma && banded(kn);
            if (sdma) stage_slab_ahead(kn, sb ^ 1);
            if (nxt2) load8(kn2, Y);
            if (wave_active) compute_tile(kt, 0, sb);
            if (sdma) {
                if (nxt2)
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoad8Ops) : "memory");
                else
                    wait_vmem();
            }
            __syncthreads();                             // kt consumed; kn's bias landed
            if (nxt) {
                store8(X, 0);
                if (!r_dma && banded(kn)) {
                    stage_slab(kn, sb ^ 1);
                    wait_vmem();
                }
            }
            __syncthreads();
            kt = kn;
            kn = kn2;
        };
        for (int it = 0; it < n_it; it += 2) {
            body(it, B, A);
            if (it + 1 < n_it) body(it + 1, A, B);
        }
    }
    if constexpr (VD && !F8) {
        if (n_it > 0) {
            stage_k(kt, 0);
            stage_vd(kt, 0);
            if (banded(kt)) stage_slab(kt, 0);
            wait_vmem();
        }
        __syncthreads();
        for (int it = 0; it < n_it; ++it) {
            fair_prio(it);
            const int cur = it & 1;
            const bool nxt = it + 1 < n_it;
            const int kn = nxt ? next_tile() : kt;
            const bool sahead = nxt && r_dma && banded(kn) && !banded(kt);
            if (nxt) {
                stage_k(kn, cur ^ 1);       // both buffers last read by the previous tile's compute
                stage_vd(kn, cur ^ 1);
            }
            if (sahead) stage_slab_ahead(kn, 0);
            if (wave_active) compute_tile(kt, cur, 0);
            wait_vmem();
            __syncthreads();            // tile kt consumed; kn's K, V and bias landed
            if (nxt && banded(kn) && !sahead) {
                stage_slab(kn, 0);
                wait_vmem();
                __syncthreads();
            }
            kt = kn;
        }
    }
    if (!VD && !F8 && n_it > 0) {
        stage_k(kt, 0);
        load_v(kt);
        if (banded(kt)) stage_slab(kt, 0);
        store_v();
        wait_vmem();
    }
    if (!VD && !F8) __syncthreads();
    for (int it = 0; it < ((F8 || VD) ? 0 : n_it); ++it) {
        fair_prio(it);
        const int cur = it & 1;
        const bool nxt = it + 1 < n_it;
        const int kn = nxt ? next_tile() : kt;
        const bool slab_ahead = !SLAB2 && nxt && r_dma && banded(kn) && !banded(kt);
        if (nxt) {
            stage_k(kn, cur ^ 1);
            if (slab_ahead) stage_slab_ahead(kn, 0);
            load_v(kn);
            if (SLAB2 && banded(kn)) stage_slab(kn, cur ^ 1);
        }
        if (wave_active) compute_tile(kt, cur, SLAB2 ? cur : 0);
        wait_vmem();
        __syncthreads();             // tile kt fully consumed; loads for kn landed
        if (nxt) {
            store_v();
            if (!SLAB2 && banded(kn) && !slab_ahead) {
                stage_slab(kn, 0);
                wait_vmem();
            }
        }
        __syncthreads();
        kt = kn;
    }

    // ------------------------------------------------------------ epilogue
    const float lt = l + __shfl_xor(l, 32);
    if (!cvalid) return;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_v = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
    if (p.splits == 1) {
        T *op = (T *)p.o + (int64_t)b * p.os0 + (int64_t)tq * p.os1 + (int64_t)hq * p.os2;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * dt + 8 * g4 + 4 * hh;
                if constexpr (BF) {
                    bf16x4 w;
#pragma unroll
                    for (int x = 0; x < 4; ++x) w[x] = (__bf16)(O[dt][4 * g4 + x] * inv);
                    *(bf16x4 *)(op + d0) = w;
                } else {
                    f32x4 w;
#pragma unroll
                    for (int x = 0; x < 4; ++x) w[x] = O[dt][4 * g4 + x] * inv;
                    *(f32x4 *)(op + d0) = w;
                }
            }
        if (p.lse != nullptr && hh == 0) p.lse[((int64_t)b * p.Hq + hq) * p.Sq + tq] = lse_v;
    } else {
        const int64_t row = (((int64_t)sp * p.B + b) * p.Sq + tq) * p.Hq + hq;
        float *op = p.o_part + row * D;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * dt + 8 * g4 + 4 * hh;
                f32x4 w;
#pragma unroll
                for (int x = 0; x < 4; ++x) w[x] = O[dt][4 * g4 + x] * inv;
                *(f32x4 *)(op + d0) = w;
            }
        if (hh == 0) p.lse_part[row] = lse_v;
    }
}

// Prefill with 8 waves in two groups (waves 0-3 and 4-7; each SIMD holds one
// wave of each).  Time is cut into phases separated by workgroup barriers.
// In every phase one group runs its matrix work (PV of its previous tile and
// S^T = K Q^T of the current one) while the other group runs the softmax of
// its latest scores, so the matrix cores and the vector ALUs of each SIMD
// work at the same time.  Roles swap every phase:
//   group 0: phase 2t   MFMA [PV(t-1), QK(t)]   phase 2t+1 VALU [softmax(t)]
//   group 1: phase 2t   VALU [softmax(t-1)]     phase 2t+1 MFMA [PV(t-1), QK(t)]
// Each group runs its own copy of the phase loop with its roles fixed at
// compile time.  All staging is global -> LDS DMA issued by group 1 during
// its even-phase softmax (one burst at its start, or four bursts spread over
// it in the fused variants) and awaited at the end of the
// following odd phase: K(t+1), V(t) and the bias windows of both groups
// (group 0's for tile t+1, group 1's for tile t).  V is kept row-major in LDS
// (16-byte chunks XOR-swizzled by row) and read as the PV A-operand with the
// LDS transpose read, so it never passes through registers.  LDS regions are
// padded to whole DMA instructions so no lane needs masking.
// Rows of R for one prefill block, computed in place of reading R ([S-RPB]:
// the relative logits of a token are its feature r times the head's P).
// Lane (lc, hh) of wave w serves query column c = 32 w + lc (head hl = c / QB,
// row qi = c % QB) and computes R[t0 + qi, hkv G + hl, e] for all e; tile eb
// of 32 distances goes to ws[((hl nEB + eb) QB + qi) 32 + e - 32 eb] (bf16),
// so the 32 rows of one tile are 2 KB of consecutive stores.  The MFMA
// operands and their order are those of relproj_kernel (A = rows of P^T in
// mfma_row_key order, B = r, k-steps ascending, fp32 accumulation, one
// rounding to bf16), so the values equal rba_relproj's bit for bit.  The A
// fragments come from the packed projection (relproj_pack_kernel), where the
// 64 lanes' fragments of one (head, tile, k-step) are 1 KB of consecutive
// memory.  FK k-steps of 16 channels are held (r_dim <= 16 FK).
template <int FK>
__device__ __forceinline__ void bias_rows(const AttnParams &p, __bf16 *ws, int b, int hkv, int t0, int nrows,
                                          int wave, int lane) {
    typedef __bf16 T;
    constexpr int NB = 8 / FK;   // distance tiles per load group; two groups in flight
    const int lc = lane & 31, hh = lane >> 5;
    const int col = wave * 32 + lc;
    const int hl = col / p.QB, qi = col - hl * p.QB;
    const bool valid = col < p.G * p.QB && qi < nrows;
    const int hq = hkv * p.G + min(hl, p.G - 1);
    const int nks = p.r_dim >> 4;
    const int nEB = (p.E + 31) >> 5;
    const T *rrow = (const T *)p.rf + (int64_t)b * p.rfs0 + (int64_t)(t0 + (valid ? qi : 0)) * p.rfs1 +
                    (int64_t)hq * p.rfs2 + 8 * hh;
    bf16x8 rfr[FK];
#pragma unroll
    for (int k = 0; k < FK; ++k) rfr[k] = k < nks ? *(const bf16x8 *)(rrow + 16 * k) : bf16x8{};
    const int h_lo = (wave * 32) / p.QB;
    const int h_hi = min((wave * 32 + 31) / p.QB, p.G - 1);
    for (int hp = h_lo; hp <= h_hi; ++hp) {
        const T *pt = (const T *)p.PT + (int64_t)(hkv * p.G + hp) * nEB * nks * 512 + lane * 8;
        const bool mine = valid && hl == hp;
        T *dst = ws + ((int64_t)hp * nEB * p.QB + qi) * 32 + 16 * hh;
        auto load = [&](bf16x8 (&a)[NB][FK], int eb0) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int k = 0; k < FK; ++k)
                    a[j][k] = (k < nks && eb0 + j < nEB) ? *(const bf16x8 *)(pt + ((int64_t)(eb0 + j) * nks + k) * 512)
                                                         : bf16x8{};
        };
        auto compute = [&](const bf16x8 (&a)[NB][FK], int eb0) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int eb = eb0 + j;
                if (eb >= nEB) break;
                f32x16 acc = f32x16{};
#pragma unroll
                for (int k = 0; k < FK; ++k)
                    if (k < nks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j][k], rfr[k], acc, 0, 0, 0);
                if (!mine) continue;
                bf16x8 w0, w1;
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    w0[x] = (__bf16)acc[x];
                    w1[x] = (__bf16)acc[8 + x];
                }
                T *d = dst + (int64_t)eb * p.QB * 32;
                *(bf16x8 *)d = w0;
                *(bf16x8 *)(d + 8) = w1;
            }
        };
        // groups of NB tiles alternate between two register sets: the loads of
        // the next group are in flight while this one is computed
        bf16x8 a0[NB][FK], a1[NB][FK];
        load(a0, 0);
        for (int eb0 = 0; eb0 < nEB; eb0 += 2 * NB) {
            if (eb0 + NB < nEB) load(a1, eb0 + NB);
            compute(a0, eb0);
            if (eb0 + NB >= nEB) break;
            if (eb0 + 2 * NB < nEB) load(a0, eb0 + 2 * NB);
            compute(a1, eb0 + NB);
        }
    }
}

// Relative logits of one banded key tile for the wave's 32 query columns,
// computed on the matrix cores straight into the wave's own slab in LDS
// ([S-RPB]: R[t, h, e] = r_t . P_h[:, e]), so that R never goes to memory.
// The tile's keys j0..j0+63 meet, over the block's rows, the distances lo =
// p_min - j0 - 63 up to lo + 63 + nrows - 1; they are computed in (at most
// four) tiles of 32 distances from the aligned one holding lo, with
// relproj_kernel's operands in its order (A = packed P^T fragments, B = r,
// k-steps ascending, fp32 accumulation, one rounding to bf16): the slab holds
// rba_relproj's values bit for bit.  Column lc's entry for distance e sits at
// slab[lc * SWD + e - 32 floor(lo / 32)]; distance tiles outside 0..E-1, and
// columns without a query row, hold zeros.  Only this wave reads its slab,
// and LDS operations of one wave complete in order, so no barrier is needed.
template <int FK, int SWD>
__device__ __forceinline__ void bias_tile(const AttnParams &p, __bf16 *slab, int b, int hkv, int t0, int nrows,
                                          int lo, int wave, int lane_in) {
    typedef __bf16 T;
    // the lane's addresses are derived here on every call, not held in
    // registers across the tile loop
    int lane = lane_in;
    asm volatile("" : "+v"(lane));
    const int lc = lane & 31, hh = lane >> 5;
    const int col = wave * 32 + lc;
    const int hl = col / p.QB, qi = col - hl * p.QB;
    const bool valid = col < p.G * p.QB && qi < nrows;
    const int hq = hkv * p.G + min(hl, p.G - 1);
    const int nks = p.r_dim >> 4;
    const int nEB = (p.E + 31) >> 5;
    const int eb_lo = lo >> 5;                                // floor, also for lo < 0
    const int nb = ((lo + 63 + nrows - 1) >> 5) - eb_lo + 1;   // 2..4
    const T *rrow = (const T *)p.rf + (int64_t)b * p.rfs0 + (int64_t)(t0 + (valid ? qi : 0)) * p.rfs1 +
                    (int64_t)hq * p.rfs2 + 8 * hh;
    const int h_lo = (wave * 32) / p.QB;
    const int h_hi = min((wave * 32 + 31) / p.QB, p.G - 1);
    const int hspan = nEB * nks * 512;   // packed entries of one head
    T *dst = slab + lc * SWD + 16 * hh;
    for (int hp = h_lo; hp <= h_hi; ++hp) {
        const rsrc_t rP = make_rsrc((const T *)p.PT + (int64_t)(hkv * p.G + hp) * hspan, (int64_t)hspan * 2);
        // a lane without a query row writes zeros (its B operand is zero) once
        const bool mine = valid ? hl == hp : hp == h_lo;
        // k-steps past r_dim multiply a zero B operand.  Every load is
        // unconditional (k-step clamped to the last one, distance tile into
        // 0..nEB-1, so all stay inside the head's operands) and each wait
        // below covers only the loads it needs; a distance tile outside
        // 0..nEB-1 writes zeros.
        auto load_a = [&](bf16x8 (&a)[FK], int j) __attribute__((always_inline)) {
            const int eb = min(max(eb_lo + j, 0), nEB - 1);
#pragma unroll
            for (int k = 0; k < FK; ++k)
                a[k] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rP, (unsigned)lane * 16, (eb * nks + min(k, nks - 1)) * 1024, 0));
        };
        bf16x8 rfr[FK], a0[FK];
#pragma unroll
        for (int k = 0; k < FK; ++k) rfr[k] = *(const bf16x8 *)(rrow + 16 * min(k, nks - 1));
        load_a(a0, 0);
        __builtin_amdgcn_sched_barrier(0);   // all in flight before the first wait
#pragma unroll
        for (int k = 0; k < FK; ++k) rfr[k] = (valid && k < nks) ? rfr[k] : bf16x8{};
        auto tile = [&](const bf16x8 (&a)[FK], int j) __attribute__((always_inline)) {
            f32x16 acc = f32x16{};
#pragma unroll
            for (int k = 0; k < FK; ++k) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], rfr[k], acc, 0, 0, 0);
            const bool live = eb_lo + j >= 0 && eb_lo + j < nEB;
            if (mine) {
                bf16x8 w0, w1;
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    w0[x] = live ? (__bf16)acc[x] : (__bf16)0.f;
                    w1[x] = live ? (__bf16)acc[8 + x] : (__bf16)0.f;
                }
                *(bf16x8 *)(dst + 32 * j) = w0;
                *(bf16x8 *)(dst + 32 * j + 8) = w1;
            }
        };
        // one register set: each distance tile waits for its own loads
        tile(a0, 0);
#pragma unroll
        for (int j = 1; j < 4; ++j) {
            if (j >= nb) break;
            load_a(a0, j);
            __builtin_amdgcn_sched_barrier(0);   // the tile's four loads in flight together
            tile(a0, j);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// FK = 0: bias rows read from R; FK > 0: computed by bias_rows<FK> into the
// workgroup's region of bias_ws; ONC (FK = 4): each banded tile's bias
// computed by bias_tile into the wave's slab, no R rows in memory at all.
template <int FK, bool ONC = false>
__global__ __launch_bounds__(512, 1) void attn_prefill_pp_kernel(const AttnParams p_arg) {
    typedef const __attribute__((address_space(4))) AttnParams CParams;
    typedef __bf16 T;
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    constexpr int ES = 2;
    constexpr int N = 64;                        // keys per tile
    constexpr int KT = N / 32;
    constexpr int CH = 8;                        // bf16 per 16-byte chunk
    constexpr int SW = N + CH;                   // slab row: the N entries a row needs, chunk-aligned
    constexpr int NCH = SW / CH;
    constexpr int HROWS = 128;                   // slab rows (query columns) of one group
    constexpr int HCH = HROWS * NCH;             // slab chunks of one group
    constexpr int CPR = D * ES / 16;             // 16-byte chunks per K/V row
    constexpr int CPRP = CPR + 1;                // K rows carry one padding chunk
    constexpr int KS = CPRP * CH;
    constexpr int KCH = N * CPRP;
    constexpr int VCH = N * CPR;
    constexpr int GT = 256;                      // threads of the issuing group
    constexpr int NKI = (KCH + GT - 1) / GT;     // 5
    constexpr int NVI = VCH / GT;                // 4
    constexpr int NSI = (HCH + GT - 1) / GT;     // 5 per group half
    constexpr int NSLOT = ONC ? NKI + NVI : NKI + NVI + 2 * NSI;   // DMA instructions per issuing lane and phase
    static_assert(NKI == 5 && NVI * GT == VCH && NSI == 5, "staging split");
    static_assert(!ONC || FK == 4, "the on-chip bias holds four k-steps of r");
    constexpr int SWD = 136;                     // on-chip slab row: four distance tiles + padding
    static_assert(!ONC || 8 * 32 * SWD <= 2 * 2 * NSI * GT * CH, "on-chip slabs fit the bias buffers");

    __shared__ __attribute__((aligned(16))) T sK[2][NKI * GT * CH];
    __shared__ __attribute__((aligned(16))) T sV[2][N * D];
    __shared__ __attribute__((aligned(16))) T sR[2][2][NSI * GT * CH];   // [group][buffer]

    // ------------------------------------------------------------ work item
    const int per_bh = p_arg.nqb * p_arg.splits;
    const int total = p_arg.B * p_arg.Hkv * per_bh;
    // The grid may be smaller than the item count (one workgroup per CU);
    // each workgroup then takes its items round by round.  With grid and
    // item counts multiples of 8 (workgroup w runs on XCD w mod 8), XCD x
    // owns the x-th eighth of the items, longest first, and its workgroups
    // take them in snake order (forward in even rounds, backward in odd
    // ones) so that long and short blocks pair up.
    const bool xcd_map = (total & 7) == 0 && (gridDim.x & 7) == 0;
    const int n8 = total >> 3, nx = gridDim.x >> 3, jx = blockIdx.x >> 3, x8 = blockIdx.x & 7;
    const int n_rounds = xcd_map ? (n8 + nx - 1) / nx : (total - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    for (int rnd = 0; rnd < n_rounds; ++rnd) {
    // The parameters are read afresh in every round (from the constant
    // kernel-argument segment, scalar loads) rather than held in registers
    // across rounds.
#if __HIP_DEVICE_COMPILE__
    CParams *pk = (CParams *)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(pk));
    const AttnParams p = *pk;
#else
    const AttnParams p = p_arg;
#endif
    // Likewise the lane's own indices, so that nothing derived from them is
    // hoisted out of the round loop and held (or spilled) across it.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int grp = wave >> 2;
    const int gw = wave & 3;
    const int hh = lane >> 5;
    const int lc = lane & 31;
    int item;
    if (xcd_map) {
        const int k = rnd * nx + ((rnd & 1) ? nx - 1 - jx : jx);
        if (k >= n8) continue;
        item = x8 * n8 + k;
    } else {
        item = blockIdx.x + rnd * gridDim.x;
    }
    const int bh = item / per_bh;
    const int rem = item - bh * per_bh;
    const int qb = p.nqb - 1 - rem / p.splits;
    const int sp = rem % p.splits;
    const int b = bh / p.Hkv;
    const int hkv = bh - b * p.Hkv;
    const int t0 = qb * p.QB;
    const int nrows = min(p.QB, p.Sq - t0);
    const int pos0 = p.Skv - p.Sq;
    const int p_min = pos0 + t0;
    const int p_max = p_min + nrows - 1;
    const int W = p.window;
    const int lo_key = W > 0 ? max(0, p_min - W + 1) : 0;
    const int kt_lo = lo_key / N;
    const int n_t = p_max / N - kt_lo + 1;
    const int kb = kt_lo + (int)((int64_t)sp * n_t / p.splits);
    const int ke = kt_lo + (int)((int64_t)(sp + 1) * n_t / p.splits);
    const int ncols = p.G * p.QB;
    const bool has_bias = (FK > 0 ? p.rf != nullptr : p.R != nullptr) && p.E > 0;

    const T *__restrict__ gk = (const T *)p.k + (int64_t)b * p.ks0 + (int64_t)hkv * p.ks2;
    const T *__restrict__ gv = (const T *)p.v + (int64_t)b * p.vs0 + (int64_t)hkv * p.vs2;

    // ------------------------------------------------------------ this lane's query column
    const int col = wave * 32 + lc;
    const int hl = col / p.QB;
    const int qi = col - hl * p.QB;
    const bool cvalid = col < ncols && qi < nrows;
    const int tq = t0 + qi;
    const int hq = hkv * p.G + min(hl, p.G - 1);
    const int prow = p_min + qi;
    // log-scale factor, kept > 0 so that masked -inf logits stay -inf
    const float fls = p.inv_ln_base > 0.f ? fmaxf(logf((float)prow + 1.f) * p.inv_ln_base, 1e-30f) : 1.f;
    // q is scaled by amul once per block (scale, log2 e and the row's
    // log-scale factor), so the scores come out of the matrix cores in the
    // exp2 domain; bmul brings the bias there
    const float amul = p.scale_log2e * fls;
    const float bmul = kLog2e * fls;
    const bool wave_active = wave * 32 < ncols;
    const int rb = (prow - N + 1) & ~(CH - 1);

    if constexpr (FK > 0 && !ONC) {
        if (has_bias) {
            if (wave_active)
                bias_rows<FK>(p, (__bf16 *)p.bias_ws + (int64_t)blockIdx.x * p.G * ((p.E + 31) >> 5) * p.QB * 32,
                              b, hkv, t0, nrows, wave, lane);
            // the rows are read back by this workgroup's direct-to-LDS loads
            wait_vmem();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        }
    }

    bf16x8 qf[8];                 // loaded after the first tile's staging is issued

    f32x16 O[4];
    f32x16 S[KT];
    bf16x8 P[2 * KT];
    float m = -INFINITY, l = 0.f;
    float o_scale = 1.f;        // rescale of O owed by the last softmax
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) O[dt] = f32x16{};
#pragma unroll
    for (int i = 0; i < 2 * KT; ++i) P[i] = bf16x8{};

    // ------------------------------------------------------------ staging offsets (lanes of the issuing group)
    // K: LDS chunk L holds chunk L % CPRP of key row lds_key_row(L / CPRP);
    // the padding chunk reloads chunk 0.  Chunks past the tile land in the
    // padding of the buffer.
    const int gl = gw * 64 + lane;               // lane index within the issuing group
    unsigned kvo[NKI];
#pragma unroll
    for (int i = 0; i < NKI; ++i) {
        const int L = i * GT + gl;
        const int R = L / CPRP, pc = L - R * CPRP;
        kvo[i] = (unsigned)((lds_key_row(R & 63) * (int)p.ks1 + (pc < CPR ? pc : 0) * CH) * ES);
    }
    // V: LDS chunk L holds chunk (L % 16) ^ 4 (r % 4) of key row r = L / 16.
    unsigned vvo[NVI];
#pragma unroll
    for (int i = 0; i < NVI; ++i) {
        const int L = i * GT + gl;
        const int r = L >> 4, c = (L & 15) ^ ((r & 3) << 2);
        vvo[i] = (unsigned)((r * (int)p.vs1 + c * CH) * ES);
    }
    // Slab of group g: chunk L holds chunk L % NCH of the bias window of
    // query column g * HROWS + L / NCH; -j0 is added per tile.
    unsigned svo[2][NSI];
    // R rows of this block: from R ([row][head][E] with strides Rs1, Rs2), or
    // from the workgroup's bias region ([head][tile of 32 distances][row][32]).
    // Either way a key tile moves every row's window by a fixed byte step.
    const int nEB = (p.E + 31) >> 5;
    const bool r_vec = FK > 0 ? true : p.r_vec != 0;
    const int64_t region = (int64_t)p.G * nEB * p.QB * 32;
    const T *Rblk = FK > 0 ? (const T *)p.bias_ws + (int64_t)blockIdx.x * region
                           : (const T *)p.R + ((int64_t)b * p.Rs0 + (int64_t)t0 * p.Rs1 + (int64_t)hkv * p.G * p.Rs2);
    const int64_t rspan = FK > 0 ? region * ES
                                 : ((int64_t)(nrows - 1) * p.Rs1 + (int64_t)(p.G - 1) * p.Rs2 + p.E) * ES;
    const int tshift = FK > 0 ? 2 * p.QB * 32 * ES : N * ES;   // bytes per key tile
    const rsrc_t rR = make_rsrc(has_bias ? Rblk : (const T *)p.q, has_bias ? rspan : 0);
    const u32x4 rR4 = make_rsrc_words(has_bias ? Rblk : (const T *)p.q, has_bias ? rspan : 0);
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < NSI; ++i) {
            const int L = i * GT + gl;
            const int row = g * HROWS + L / NCH, ch = L % NCH;
            const int rhl = row / p.QB, rqi = row - rhl * p.QB;
            const bool live = L < HCH && row < ncols && rqi < nrows;
            const int rrb = (p_min + rqi - N + 1) & ~(CH - 1);
            // dead chunks point far past the span: they read zeros
            const int dd = rrb + ch * CH;   // distance of the chunk's first entry at key tile 0
            const int64_t off = FK > 0 ? (((int64_t)rhl * nEB + (dd >> 5)) * p.QB + rqi) * 32 + (dd & 31)
                                       : (int64_t)rqi * p.Rs1 + (int64_t)rhl * p.Rs2 + dd;
            svo[g][i] = live ? (unsigned)(off * ES)
                             : 0x80000000u;
        }

    // ------------------------------------------------------------ tile sequence (banded tiles spread out)
    const int n_it = ke - kb;
    int kband = ke;
    if (has_bias) {
        const int x = p_min - N + 1 - p.E;
        const int first = x < 0 ? 0 : x / N + 1;
        kband = min(max(first, kb), ke);
    }
    const int n_band = ke - kband;
    // iteration i is banded iff floor((i+1) nb / n) > floor(i nb / n); scalar, incremental
    int g_rem = 0, g_cnt = 0, g_idx = 0;
    auto next_tile = [&]() __attribute__((always_inline)) {
        const bool bnd = g_rem + n_band >= n_it;
        const int kt = bnd ? kband + g_cnt : kb + g_idx - g_cnt;
        g_rem += n_band;
        if (g_rem >= n_it) {
            g_rem -= n_it;
            ++g_cnt;
        }
        ++g_idx;
        return kt;
    };
    auto banded = [&](int kt) __attribute__((always_inline)) { return has_bias && (p_min - (kt * N + N - 1) < p.E); };
    // K/V descriptors of a key tile: rows from j0 to the end of the sequence
    // (the host guarantees these spans fit 31 bits).
    const unsigned kstep = (unsigned)(N * (int)p.ks1 * ES), vstep = (unsigned)(N * (int)p.vs1 * ES);
    const unsigned kspan = (unsigned)(((p.Skv - 1) * (int)p.ks1 + D) * ES);
    const unsigned vspan = (unsigned)(((p.Skv - 1) * (int)p.vs1 + D) * ES);
    const u32x4 rk0 = make_rsrc_words(gk, kspan), rv0 = make_rsrc_words(gv, vspan);
    auto tile_rsrc = [&](u32x4 r0, unsigned step, unsigned span, int kt) __attribute__((always_inline)) {
        const unsigned off = (unsigned)kt * step;
        const uint64_t a = ((uint64_t)r0[1] << 32 | r0[0]) + off;
        return u32x4{(unsigned)a, (unsigned)(a >> 32) & 0xffffu, span - off, r0[3]};
    };

    // DMA plan of the current even phase (wave-uniform)
    bool dk = false, dv = false, ds0 = false, ds1 = false;
    int kbuf = 0, vbuf = 0, s0buf = 0, s1buf = 0;
    unsigned s0off = 0, s1off = 0;
    u32x4 rk = rk0, rv = rv0;
    auto issue = [&](int s) __attribute__((always_inline)) {
        if (s < NKI) {
            if (dk) dma16_untracked(rk, kvo[s], &sK[kbuf][(s * GT + gw * 64) * CH]);
        } else if (s < NKI + NVI) {
            const int i = s - NKI;
            if (dv) dma16_untracked(rv, vvo[i], &sV[vbuf][(i * GT + gw * 64) * CH]);
        } else if constexpr (!ONC) {
            if (s < NKI + NVI + NSI) {
                const int i = s - NKI - NVI;
                if (ds0) dma16_untracked(rR4, svo[0][i] + s0off, &sR[0][s0buf][(i * GT + gw * 64) * CH]);
            } else {
                const int i = s - NKI - NVI - NSI;
                if (ds1) dma16_untracked(rR4, svo[1][i] + s1off, &sR[1][s1buf][(i * GT + gw * 64) * CH]);
            }
        }
    };
    // bias rows not 16-byte aligned: element loads through registers
    auto slab_fallback = [&](int g, int buf, int kt) __attribute__((always_inline)) {
        const unsigned eoff = (unsigned)(-kt * N * ES);
#pragma unroll
        for (int i = 0; i < NSI; ++i) {
            u32x4 val = u32x4{};
#pragma unroll
            for (int x = 0; x < CH; ++x)
                val[x >> 1] |= (unsigned)__builtin_amdgcn_raw_buffer_load_b16(rR, svo[g][i] + eoff + x * ES, 0, 0)
                               << (16 * (x & 1));
            *(u32x4 *)&sR[g][buf][(i * GT + gl) * CH] = val;
        }
    };
    // Sets up (and for unaligned bias rows, performs) the staging of even
    // phase 2t: K(t+1), V(t), group 0's bias windows of tile t+1 and group
    // 1's of tile t.  w1, w2 are the key tiles of sequence indices t, t+1.
    auto plan_even = [&](int t, int w1, int w2) __attribute__((always_inline)) {
        dk = t + 1 < n_it;
        kbuf = (t + 1) & 1;
        rk = tile_rsrc(rk0, kstep, kspan, w2);
        dv = t >= 1 && t < n_it;
        vbuf = t & 1;
        rv = tile_rsrc(rv0, vstep, vspan, w1);
        ds0 = t + 1 < n_it && banded(w2);
        s0buf = (t + 1) & 1;
        s0off = (unsigned)(-w2 * tshift);
        ds1 = t < n_it && banded(w1);
        s1buf = t & 1;
        s1off = (unsigned)(-w1 * tshift);
        if (!r_vec) {
            if (ds0) slab_fallback(0, s0buf, w2);
            if (ds1) slab_fallback(1, s1buf, w1);
            ds0 = ds1 = false;
        }
    };

    // ------------------------------------------------------------ phase work
    const int kr0 = lds_key_row(mfma_row_key(lc));
    const int s_lane = (col - grp * HROWS) * SW + (prow - rb) - 16 * hh;
    // on-chip bias: the wave's slab, and the lane's entry offset in it (the
    // same for every key tile: 32 floor((p_min - 63 - j0) / 32) + j0 is fixed)
    T *const sB = &sR[0][0][0] + wave * 32 * SWD;
    const int s_lane_b = lc * SWD + (prow - (((p_min - (N - 1)) >> 5) << 5)) - 16 * hh;
    // V^T fragment of PV step (u, h2, dt): two transpose reads of 4 keys each.
    // Lane (g = lane / 16, a = lane % 4, i = lane / 4 % 4) addresses key row
    // 32u + 16(g / 2) + 8h2 + 4x + i and head-dim entries 32dt + 16(g % 2) + 4a,
    // and receives key rows of one head-dim entry back.
    const int tr_i = (lane >> 2) & 3;
    int vt_off[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
        vt_off[dt] = (16 * hh + tr_i) * D + CH * ((((dt ^ tr_i) << 2) | (((lane >> 4) & 1) << 1) | ((lane >> 1) & 1))) +
                     4 * (lane & 1);

    // Matrix phase: the 16 PV steps of tile tp, then the 16 QK^T steps of
    // tile tqk, one MFMA per step, A-operand fragments read LA steps ahead;
    // with DMA, one staging instruction is issued per step.
    auto mfma_phase = [&](int tp, int tqk, auto dma_c) __attribute__((always_inline)) {
        constexpr bool DMA = decltype(dma_c)::value;
        constexpr int LA = 6;
        const T *vb = &sV[tp & 1][0];
        const T *kb_ = &sK[tqk & 1][kr0 * KS];
        auto trv = [&](const T *ptr) __attribute__((always_inline)) {
            return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t *)ptr);
        };
        auto frag = [&](int st) __attribute__((always_inline)) {
            if (st < 16) {   // PV step: sub-tile u = st / 8, half h2 = (st / 4) & 1, dims dt = st & 3
                const T *base = vb + vt_off[st & 3] + (32 * (st >> 3) + 8 * ((st >> 2) & 1)) * D;
                const bf16x4_t lo = trv(base), hi = trv(base + 4 * D);
                return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            const int q = st - 16;   // QK step: k-step q / 2, sub-tile q & 1
            return *(const bf16x8 *)(kb_ + (q & 1) * 32 * KS + 16 * (q >> 1) + 8 * hh);
        };
        bf16x8 fr[32];
#pragma unroll
        for (int st = 0; st < LA; ++st) fr[st] = frag(st);
        if (__builtin_amdgcn_ballot_w64(o_scale != 1.f) != 0) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) O[dt] *= o_scale;
        }
#pragma unroll
        for (int st = 0; st < 32; ++st) {
            if (st + LA < 32) fr[st + LA] = frag(st + LA);
            if constexpr (DMA) {
                if (st < NSLOT) issue(st);
            }
            if (st < 16) {
                O[st & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[st], P[st >> 2], O[st & 3], 0, 0, 0);
            } else {
                const int q = st - 16;
                // scores start at -m0 (m0: the reference max, 0 before the
                // column's first visible tile), so exp2(S) needs no subtraction
                if (q < KT) S[q] = f32x16{} - (m == -INFINITY ? 0.f : m);
                S[q & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[st], qf[q >> 1], S[q & 1], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Vector phase: bias, mask, running max and exponentials of tile t
    // (sequence index), key tile kt.
    // With DMA the group issues this phase's staging instructions in one burst
    // at its start (FK = 0) or in four bursts spread over the softmax.
    auto softmax = [&](int t, int kt, auto dma_c) __attribute__((always_inline)) {
        constexpr bool DMA = decltype(dma_c)::value;
        auto burst = [&](int s0, int s1) __attribute__((always_inline)) {
            if constexpr (DMA) {
#pragma unroll
                for (int s = s0; s < s1; ++s) issue(s);
            }
        };
        const int j0 = kt * N;
        const bool band = banded(kt);
        if constexpr (ONC) {
            if (band) bias_tile<FK, SWD>(p, sB, b, hkv, t0, nrows, p_min - j0 - (N - 1), wave, lane);
        }
        // the kernel reading R: all in one burst (full causal 29.29 -> 29.01 ms,
        // A/B); the fused variants keep four bursts spread over the softmax
        // (one burst made them 1-2 % slower)
        burst(0, FK == 0 ? NSLOT : 6);
        const bool edge = !((j0 + N - 1 <= p_min) && (W == 0 || p_max - j0 < W));
        float mt = -INFINITY;
        if (band || edge) {
            int slb = s_lane_b;
            if constexpr (ONC) asm volatile("" : "+v"(slb));   // one address register, offsets folded in
            const T *sr = ONC ? sB + slb : &sR[grp][t & 1][s_lane];
            const bool partial = p_max - j0 >= p.E;
            const int elim = prow - j0 - 16 * hh - p.E;   // key offset r of a half has e < E iff r > elim
            const int dbase = prow - j0 - 16 * hh;        // distance of key offset 0 of this half
#pragma unroll
            for (int u = 0; u < KT; ++u) {
                if (band) {
                    // entries r = 0..7 of sub-tile u are the 8 bf16 ending at
                    // sr - 32u (reversed), r = 8..15 the 8 ending at sr - 32u - 8;
                    // added in the unscaled domain (s + bias / scale), scaled
                    // with the dot product in the exponent below
                    bf16x8 braw[2];
#pragma unroll
                    for (int h8 = 0; h8 < 2; ++h8) __builtin_memcpy(&braw[h8], sr - 32 * u - 8 * h8 - 7, 16);
                    if (partial) {
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            S[u][r] = fmaf(32 * u + r > elim ? (float)braw[r >> 3][7 - (r & 7)] : 0.f, bmul, S[u][r]);
                    } else {
#pragma unroll
                        for (int r = 0; r < 16; ++r) S[u][r] = fmaf((float)braw[r >> 3][7 - (r & 7)], bmul, S[u][r]);
                    }
                }
                if (edge) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int dist = dbase - 32 * u - r;
                        const bool vis = dist >= 0 && (W == 0 || dist < W);
                        S[u][r] = vis ? S[u][r] : -INFINITY;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (FK != 0) burst(6, 11);
        // Probabilities against the current reference max m (exp2 domain),
        // rounded to bf16 for the PV product; the row sum adds the fp32 values
        // in two chains.  (A v_dot2c sum over the bf16 values keeps numerator
        // and denominator on the same rounding, but those instructions stall
        // next to the other wave's MFMAs; full-causal workload 31.0 -> 30.2 ms.)
        // S holds scores minus m0 in the exp2 domain (see the matrix phase)
        const float m0 = m == -INFINITY ? 0.f : m;
        float sum = 0.f;
        // mu: the reference max the probabilities are taken against, as a
        // shift from m0 (0 on the first pass)
        auto exps = [&](float mu, auto dma_b) __attribute__((always_inline)) {
            constexpr bool DB = decltype(dma_b)::value;
            float sm[2] = {0.f, 0.f};
#pragma unroll
            for (int u = 0; u < KT; ++u)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    bf16x8 pb;
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        const float e = fast_exp2(S[u][8 * h2 + x] - mu);   // mu = 0.f folds away
                        pb[x] = (__bf16)e;
                        sm[x & 1] += e;
                    }
                    P[2 * u + h2] = pb;
                    if constexpr (DB && FK != 0) {
                        if (u == 0 && h2 == 0) burst(11, 15);
                        if (u == 0 && h2 == 1) burst(15, NSLOT);
                    }
                }
            sum = sm[0] + sm[1];
        };
        exps(0.f, std::integral_constant<bool, DMA>{});
        o_scale = 1.f;
        // The reference max m only moves when the tile max exceeds it by more
        // than kRescaleSlack.  While the lane's probabilities sum to at most
        // 2^kRescaleSlack none of them exceeds that bound, so the tile max is
        // not needed (an overflow makes the sum inf, a NaN fails the test);
        // otherwise, and at a column's first visible tile, it is taken as
        // before and, if m moves, O and l are rescaled and P recomputed.
        // Wave-uniform, so both halves of a column decide alike.
        const bool slow = !(sum <= kRescaleLimit) || m == -INFINITY;
        if (__builtin_amdgcn_ballot_w64(slow) != 0) {
#pragma unroll
            for (int u = 0; u < KT; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt = fmaxf(mt, S[u][r]);
            mt += m0;
            mt = max_across_halves(mt);
            const bool grow = mt > m + kRescaleSlack;
            const float mn = grow ? mt : m;
            const float alpha = m == -INFINITY ? 0.f : (grow ? fast_exp2(m - mn) : 1.f);
            m = mn;
            l *= alpha;
            o_scale = alpha;        // applied to O at the start of the next matrix phase
            if (__builtin_amdgcn_ballot_w64(grow) != 0) exps((m == -INFINITY ? 0.f : m) - m0, std::false_type{});
        }
        l += sum;
    };

    // ------------------------------------------------------------ prologue: first tile
    int w0 = 0, w1 = 0, w2 = 0;     // key tiles of sequence indices t-1, t, t+1
    if (n_it > 0) {
        w1 = next_tile();
        w2 = n_it > 1 ? next_tile() : 0;
        if (grp == 0) {
            // K(0), V(0) and group 0's bias windows of tile 0
            dk = dv = true;
            rk = tile_rsrc(rk0, kstep, kspan, w1);
            rv = tile_rsrc(rv0, vstep, vspan, w1);
            ds0 = banded(w1);
            s0off = (unsigned)(-w1 * tshift);
            if (ds0 && !r_vec) {
                slab_fallback(0, 0, w1);
                ds0 = false;
            }
#pragma unroll
            for (int s = 0; s < NKI + NVI + NSI; ++s) issue(s);
        }
    }
    // Q fragments, in flight together with the first tile's staging.  Settle
    // them here: otherwise the compiler's wait for them sits inside the phase
    // loop, where it would also wait for the DMA.  vmcnt counts in order, so
    // the wait for Q also lands the staging.
    {
        const T *qp = (const T *)p.q + (int64_t)b * p.qs0 + (int64_t)tq * p.qs1 + (int64_t)hq * p.qs2;
#pragma unroll
        for (int k = 0; k < 8; ++k) qf[k] = cvalid ? *(const bf16x8 *)(qp + 16 * k + 8 * hh) : bf16x8{};
#pragma unroll
        for (int k = 0; k < 8; ++k) asm volatile("" : "+v"(qf[k]));
    }
    wait_vmem();
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int x = 0; x < 8; ++x) qf[k][x] = (__bf16)((float)qf[k][x] * amul);
    lds_barrier();

    // ------------------------------------------------------------ phases 2t, 2t+1 for t = 0..n_it
    auto run = [&](auto grp_c) __attribute__((always_inline)) {
        constexpr int G = decltype(grp_c)::value;
        for (int t = 0; t <= n_it && n_it > 0; ++t) {
            if (t > 0) {          // slide the window to t-1, t, t+1
                w0 = w1;
                w1 = w2;
                w2 = t + 1 < n_it ? next_tile() : 0;
            }
            // even phase
            if constexpr (G == 0) {
                // P is zero before the first softmax (PV then adds nothing;
                // V buffer 0 holds the first tile); the QK after the last
                // tile is never used.
                mfma_phase(t >= 1 ? t - 1 : 0, t, std::false_type{});
            } else {
                // group 1 stages the tiles of this even phase while it runs
                // its softmax (the matrix group's phase is the longer one)
                plan_even(t, w1, w2);
                if (wave_active && t >= 1) {
                    softmax(t - 1, w0, std::true_type{});
                } else {
#pragma unroll
                    for (int s = 0; s < NSLOT; ++s) issue(s);
                }
            }
            lds_barrier();
            // odd phase
            if constexpr (G == 0) {
                if (t < n_it) softmax(t, w1, std::false_type{});
            } else {
                if (wave_active) mfma_phase(t >= 1 ? t - 1 : 0, t, std::false_type{});
                wait_vmem();      // staging of the even phase has landed
            }
            lds_barrier();
        }
    };
    if (grp == 0)
        run(std::integral_constant<int, 0>{});
    else
        run(std::integral_constant<int, 1>{});

    // ------------------------------------------------------------ epilogue
    const float lt = l + __shfl_xor(l, 32);
    if (cvalid) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_v = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
    if (p.splits == 1) {
        T *op = (T *)p.o + (int64_t)b * p.os0 + (int64_t)tq * p.os1 + (int64_t)hq * p.os2;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 w;
#pragma unroll
                for (int x = 0; x < 4; ++x) w[x] = (__bf16)(O[dt][4 * g4 + x] * inv);
                *(bf16x4 *)(op + 32 * dt + 8 * g4 + 4 * hh) = w;
            }
        if (p.lse != nullptr && hh == 0) p.lse[((int64_t)b * p.Hq + hq) * p.Sq + tq] = lse_v;
    } else {
        const int64_t row = (((int64_t)sp * p.B + b) * p.Sq + tq) * p.Hq + hq;
        float *op = p.o_part + row * D;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 w;
#pragma unroll
                for (int x = 0; x < 4; ++x) w[x] = O[dt][4 * g4 + x] * inv;
                *(f32x4 *)(op + 32 * dt + 8 * g4 + 4 * hh) = w;
            }
        if (hh == 0) p.lse_part[row] = lse_v;
    }
    }  // cvalid
    }  // work items
}

// Split-KV merge.  32 lanes cover one output row (4 head-dim entries each);
// SG groups of 32 lanes share a row and each merge every SG-th split, then
// the groups' partial (max, sum, weighted output) are merged through LDS.
// SG = 8 serves few rows with many splits (long-context decode), SG = 1 many
// rows with few splits.
template <typename TO, int SG>
__global__ __launch_bounds__(NT) void combine_kernel(const float *__restrict__ o_part,
                                                     const float *__restrict__ lse_part, int splits, int B, int Sq,
                                                     int Hq, TO *__restrict__ o, int64_t os0, int64_t os1,
                                                     int64_t os2, float *__restrict__ lse) {
    constexpr int RPB = NT / 32 / SG;   // rows per block
    __shared__ float part[SG > 1 ? NT / 32 : 1][2 + 32 * 4];
    const int64_t rows = (int64_t)B * Sq * Hq;
    const int g32 = threadIdx.x >> 5;   // 32-lane group
    const int grp = g32 % SG;           // split group of the row
    const int64_t row = (int64_t)blockIdx.x * RPB + g32 / SG;
    const int c = threadIdx.x & 31;
    const bool live = row < rows;
    float M = -INFINITY;
    if (live) {
#pragma unroll 4
        for (int s = grp; s < splits; s += SG) M = fmaxf(M, lse_part[s * rows + row]);
    }
    const float Ms = M == -INFINITY ? 0.f : M;
    f32x4 acc = f32x4{};
    float den = 0.f;
    if (live) {
#pragma unroll 4
        for (int s = grp; s < splits; s += SG) {
            const float w = fast_exp2((lse_part[s * rows + row] - Ms) * kLog2e);
            den += w;
            const f32x4 x = *(const f32x4 *)(o_part + (s * rows + row) * D + 4 * c);
            acc += w * x;
        }
    }
    float Mt = M;
    if constexpr (SG > 1) {
        float *mine = part[g32];
        if (c == 0) {
            mine[0] = M;
            mine[1] = den;
        }
        *(f32x4 *)&mine[2 + 4 * c] = acc;
        __syncthreads();
        if (grp != 0) return;
        Mt = -INFINITY;
#pragma unroll
        for (int g = 0; g < SG; ++g) Mt = fmaxf(Mt, part[g32 + g][0]);
        acc = f32x4{};
        den = 0.f;
#pragma unroll
        for (int g = 0; g < SG; ++g) {
            const float *pg = part[g32 + g];
            const float w = pg[0] == -INFINITY ? 0.f : fast_exp2((pg[0] - Mt) * kLog2e);
            den += w * pg[1];
            acc += w * *(const f32x4 *)&pg[2 + 4 * c];
        }
    }
    if (!live) return;
    const float Mf = Mt == -INFINITY ? 0.f : Mt;
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const int h = (int)(row % Hq);
    const int64_t bt = row / Hq;
    const int t = (int)(bt % Sq);
    const int b = (int)(bt / Sq);
    TO *op = o + (int64_t)b * os0 + (int64_t)t * os1 + (int64_t)h * os2 + 4 * c;
#pragma unroll
    for (int x = 0; x < 4; ++x) op[x] = (TO)(acc[x] * inv);
    if (lse != nullptr && c == 0) lse[((int64_t)b * Hq + h) * Sq + t] = den > 0.f ? Mf + logf(den) : -INFINITY;
}

}  // namespace

// Grid of the persistent prefill kernel: one workgroup per CU (a multiple
// of 8, so the XCD-aware item order holds) when the items outnumber the CUs
// and split evenly over the 8 XCDs; else one workgroup per item.
static int pp_grid(int64_t items) {
    static std::atomic<int> cus_of[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return (int)items;
    int cus = cus_of[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return (int)items;
        cus_of[dev].store(cus, std::memory_order_relaxed);
    }
    const int g = cus & ~7;
    return (items % 8 == 0 && g >= 8 && items > g) ? g : (int)items;
}

int fused_grid(int64_t items, int cus) {
    const int64_t g = cus >= 8 ? (cus & ~7) : std::max(cus, 1);
    return (int)std::min<int64_t>(items, g);
}

hipError_t launch_attention_fused(const AttnParams &p, int grid, hipStream_t stream) {
    if (p.bias_ws == nullptr) {   // the bias of each banded tile computed into LDS (r_dim <= 64)
        const int64_t items = (int64_t)p.B * p.Hkv * p.nqb;
        if (items <= 0) return hipSuccess;
        hipLaunchKernelGGL((attn_prefill_pp_kernel<4, true>), dim3(pp_grid(items)), dim3(512), 0, stream, p);
        return hipGetLastError();
    }
    if (grid <= 0) return hipSuccess;
    if (p.r_dim <= 64)
        hipLaunchKernelGGL(attn_prefill_pp_kernel<4>, dim3(grid), dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL(attn_prefill_pp_kernel<8>, dim3(grid), dim3(512), 0, stream, p);
    return hipGetLastError();
}

int attn_max_columns(AttnVariant v) { return v == AttnVariant::BF16_WIDE ? 256 : 128; }

hipError_t launch_attention(const AttnParams &p, AttnVariant v, hipStream_t stream) {
    const int64_t blocks = (int64_t)p.B * p.Hkv * p.nqb * p.splits;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    const bool paged = p.block_table != nullptr;
    const bool f8 = p.k_scale != nullptr;
    // K/V in plain bf16 or fp32 (the pp kernel needs 32-bit K/V offsets), or MXFP8
#define RBA_FWD(T, NW, SLAB2, PG, F8)                                                                   \
    hipLaunchKernelGGL((attn_fwd_kernel<T, NW, SLAB2, PG, F8>), grid, dim3(64 * NW), 0, stream, p)
#define RBA_FWDQ(NW, SLAB2, PG)                                                                         \
    hipLaunchKernelGGL((attn_fwd_kernel<__bf16, NW, SLAB2, PG, true, true>), grid, dim3(64 * NW), 0, stream, p)
#define RBA_FWDV(PG)                                                                                    \
    hipLaunchKernelGGL((attn_fwd_kernel<__bf16, 4, false, PG, false, false, true>), grid, dim3(256), 0, stream, p)
    const bool vd = p.G * p.QB <= 96;
    const bool fq = f8 && p.qk8;
    switch (v) {
        case AttnVariant::BF16_WIDE:    // 8 waves, 256 columns
            if (fq && paged)
                RBA_FWDQ(8, true, true);
            else if (fq)
                RBA_FWDQ(8, true, false);
            else if (f8 && paged)
                RBA_FWD(__bf16, 8, true, true, true);
            else if (f8)
                RBA_FWD(__bf16, 8, true, false, true);
            else if (paged)
                RBA_FWD(__bf16, 8, true, true, false);
            else if (p.kv32)            // two ping-pong groups, one workgroup per CU
                hipLaunchKernelGGL(attn_prefill_pp_kernel<0>, dim3(pp_grid(blocks)), dim3(512), 0, stream, p);
            else
                RBA_FWD(__bf16, 8, true, false, false);
            break;
        case AttnVariant::BF16_NARROW:  // 4 waves: 128 columns, small LDS footprint
            if (fq && paged)
                RBA_FWDQ(4, false, true);
            else if (fq)
                RBA_FWDQ(4, false, false);
            else if (f8 && paged && vd)
                hipLaunchKernelGGL((attn_fwd_kernel<__bf16, 4, false, true, true, false, true>), grid, dim3(256), 0,
                                   stream, p);
            else if (f8 && vd)
                hipLaunchKernelGGL((attn_fwd_kernel<__bf16, 4, false, false, true, false, true>), grid, dim3(256), 0,
                                   stream, p);
            else if (f8 && paged)
                RBA_FWD(__bf16, 4, false, true, true);
            else if (f8)
                RBA_FWD(__bf16, 4, false, false, true);
            else if (paged && vd)
                RBA_FWDV(true);
            else if (paged)
                RBA_FWD(__bf16, 4, false, true, false);
            else if (vd)
                RBA_FWDV(false);
            else
                RBA_FWD(__bf16, 4, false, false, false);
            break;
        case AttnVariant::FP32:         // MXFP8 K/V is bf16-only (rejected by the caller)
            if (f8) return hipErrorInvalidValue;
            if (paged)
                RBA_FWD(float, 4, false, true, false);
            else
                RBA_FWD(float, 4, false, false, false);
            break;
    }
#undef RBA_FWD
#undef RBA_FWDQ
#undef RBA_FWDV
    return hipGetLastError();
}

hipError_t launch_combine(const float *o_part, const float *lse_part, int splits, int B, int Sq, int Hq, void *o,
                          bool o_bf16, int64_t os0, int64_t os1, int64_t os2, float *lse, hipStream_t stream) {
    const int64_t rows = (int64_t)B * Sq * Hq;
    if (rows <= 0) return hipSuccess;
    // few rows: one row per block, the splits spread over 8 lane groups
    const bool wide = rows < 8192 && splits >= 8;
    const int64_t blocks = wide ? rows : (rows + 7) / 8;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks), block(NT);
    if (o_bf16) {
        if (wide)
            hipLaunchKernelGGL((combine_kernel<__bf16, 8>), grid, block, 0, stream, o_part, lse_part, splits, B, Sq, Hq,
                               (__bf16 *)o, os0, os1, os2, lse);
        else
            hipLaunchKernelGGL((combine_kernel<__bf16, 1>), grid, block, 0, stream, o_part, lse_part, splits, B, Sq, Hq,
                               (__bf16 *)o, os0, os1, os2, lse);
    } else {
        if (wide)
            hipLaunchKernelGGL((combine_kernel<float, 8>), grid, block, 0, stream, o_part, lse_part, splits, B, Sq, Hq,
                               (float *)o, os0, os1, os2, lse);
        else
            hipLaunchKernelGGL((combine_kernel<float, 1>), grid, block, 0, stream, o_part, lse_part, splits, B, Sq, Hq,
                               (float *)o, os0, os1, os2, lse);
    }
    return hipGetLastError();
}

// Split-KV workspace of rba_attn_decode_noalloc: a file-scope device array of
// RBA_DECODE_SCRATCH_BYTES.  Every device the library runs on holds its own
// copy until the process ends, and every call on that device shares it.  In
// host code the name `scratch` is only a stand-in for the symbol, not a
// device address: host code uses the address scratch_address() looks up once
// per device (with that device current), never the name itself.
static __device__ __align__(256) float scratch[RBA_DECODE_SCRATCH_BYTES / sizeof(float)];

hipError_t scratch_address(void **out) {
    static std::mutex mu;
    static void *addr[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = ptr;
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace rba
