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
// Design (one kernel serves prefill and split-KV decode):
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

constexpr int D = 128;                // head size
constexpr int NT = 256;               // threads per workgroup of the combine kernel
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;  // log2 growth of the running max tolerated before O is rescaled

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

template <typename T, int NW, bool SLAB2>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_fwd_kernel(const AttnParams p) {
    using TL = Tile<T>;
    constexpr bool BF = sizeof(T) == 2;
    constexpr int ES = (int)sizeof(T);
    constexpr int NTH = 64 * NW;                 // threads per workgroup
    constexpr int N = TL::N;
    constexpr int KT = N / 32;                   // 32-key sub-tiles per tile
    constexpr int CH = TL::CH;
    constexpr int VS = TL::VS;
    constexpr int SW = TL::SW;
    constexpr int NCH = SW / CH;                 // chunks per slab row
    constexpr int SROWS = NW * 32;               // slab rows = max columns per workgroup
    constexpr int SCH = SROWS * NCH;             // slab chunks
    constexpr int NSI = (SCH + NTH - 1) / NTH;   // slab DMA instructions per thread
    constexpr int CPR = D * ES / 16;             // 16-byte chunks per K/V row
    constexpr int CPRP = CPR + 1;                // with the padding chunk
    constexpr int KS = CPRP * CH;                // K row stride in LDS (elements)
    constexpr int KCH = N * CPRP;                // K chunks per tile incl. padding
    constexpr int NKI = (KCH + NTH - 1) / NTH;   // K DMA instructions per thread
    constexpr int NVI = BF ? N * D / (NTH * 4) : N * CPR / NTH;  // V loads per thread
    constexpr int NSB = SLAB2 ? 2 : 1;
    static_assert(NVI * NTH * (BF ? 4 : CH) == N * D, "V tile must split evenly over threads");

    __shared__ __attribute__((aligned(16))) T sK[2][N * KS];
    __shared__ __attribute__((aligned(16))) T sV[TL::VROWS * VS];
    __shared__ __attribute__((aligned(16))) T sR[NSB][SROWS * SW];

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
    const bool has_bias = p.R != nullptr && p.E > 0;

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
    constexpr int QREGS = BF ? 8 : 64;
    typedef typename std::conditional<BF, bf16x8, float>::type QFrag;
    QFrag qf[QREGS];
    {
        const T *qp = (const T *)p.q + (int64_t)b * p.qs0 + (int64_t)tq * p.qs1 + (int64_t)hq * p.qs2;
        if constexpr (BF) {
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
    unsigned vvo[NVI];
#pragma unroll
    for (int i = 0; i < NVI; ++i) {
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
    {
        const int64_t rbase = (int64_t)b * p.Rs0 + (int64_t)t0 * p.Rs1 + (int64_t)hkv * p.G * p.Rs2;
        const int64_t rspan = ((int64_t)(nrows - 1) * p.Rs1 + (int64_t)(p.G - 1) * p.Rs2 + p.E) * ES;
        rR = make_rsrc(has_bias ? (const T *)p.R + rbase : (const T *)p.q, has_bias ? rspan : 0);
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

    auto banded = [&](int kt) { return has_bias && (p_min - (kt * N + N - 1) < p.E); };

    auto kv_rsrc = [&](const T *g, int64_t stride, int j0) {
        return make_rsrc(g + (int64_t)j0 * stride, ((int64_t)(p.Skv - 1 - j0) * stride + D) * ES);
    };

    auto stage_k = [&](int kt, int buf) {
        const rsrc_t rk = kv_rsrc(gk, p.ks1, kt * N);
#pragma unroll
        for (int i = 0; i < NKI; ++i) {
            const int wc = (i * NW + wave) * 64;
            if (i < NKI - 1 || wc + lane < KCH) dma16(rk, kvo[i], &sK[buf][wc * CH]);
        }
    };

    auto load_v = [&](int kt) {
        const rsrc_t rv = kv_rsrc(gv, p.vs1, kt * N);
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

    // ------------------------------------------------------------ one key tile
    const int kr0 = lds_key_row(mfma_row_key(lc));   // LDS row of this lane's A-operand key (+32: sub-tile 1)
    const T *k_lane = &sK[0][kr0 * KS];
    const T *v_lane = BF ? &sV[lc * VS + 16 * hh] : &sV[16 * hh * VS + lc];
    const int s_lane = col * SW + (prow - rb) - 16 * hh;   // slab entry of key offset 16*hh

    auto compute_tile = [&](int kt, int buf, int sbuf) {
        const int j0 = kt * N;
        f32x16 S[KT];
#pragma unroll
        for (int u = 0; u < KT; ++u) S[u] = f32x16{};

        // S^T = K . Q^T
        const T *kb_ = k_lane + buf * (N * KS);
        if constexpr (BF) {
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

        float mt = -INFINITY;
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
#pragma unroll
            for (int u = 0; u < KT; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt = fmaxf(mt, S[u][r]);
        } else {
            // raw dot products; the scale is applied inside the exponent
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
#pragma unroll
            for (int u = 0; u < KT; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt = fmaxf(mt, S[u][r]);
            mt *= amul;
        }

        // online softmax (exp2 domain).  The reference max only moves when the
        // tile max exceeds it by more than kRescaleSlack; O and l are rescaled
        // only when some lane of the wave moves it.  Exact: numerator and
        // denominator always share the reference.
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const bool grow = mt > m + kRescaleSlack;
        if (__ballot(grow) != 0) {
            const float mn = grow ? mt : m;
            const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mn);
            m = mn;
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) O[dt] *= alpha;
        }
        const float mu = m == -INFINITY ? 0.f : m;
        const float sa = band ? 1.f : amul;     // multiplier still to apply to S
#pragma unroll
        for (int u = 0; u < KT; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) S[u][r] = fast_exp2(fmaf(S[u][r], sa, -mu));

        // O^T += V^T . P^T ; the row sum uses the same rounded P as the product
        if constexpr (BF) {
            float sum = 0.f;
#pragma unroll
            for (int u = 0; u < KT; ++u) {
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    bf16x8 pb;
#pragma unroll
                    for (int x = 0; x < 8; ++x) pb[x] = (__bf16)S[u][8 * h2 + x];
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        sum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[2 * x], pb[2 * x + 1]},
                                                              bf16x2{(__bf16)1.f, (__bf16)1.f}, sum, false);
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) {
                        const bf16x8 a = *(const bf16x8 *)(v_lane + 32 * dt * VS + 32 * u + 8 * h2);
                        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, O[dt], 0, 0, 0);
                    }
                }
            }
            l += sum;
        } else {
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

    int kt = n_it > 0 ? next_tile() : 0;
    if (n_it > 0) {
        stage_k(kt, 0);
        load_v(kt);
        if (banded(kt)) stage_slab(kt, 0);
        store_v();
        wait_vmem();
    }
    __syncthreads();
    for (int it = 0; it < n_it; ++it) {
        const int cur = it & 1;
        const bool nxt = it + 1 < n_it;
        const int kn = nxt ? next_tile() : kt;
        if (nxt) {
            stage_k(kn, cur ^ 1);
            load_v(kn);
            if (SLAB2 && banded(kn)) stage_slab(kn, cur ^ 1);
        }
        if (wave_active) compute_tile(kt, cur, SLAB2 ? cur : 0);
        wait_vmem();
        __syncthreads();             // tile kt fully consumed; loads for kn landed
        if (nxt) {
            store_v();
            if (!SLAB2 && banded(kn)) {
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

// Split-KV merge.  32 threads per output row, 4 head-dim entries each.
template <typename TO>
__global__ __launch_bounds__(NT) void combine_kernel(const float *__restrict__ o_part,
                                                     const float *__restrict__ lse_part, int splits, int B, int Sq,
                                                     int Hq, TO *__restrict__ o, int64_t os0, int64_t os1,
                                                     int64_t os2, float *__restrict__ lse) {
    const int64_t rows = (int64_t)B * Sq * Hq;
    const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    const int c = threadIdx.x & 31;
    if (row >= rows) return;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, lse_part[s * rows + row]);
    const float Ms = M == -INFINITY ? 0.f : M;
    f32x4 acc = f32x4{};
    float den = 0.f;
    for (int s = 0; s < splits; ++s) {
        const float w = fast_exp2((lse_part[s * rows + row] - Ms) * kLog2e);
        den += w;
        const f32x4 x = *(const f32x4 *)(o_part + (s * rows + row) * D + 4 * c);
        acc += w * x;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const int h = (int)(row % Hq);
    const int64_t bt = row / Hq;
    const int t = (int)(bt % Sq);
    const int b = (int)(bt / Sq);
    TO *op = o + (int64_t)b * os0 + (int64_t)t * os1 + (int64_t)h * os2 + 4 * c;
#pragma unroll
    for (int x = 0; x < 4; ++x) op[x] = (TO)(acc[x] * inv);
    if (lse != nullptr && c == 0) lse[((int64_t)b * Hq + h) * Sq + t] = den > 0.f ? Ms + logf(den) : -INFINITY;
}

}  // namespace

int attn_max_columns(AttnVariant v) { return v == AttnVariant::BF16_WIDE ? 256 : 128; }

hipError_t launch_attention(const AttnParams &p, AttnVariant v, hipStream_t stream) {
    const int64_t blocks = (int64_t)p.B * p.Hkv * p.nqb * p.splits;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    switch (v) {
        case AttnVariant::BF16_WIDE:    // 8 waves, 256 columns, two bias slab buffers
            hipLaunchKernelGGL((attn_fwd_kernel<__bf16, 8, true>), grid, dim3(512), 0, stream, p);
            break;
        case AttnVariant::BF16_NARROW:  // 4 waves: 128 columns, small LDS footprint
            hipLaunchKernelGGL((attn_fwd_kernel<__bf16, 4, false>), grid, dim3(256), 0, stream, p);
            break;
        case AttnVariant::FP32:
            hipLaunchKernelGGL((attn_fwd_kernel<float, 4, false>), grid, dim3(256), 0, stream, p);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_combine(const float *o_part, const float *lse_part, int splits, int B, int Sq, int Hq, void *o,
                          bool o_bf16, int64_t os0, int64_t os1, int64_t os2, float *lse, hipStream_t stream) {
    const int64_t rows = (int64_t)B * Sq * Hq;
    if (rows <= 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + 7) / 8)), block(NT);
    if (o_bf16)
        hipLaunchKernelGGL((combine_kernel<__bf16>), grid, block, 0, stream, o_part, lse_part, splits, B, Sq, Hq,
                           (__bf16 *)o, os0, os1, os2, lse);
    else
        hipLaunchKernelGGL((combine_kernel<float>), grid, block, 0, stream, o_part, lse_part, splits, B, Sq, Hq,
                           (float *)o, os0, os1, os2, lse);
    return hipGetLastError();
}

}  // namespace rba
