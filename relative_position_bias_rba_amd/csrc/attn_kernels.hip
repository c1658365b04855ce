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
//  * A workgroup (4 waves) owns one (batch, kv head, block of QB query rows,
//    key-range split) and all G query heads of that kv head: its G*QB query
//    columns all read the K/V tiles it stages in LDS once (the GQA group loop).
//  * Scores are computed transposed, S^T = K . Q^T, with
//    v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator a lane owns one query
//    column and 16 of the 32 keys; the A-operand rows are permuted so those 16
//    keys are consecutive.  Row max/sum need one cross-half exchange, the bias
//    for 16 consecutive keys is 16 consecutive (reversed) entries of one R row,
//    and the probabilities feed the PV product (O^T = V^T . P^T) as the
//    B operand straight from registers.
//  * For key tiles whose smallest distance is below E, the R rows of the
//    block's columns are staged in LDS (the entries that tile can touch) and
//    each lane gathers its bias by diagonal offset p - j.  Other tiles skip
//    the bias entirely; tiles wholly inside the causal/window band skip the
//    mask; tiles outside it are never visited.
//  * Online softmax in the exp2 domain with fp32 state; bf16 P for PV.
//  * Work items are ordered longest-first and laid out so that each of the 8
//    XCDs processes contiguous (batch, kv head) ranges, keeping their K/V in
//    that XCD's L2.
#include "rba_internal.h"

#include <type_traits>

#include <math.h>

namespace rba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;       // head size
constexpr int NT = 256;      // threads per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
struct Tile;

// bf16: 64-key tiles; V stored transposed so PV A-operands are 16-byte reads.
template <>
struct Tile<__bf16> {
    static constexpr int N = 64;              // keys per tile
    static constexpr int CH = 8;              // elements per 16-byte chunk
    static constexpr int KS = D + 8;          // K row stride (elements): 68 dwords
    static constexpr int VROWS = D;           // V^T rows (head dim)
    static constexpr int VS = N + 8;          // V^T row stride: 36 dwords
    static constexpr int SW = 104;            // slab row width >= 32 + N - 1 + CH - 1
};

// fp32: 32-key tiles; V kept row-major (fp32 MFMA takes one element per lane).
template <>
struct Tile<float> {
    static constexpr int N = 32;
    static constexpr int CH = 4;
    static constexpr int KS = D + 4;
    static constexpr int VROWS = 32;
    static constexpr int VS = D + 4;
    static constexpr int SW = 68;
};

// A-operand row i of a 32x32 MFMA -> key offset inside a 32-key sub-tile.  With
// this order the accumulator register r of lane half hh holds key 16*hh + r.
__device__ __forceinline__ int mfma_row_key(int i) { return ((i >> 2) & 1) * 16 + (i >> 3) * 4 + (i & 3); }

// Physical LDS row of key j of a tile: spreads the rows one MFMA A-operand
// read touches over distinct banks.
__device__ __forceinline__ int lds_key_row(int j) { return j ^ (((j >> 4) & 1) * 12); }

__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T, int HW>
__global__ __launch_bounds__(NT) void attn_fwd_kernel(const AttnParams p) {
    using TL = Tile<T>;
    constexpr bool BF = sizeof(T) == 2;
    constexpr int N = TL::N;
    constexpr int KT = N / 32;                   // 32-key sub-tiles per tile
    constexpr int CH = TL::CH;
    constexpr int KS = TL::KS;
    constexpr int VS = TL::VS;
    constexpr int SW = TL::SW;
    constexpr int NCH = SW / CH;                 // chunks per slab row
    constexpr int SROWS = HW * 128;              // slab rows = max columns per workgroup
    constexpr int NSC = (SROWS * NCH + NT - 1) / NT;
    constexpr int CPR = D * (int)sizeof(T) / 16; // 16-byte chunks per K/V row

    __shared__ __attribute__((aligned(16))) T sK[N * KS];
    __shared__ __attribute__((aligned(16))) T sV[TL::VROWS * VS];
    __shared__ __attribute__((aligned(16))) T sR[SROWS * SW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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
    const int ebase0 = (p_min - N + 1) & ~(CH - 1);   // floor to a chunk; tile j0 uses ebase0 - j0

    const T *__restrict__ gq = (const T *)p.q;
    const T *__restrict__ gk = (const T *)p.k + (int64_t)b * p.ks0 + (int64_t)hkv * p.ks2;
    const T *__restrict__ gv = (const T *)p.v + (int64_t)b * p.vs0 + (int64_t)hkv * p.vs2;
    const T *__restrict__ gR = (const T *)p.R;

    // ------------------------------------------------------------ per-column state
    int col[HW], prow[HW], tq[HW], hq[HW];
    bool cvalid[HW];
    float amul[HW], bmul[HW];
#pragma unroll
    for (int s = 0; s < HW; ++s) {
        const int c = (wave * HW + s) * 32 + lc;
        const int hl = c / p.QB;
        const int qi = c - hl * p.QB;
        col[s] = c;
        cvalid[s] = c < ncols && qi < nrows;
        tq[s] = t0 + qi;
        hq[s] = hkv * p.G + min(hl, p.G - 1);
        prow[s] = p_min + qi;
        const float f = p.inv_ln_base > 0.f ? logf((float)prow[s] + 1.f) * p.inv_ln_base : 1.f;
        amul[s] = p.scale_log2e * f;
        bmul[s] = kLog2e * f;
    }
    const bool wave_active = wave * HW * 32 < ncols;

    // Q fragments (B operand of S^T = K Q^T), loaded once.
    constexpr int QREGS = BF ? 8 : 64;
    typedef typename std::conditional<BF, bf16x8, float>::type QFrag;
    QFrag qf[HW][QREGS];
#pragma unroll
    for (int s = 0; s < HW; ++s) {
        const T *qp = gq + (int64_t)b * p.qs0 + (int64_t)tq[s] * p.qs1 + (int64_t)hq[s] * p.qs2;
        if constexpr (BF) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                qf[s][k] = cvalid[s] ? *(const bf16x8 *)(qp + 16 * k + 8 * hh) : bf16x8{};
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                f32x4 x = cvalid[s] ? *(const f32x4 *)(qp + 64 * hh + 4 * k) : f32x4{};
                qf[s][4 * k + 0] = x[0];
                qf[s][4 * k + 1] = x[1];
                qf[s][4 * k + 2] = x[2];
                qf[s][4 * k + 3] = x[3];
            }
        }
    }

    f32x16 O[HW][4];
    float m[HW], l[HW];
#pragma unroll
    for (int s = 0; s < HW; ++s) {
        m[s] = -INFINITY;
        l[s] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) O[s][dt] = f32x16{};
    }

    // ------------------------------------------------------------ tile staging
    u32x4 kreg[4];
    typedef typename std::conditional<BF, u32x2, u32x4>::type VChunk;
    constexpr int NVC = BF ? 8 : 4;
    VChunk vreg[NVC];
    u32x4 sreg[NSC];
    // bf16 V^T staging: 8 keys x 4 head-dim entries per thread
    const int v_kq = (tid >> 2) & 7;
    const int v_dq = (tid & 3) | ((tid >> 5) << 2);

    auto banded = [&](int kt) { return has_bias && (p_min - (kt * N + N - 1) < p.E); };

    auto load_tile = [&](int kt) {
        const int j0 = kt * N;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ci = tid + NT * i;
            const int row = ci / CPR, cc = ci - row * CPR;
            const int j = j0 + row;
            kreg[i] = j < p.Skv ? *(const u32x4 *)(gk + (int64_t)j * p.ks1 + cc * CH) : u32x4{};
        }
        if constexpr (BF) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int j = j0 + 8 * v_kq + i;
                vreg[i] = j < p.Skv ? *(const u32x2 *)(gv + (int64_t)j * p.vs1 + 4 * v_dq) : u32x2{};
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ci = tid + NT * i;
                const int row = ci / CPR, cc = ci - row * CPR;
                const int j = j0 + row;
                vreg[i] = j < p.Skv ? *(const u32x4 *)(gv + (int64_t)j * p.vs1 + cc * CH) : u32x4{};
            }
        }
        if (banded(kt)) {
            const int ebase = ebase0 - j0;
#pragma unroll
            for (int i = 0; i < NSC; ++i) {
                const int ci = tid + NT * i;
                u32x4 val = u32x4{};
                if (ci < SROWS * NCH) {
                    const int row = ci / NCH, ch = ci - row * NCH;
                    const int hl = row / p.QB, qi = row - hl * p.QB;
                    const int e0 = ebase + ch * CH;
                    if (row < ncols && qi < nrows) {
                        const T *src = gR + (int64_t)b * p.Rs0 + (int64_t)(t0 + qi) * p.Rs1 +
                                       (int64_t)(hkv * p.G + hl) * p.Rs2;
                        if (p.r_vec) {
                            if (e0 >= 0 && e0 + CH <= p.E) val = *(const u32x4 *)(src + e0);
                        } else {
                            T tmp[CH];
#pragma unroll
                            for (int x = 0; x < CH; ++x) {
                                const int e = e0 + x;
                                tmp[x] = (e >= 0 && e < p.E) ? src[e] : (T)0.f;
                            }
                            __builtin_memcpy(&val, tmp, 16);
                        }
                    }
                }
                sreg[i] = val;
            }
        }
    };

    auto store_tile = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ci = tid + NT * i;
            const int row = ci / CPR, cc = ci - row * CPR;
            *(u32x4 *)&sK[lds_key_row(row) * KS + cc * CH] = kreg[i];
        }
        if constexpr (BF) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int w = e >> 1;
                u32x4 out;
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    const unsigned lo = vreg[2 * mm][w], hi = vreg[2 * mm + 1][w];
                    out[mm] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                }
                *(u32x4 *)&sV[(4 * v_dq + e) * VS + 8 * v_kq] = out;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ci = tid + NT * i;
                const int row = ci / CPR, cc = ci - row * CPR;
                *(u32x4 *)&sV[row * VS + cc * CH] = vreg[i];
            }
        }
        if (banded(kt)) {
#pragma unroll
            for (int i = 0; i < NSC; ++i) {
                const int ci = tid + NT * i;
                if (ci < SROWS * NCH) {
                    const int row = ci / NCH, ch = ci - row * NCH;
                    *(u32x4 *)&sR[row * SW + ch * CH] = sreg[i];
                }
            }
        }
    };

    // ------------------------------------------------------------ one key tile
    const int kr0 = lds_key_row(mfma_row_key(lc));
    const int kr1 = lds_key_row(32 + mfma_row_key(lc));

    auto compute_tile = [&](int kt) {
        const int j0 = kt * N;
        f32x16 S[HW][KT];
#pragma unroll
        for (int s = 0; s < HW; ++s)
#pragma unroll
            for (int u = 0; u < KT; ++u) S[s][u] = f32x16{};

        // S^T = K . Q^T
        if constexpr (BF) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
#pragma unroll
                for (int u = 0; u < KT; ++u) {
                    const bf16x8 a = *(const bf16x8 *)&sK[(u == 0 ? kr0 : kr1) * KS + 16 * k + 8 * hh];
#pragma unroll
                    for (int s = 0; s < HW; ++s)
                        S[s][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s][k], S[s][u], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const f32x4 a = *(const f32x4 *)&sK[kr0 * KS + 64 * hh + 4 * k];
#pragma unroll
                for (int x = 0; x < 4; ++x)
#pragma unroll
                    for (int s = 0; s < HW; ++s)
                        S[s][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[x], qf[s][4 * k + x], S[s][0], 0, 0, 0);
            }
        }

        const bool band = banded(kt);
        const bool edge = !((j0 + N - 1 <= p_min) && (W == 0 || p_max - j0 < W));

        // scale, bias, mask, online softmax (exp2 domain)
#pragma unroll
        for (int s = 0; s < HW; ++s) {
#pragma unroll
            for (int u = 0; u < KT; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r) S[s][u][r] *= amul[s];
            if (band) {
                const T *srow = sR + col[s] * SW + (prow[s] - ebase0) - 16 * hh;
#pragma unroll
                for (int u = 0; u < KT; ++u)
#pragma unroll
                    for (int r = 0; r < 16; ++r) S[s][u][r] += bmul[s] * to_f32(srow[-(32 * u + r)]);
            }
            if (edge) {
#pragma unroll
                for (int u = 0; u < KT; ++u)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int dist = prow[s] - (j0 + 32 * u + 16 * hh + r);
                        const bool vis = dist >= 0 && (W == 0 || dist < W);
                        S[s][u][r] = vis ? S[s][u][r] : -INFINITY;
                    }
            }
            float mt = -INFINITY;
#pragma unroll
            for (int u = 0; u < KT; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt = fmaxf(mt, S[s][u][r]);
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float mn = fmaxf(m[s], mt);
            const float mu = mn == -INFINITY ? 0.f : mn;
            const float alpha = fast_exp2(m[s] - mu);
            m[s] = mn;
            float sum = 0.f;
#pragma unroll
            for (int u = 0; u < KT; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = fast_exp2(S[s][u][r] - mu);
                    S[s][u][r] = e;
                    sum += e;
                }
            l[s] = l[s] * alpha + sum;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) O[s][dt] *= alpha;
        }

        // O^T += V^T . P^T
        if constexpr (BF) {
#pragma unroll
            for (int u = 0; u < KT; ++u) {
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    bf16x8 pb[HW];
#pragma unroll
                    for (int s = 0; s < HW; ++s)
#pragma unroll
                        for (int x = 0; x < 8; ++x) pb[s][x] = (__bf16)S[s][u][8 * h2 + x];
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) {
                        const bf16x8 a = *(const bf16x8 *)&sV[(32 * dt + lc) * VS + 32 * u + 16 * hh + 8 * h2];
#pragma unroll
                        for (int s = 0; s < HW; ++s)
                            O[s][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s], O[s][dt], 0, 0, 0);
                    }
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const float a = sV[(16 * hh + r) * VS + 32 * dt + lc];
#pragma unroll
                    for (int s = 0; s < HW; ++s)
                        O[s][dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, S[s][0][r], O[s][dt], 0, 0, 0);
                }
            }
        }
    };

    // ------------------------------------------------------------ main loop
    if (kb < ke) {
        load_tile(kb);
        store_tile(kb);
    }
    __syncthreads();
    for (int kt = kb; kt < ke; ++kt) {
        const bool nxt = kt + 1 < ke;
        if (nxt) load_tile(kt + 1);
        if (wave_active) compute_tile(kt);
        __syncthreads();
        if (nxt) store_tile(kt + 1);
        __syncthreads();
    }

    // ------------------------------------------------------------ epilogue
#pragma unroll
    for (int s = 0; s < HW; ++s) {
        const float lt = l[s] + __shfl_xor(l[s], 32);
        if (!cvalid[s]) continue;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const float lse_v = lt > 0.f ? (m[s] + log2f(lt)) * kLn2 : -INFINITY;
        if (p.splits == 1) {
            T *op = (T *)p.o + (int64_t)b * p.os0 + (int64_t)tq[s] * p.os1 + (int64_t)hq[s] * p.os2;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d0 = 32 * dt + 8 * g4 + 4 * hh;
                    if constexpr (BF) {
                        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                        bf16x4 w;
#pragma unroll
                        for (int x = 0; x < 4; ++x) w[x] = (__bf16)(O[s][dt][4 * g4 + x] * inv);
                        *(bf16x4 *)(op + d0) = w;
                    } else {
                        f32x4 w;
#pragma unroll
                        for (int x = 0; x < 4; ++x) w[x] = O[s][dt][4 * g4 + x] * inv;
                        *(f32x4 *)(op + d0) = w;
                    }
                }
            if (p.lse != nullptr && hh == 0) p.lse[((int64_t)b * p.Hq + hq[s]) * p.Sq + tq[s]] = lse_v;
        } else {
            const int64_t row = (((int64_t)sp * p.B + b) * p.Sq + tq[s]) * p.Hq + hq[s];
            float *op = p.o_part + row * D;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d0 = 32 * dt + 8 * g4 + 4 * hh;
                    f32x4 w;
#pragma unroll
                    for (int x = 0; x < 4; ++x) w[x] = O[s][dt][4 * g4 + x] * inv;
                    *(f32x4 *)(op + d0) = w;
                }
            if (hh == 0) p.lse_part[row] = lse_v;
        }
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
    const dim3 grid((unsigned)blocks), block(NT);
    switch (v) {
        case AttnVariant::BF16_WIDE:
            hipLaunchKernelGGL((attn_fwd_kernel<__bf16, 2>), grid, block, 0, stream, p);
            break;
        case AttnVariant::BF16_NARROW:
            hipLaunchKernelGGL((attn_fwd_kernel<__bf16, 1>), grid, block, 0, stream, p);
            break;
        case AttnVariant::FP32:
            hipLaunchKernelGGL((attn_fwd_kernel<float, 1>), grid, block, 0, stream, p);
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
