// Relative-logit projection R[t, h, :] = r[t, :] . P[h]  for gfx950.
//
// Each token's relative feature r is mapped by a learned per-head matrix P to
// a row of relative logits indexed by causal distance ("SGLang と Miles が
// Inkling を初日からサポート", sections "Inkling のモデルアーキテクチャ" and
// "相対位置バイアス付き Attention").
//
// The contraction is short (r_dim <= 128) and the output is E entries per
// (token, head), so the kernel is bound by writing R.  A workgroup owns one
// head, one chunk of up to 256 distances and NTB blocks of 128 tokens (32 per
// wave); it stages that chunk of P[h]^T in LDS once (all loads in flight
// together) and for each token block computes R^T tiles (32 distances x 32
// tokens) with MFMA, A = P^T from LDS and B = r^T from registers.  The
// A-operand row order makes every lane hold 16 consecutive distances of one
// token, so R is written with 16-byte stores.  Registers are kept low (one
// token tile per wave, k-steps sized to r_dim) so that enough waves stay
// resident to keep the store stream going, and workgroups are numbered so that
// those resident together cover whole rows of R.
#include "rba_internal.h"

#include <algorithm>
#include <type_traits>

namespace rba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = 256;
constexpr int TT = 1;         // 32-token column tiles per wave
constexpr int TPW = 32 * TT;  // tokens per wave
constexpr int TPB = 4 * TPW;  // tokens per workgroup
constexpr int KMAX = 128;     // largest r_dim
constexpr int kMaxTokenBlocks = 4;
constexpr int kMinWorkgroups = 4096;

__device__ __forceinline__ int mfma_row_key(int i) { return ((i >> 2) & 1) * 16 + (i >> 3) * 4 + (i & 3); }
__device__ __forceinline__ int lds_row(int j) { return j ^ (((j >> 4) & 1) * 12); }

// NK: 16-channel k-steps held in registers for bf16 input (r_dim <= 16 NK); it
// sizes the register file use, and with it how many waves a CU keeps in flight
// to stream the output.
template <typename TI, typename TO, int NK>
__global__ __launch_bounds__(NT) void relproj_kernel(const TI *__restrict__ r, int64_t rs, int64_t rsh,
                                                     const TI *__restrict__ P,
                                                     TO *__restrict__ R, int64_t T, int Hq, int r_dim, int E, int EC,
                                                     int NTB) {
    constexpr bool BF = sizeof(TI) == 2;
    constexpr int PAD = BF ? 8 : 4;
    // P^T chunk in LDS: EC rows (distances) x KP (+pad) channels; the workgroup's
    // distance chunk is zc
    extern __shared__ __attribute__((aligned(16))) unsigned char relproj_lds[];
    TI *sP = (TI *)relproj_lds;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5, lc = lane & 31;
    // Workgroup order: distance chunk fastest, then head, then token blocks, so
    // the workgroups resident at one time write whole R rows (all heads and
    // distances of their tokens) rather than strided pieces of many rows.
    const int nz = (E + EC - 1) / EC;
    const int zc = (int)(blockIdx.x % (unsigned)nz);
    const int h = (int)((blockIdx.x / (unsigned)nz) % (unsigned)Hq);
    const int64_t xb = blockIdx.x / ((unsigned)nz * (unsigned)Hq);
    const int KP = (r_dim + 15) & ~15;     // channels padded to a 16-multiple
    const int PS = KP + PAD;               // LDS row stride
    const bool r_vec = (r_dim % 8 == 0) && (rs % 8 == 0) && (rsh % 8 == 0);
    const bool e_vec = (E % (16 / (int)sizeof(TO))) == 0;
    const int nks = BF ? KP / 16 : KP / 2;
    const int arow_key = mfma_row_key(lc);
    const int e0 = zc * EC;

    // ---- stage P[h][:, e0:e0+EC]^T once for all NTB token blocks: each unit =
    // 4 channels x 8 distances.  All loads of a pass are issued before any is
    // used (one wait per pass).
    {
        const int units = (KP / 4) * (EC / 8);
        constexpr int UPT = 2;   // units per thread and pass
        for (int u0 = 0; u0 < units; u0 += UPT * NT) {
            TI v[UPT][4][8];
#pragma unroll
            for (int j = 0; j < UPT; ++j) {
                const int u = u0 + j * NT + tid;
                const int cq = u / (EC / 8), eq = u - cq * (EC / 8);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 4 * cq + i;
                    const int e = e0 + 8 * eq;
                    const TI *src = P + ((int64_t)h * r_dim + c) * E + e;
                    if (u < units && c < r_dim && (E % 8 == 0) && e + 8 <= E) {
                        if constexpr (BF) {
                            *(u32x4 *)v[j][i] = *(const u32x4 *)src;
                        } else {
                            *(u32x4 *)&v[j][i][0] = *(const u32x4 *)src;
                            *(u32x4 *)&v[j][i][4] = *(const u32x4 *)(src + 4);
                        }
                    } else {
#pragma unroll
                        for (int x = 0; x < 8; ++x) v[j][i][x] = (u < units && c < r_dim && e + x < E) ? src[x] : (TI)0.f;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < UPT; ++j) {
                const int u = u0 + j * NT + tid;
                if (u >= units) continue;
                const int cq = u / (EC / 8), eq = u - cq * (EC / 8);
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    TI w[4] = {v[j][0][x], v[j][1][x], v[j][2][x], v[j][3][x]};
                    const int er = 8 * eq + x;  // distance row inside the chunk
                    TI *dst = &sP[(32 * (er >> 5) + lds_row(er & 31)) * PS + 4 * cq];
                    if constexpr (BF)
                        *(u32x2 *)dst = *(const u32x2 *)w;
                    else
                        *(u32x4 *)dst = *(const u32x4 *)w;
                }
            }
        }
        __syncthreads();
    }

    for (int tb = 0; tb < NTB; ++tb) {
    const int64_t tbase = (xb * NTB + tb) * TPB + wave * TPW;
    if (tbase >= T) break;

    // B operands: r^T for this lane's token columns.
    typedef typename std::conditional<BF, bf16x8, float>::type Frag;
    Frag rf[TT][BF ? NK : 64];
#pragma unroll
    for (int c = 0; c < TT; ++c) {
        const int64_t t = tbase + 32 * c + lc;
        const bool ok = t < T;
        const TI *rp = r + (ok ? t : 0) * rs + (int64_t)h * rsh;   // rsh = 0: r shared by all heads
        if constexpr (BF) {
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                bf16x8 x = bf16x8{};
                const int c0 = 16 * k + 8 * hh;
                if (ok && k < nks) {
                    if (r_vec && c0 + 8 <= r_dim) {
                        x = *(const bf16x8 *)(rp + c0);
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i) x[i] = c0 + i < r_dim ? rp[c0 + i] : (__bf16)0.f;
                    }
                }
                rf[c][k] = x;
            }
        } else {
            const int KH = KP / 2;  // channels per lane half
#pragma unroll
            for (int k = 0; k < 64; ++k) {
                const int ch = KH * hh + k;
                rf[c][k] = (ok && k < KH && ch < r_dim) ? rp[ch] : 0.f;
            }
        }
    }
    // Settle the r loads here.  On this target stores also count in vmcnt, so
    // a wait for these loads left inside the loop would wait for every store
    // issued so far as well.
#pragma unroll
    for (int c = 0; c < TT; ++c)
#pragma unroll
        for (int k = 0; k < (BF ? NK : 64); ++k) asm volatile("" : "+v"(rf[c][k]));

    {
        // ---- the distance tiles of 32 of the chunk
#pragma unroll
        for (int et = 0; et < EC / 32; ++et) {
            if (e0 + 32 * et >= E) break;
            f32x16 acc[TT];
#pragma unroll
            for (int c = 0; c < TT; ++c) acc[c] = f32x16{};
            const TI *arow = &sP[(32 * et + lds_row(arow_key)) * PS];
            if constexpr (BF) {
#pragma unroll
                for (int k = 0; k < NK; ++k) {
                    if (k < nks) {
                        const bf16x8 a = *(const bf16x8 *)(arow + 16 * k + 8 * hh);
#pragma unroll
                        for (int c = 0; c < TT; ++c)
                            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, rf[c][k], acc[c], 0, 0, 0);
                    }
                }
            } else {
                const int KH = KP / 2;
#pragma unroll
                for (int k4 = 0; k4 < 16; ++k4) {
                    if (4 * k4 < KH) {
                        const f32x4 a = *(const f32x4 *)(arow + KH * hh + 4 * k4);
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
#pragma unroll
                            for (int c = 0; c < TT; ++c)
                                acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[x], rf[c][4 * k4 + x], acc[c], 0, 0, 0);
                        }
                    }
                }
            }
            // lane holds distances e0 + 32et + 16hh + 0..15 of token column lc
            const int eb = e0 + 32 * et + 16 * hh;
#pragma unroll
            for (int c = 0; c < TT; ++c) {
                const int64_t t = tbase + 32 * c + lc;
                if (t >= T) continue;
                TO *dst = R + (t * Hq + h) * (int64_t)E + eb;
                if (e_vec && eb + 16 <= E) {
                    if constexpr (sizeof(TO) == 2) {
                        bf16x8 w0, w1;
#pragma unroll
                        for (int x = 0; x < 8; ++x) {
                            w0[x] = (__bf16)acc[c][x];
                            w1[x] = (__bf16)acc[c][8 + x];
                        }
                        *(bf16x8 *)dst = w0;
                        *(bf16x8 *)(dst + 8) = w1;
                    } else {
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            f32x4 w;
#pragma unroll
                            for (int x = 0; x < 4; ++x) w[x] = acc[c][4 * q4 + x];
                            *(f32x4 *)(dst + 4 * q4) = w;
                        }
                    }
                } else {
#pragma unroll
                    for (int x = 0; x < 16; ++x)
                        if (eb + x < E) dst[x] = (TO)acc[c][x];
                }
            }
        }
    }
    }  // token blocks
}

// The projection packed as MFMA A-operand fragments for the prefill kernel
// that computes its own R rows: for head h, tile eb of 32 distances, k-step k
// (channels 16k..16k+15) and lane l = (lc = l % 32, hh = l / 32), the 8
// entries P[h, 16k + 8hh + x, 32 eb + mfma_row_key(lc)], x = 0..7, at
// PT[(((h nEB + eb) nks + k) 64 + l) 8 + x] (zero past E).  One workgroup
// per (tile, head); bf16.
__global__ __launch_bounds__(256) void relproj_pack_kernel(const __bf16 *__restrict__ P, __bf16 *__restrict__ PT,
                                                           int r_dim, int E) {
    const int eb = blockIdx.x, h = blockIdx.y, nEB = gridDim.x;
    const int nks = r_dim >> 4;
    const __bf16 *src = P + (int64_t)h * r_dim * E;
    for (int idx = threadIdx.x; idx < nks * 64; idx += blockDim.x) {
        const int k = idx >> 6, l = idx & 63;
        const int e = 32 * eb + mfma_row_key(l & 31);
        const int c0 = 16 * k + 8 * (l >> 5);
        bf16x8 v;
#pragma unroll
        for (int x = 0; x < 8; ++x) v[x] = e < E ? src[(int64_t)(c0 + x) * E + e] : (__bf16)0.f;
        *(bf16x8 *)(PT + ((((int64_t)h * nEB + eb) * nks + k) * 64 + l) * 8) = v;
    }
}

}  // namespace

hipError_t launch_relproj_pack(int Hq, int r_dim, int E, const void *P, void *PT, hipStream_t stream) {
    if (Hq <= 0 || r_dim <= 0 || E <= 0) return hipSuccess;
    const dim3 grid((unsigned)((E + 31) / 32), (unsigned)Hq);
    hipLaunchKernelGGL(relproj_pack_kernel, grid, dim3(256), 0, stream, (const __bf16 *)P, (__bf16 *)PT, r_dim, E);
    return hipGetLastError();
}

hipError_t launch_relproj(bool in_bf16, bool out_bf16, int64_t T, int Hq, int r_dim, int E, const void *r,
                          int64_t r_stride, int64_t r_stride_h, const void *P, void *R, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    // distances per workgroup: the largest of 256 / 128 / 64 whose P^T chunk fits 64 KiB of LDS
    const int es = in_bf16 ? 2 : 4;
    const int ps = ((r_dim + 15) & ~15) + (in_bf16 ? 8 : 4);
    int EC = 256;
    while (EC > 64 && (size_t)EC * ps * es > 65536) EC /= 2;
    const size_t lds = (size_t)EC * ps * es;
    const int64_t gz = (E + EC - 1) / EC;
    // token blocks per workgroup: each staged P chunk serves several blocks
    // while the grid still holds >= kMinWorkgroups workgroups
    const int64_t blocks = (T + TPB - 1) / TPB;
    const int64_t base = blocks * Hq * gz;
    const int NTB = (int)std::max<int64_t>(1, std::min<int64_t>(kMaxTokenBlocks, base / kMinWorkgroups));
    const int64_t gx = (blocks + NTB - 1) / NTB;
    const int64_t nwg = gx * Hq * gz;
    if (nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nwg), block(NT);
    const bool k4 = r_dim <= 64;
    if (in_bf16 && out_bf16) {
        if (k4)
            hipLaunchKernelGGL((relproj_kernel<__bf16, __bf16, 4>), grid, block, lds, stream, (const __bf16 *)r,
                               r_stride, r_stride_h, (const __bf16 *)P, (__bf16 *)R, T, Hq, r_dim, E, EC, NTB);
        else
            hipLaunchKernelGGL((relproj_kernel<__bf16, __bf16, 8>), grid, block, lds, stream, (const __bf16 *)r,
                               r_stride, r_stride_h, (const __bf16 *)P, (__bf16 *)R, T, Hq, r_dim, E, EC, NTB);
    } else if (in_bf16) {
        if (k4)
            hipLaunchKernelGGL((relproj_kernel<__bf16, float, 4>), grid, block, lds, stream, (const __bf16 *)r,
                               r_stride, r_stride_h, (const __bf16 *)P, (float *)R, T, Hq, r_dim, E, EC, NTB);
        else
            hipLaunchKernelGGL((relproj_kernel<__bf16, float, 8>), grid, block, lds, stream, (const __bf16 *)r,
                               r_stride, r_stride_h, (const __bf16 *)P, (float *)R, T, Hq, r_dim, E, EC, NTB);
    } else if (out_bf16) {
        hipLaunchKernelGGL((relproj_kernel<float, __bf16, 8>), grid, block, lds, stream, (const float *)r, r_stride,
                           r_stride_h, (const float *)P, (__bf16 *)R, T, Hq, r_dim, E, EC, NTB);
    } else {
        hipLaunchKernelGGL((relproj_kernel<float, float, 8>), grid, block, lds, stream, (const float *)r, r_stride,
                           r_stride_h, (const float *)P, (float *)R, T, Hq, r_dim, E, EC, NTB);
    }
    return hipGetLastError();
}

}  // namespace rba
