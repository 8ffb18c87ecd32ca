// attn_fwd.hip -- causal GQA attention forward on gfx950 (attn_fwd).
//
// What it computes: for each query row t of each query head, O_t = softmax(scale * q_t K^T
// over keys s <= t) V and LSE_t ("Tiny Hackable CUDA Language Model Implementation",
// section 1: causal scaled dot-product attention; "Show HN: NanoEuler", section 2: query
// heads share K/V heads).  As the NanoEuler engine does ("Show HN: NanoEuler", section 4;
// the blog's "Tiled FlashAttention" section), keys are consumed tile by tile with an online
// softmax (running max m, running sum l, rescale of the partial output by 2^(m_old-m_new)),
// so no T x T matrix exists anywhere.
//
// gfx950 design:
//  * One workgroup = one query tile of one batch and G heads of one K/V head group (G
//    waves, or G * WPH waves when a head gets several waves).  Each K/V tile is read from
//    HBM once into LDS and shared by every head of the group.
//  * Each wave owns 32*QB query rows of one head and keeps them, their output accumulator
//    and their softmax state in registers.  Scores are formed transposed, S^T = K Q^T, on
//    32x32 MFMA tiles: a lane then holds one query column and 16 keys per tile, so the
//    row max and row sum are in-lane reductions plus one exchange between the two lane
//    halves.  O^T += V^T P^T reuses the score registers directly as the B operand.
//  * K is staged row-major (A operand of S^T, read as 16-byte runs); V is staged
//    transposed and in "slot" order (A operand of O^T).  LDS rows carry 16 bytes of
//    padding so that 16 lanes of a 16-byte read hit distinct banks.
//  * The next K/V tile is fetched from HBM into registers (16-byte coalesced loads)
//    while the current tile is computed.
//  * Tiles strictly above the diagonal are never visited; the mask is evaluated only on
//    tiles that cross the diagonal.  The launch order puts the longest (latest) query
//    tiles first, and workgroups of one K/V head land on the same XCD for L2 reuse.
#include <cmath>

#include "ea_common.h"
#include "ea_kernels.h"

namespace ea {
namespace {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, T, Hq, Hkv;
    int G;    // heads of the group handled by one workgroup
    int WPH;  // waves per head
    int nhc;  // head chunks per K/V head (g / G)
    int ntq;  // query tiles
    float sl2;  // scale * log2(e)
};

template <typename T, int D, int QB, int BN, int NW>
struct FwdCfg {
    static constexpr int KPL = Mfma<T>::KPL;
    static constexpr int NS = D / (2 * KPL);  // MFMA steps over head_dim
    static constexpr int NKB = BN / 32;       // 32-key blocks per tile
    static constexpr int NDB = D / 32;        // 32-row blocks of head_dim
    static constexpr int PS = 16 / KPL;       // MFMA steps per 32-key block
    static constexpr int EPC = 16 / sizeof(T);
    static constexpr int CPR = D / EPC;       // 16-byte chunks per K/V row
    static constexpr int KS = D + EPC;        // K tile row stride (16 bytes of padding)
    static constexpr int VS = BN + EPC;       // V^T tile row stride
    static constexpr int NT = 64 * NW;
    static constexpr int NCH = (BN * CPR + NT - 1) / NT;
    static constexpr int QW = 32 * QB;
};

template <typename T, int D, int QB, int BN, int NW>
__global__ __launch_bounds__(64 * NW) void attn_fwd_kernel(FwdArgs a) {
    using C = FwdCfg<T, D, QB, BN, NW>;
    using M = Mfma<T>;
    using frag = typename M::frag;
    constexpr int KPL = C::KPL;

    __shared__ __attribute__((aligned(16))) T Ks[BN * C::KS];
    __shared__ __attribute__((aligned(16))) T Vt[D * C::VS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int half = lane >> 5;
    const int l32 = lane & 31;

    const int HB = a.B * a.Hkv * a.nhc;
    const int L = blockIdx.x;
    const int tile = a.ntq - 1 - L / HB;
    const int rem = L % HB;
    const int hc = rem % a.nhc;
    const int kvh = (rem / a.nhc) % a.Hkv;
    const int b = rem / (a.nhc * a.Hkv);
    const int g = a.Hq / a.Hkv;
    const int BM = a.WPH * C::QW;
    const int hs = w / a.WPH;
    const int sub = w % a.WPH;
    const int head = kvh * g + hc * a.G + hs;
    const int q0 = tile * BM + sub * C::QW;
    const bool active = q0 < a.T;
    const int qlast = min(q0 + C::QW, a.T) - 1;
    const int wg_last = min(tile * BM + BM, a.T) - 1;
    const int jmax = wg_last / BN;

    const T* __restrict__ qp = static_cast<const T*>(a.q);
    const T* __restrict__ kp = static_cast<const T*>(a.k);
    const T* __restrict__ vp = static_cast<const T*>(a.v);

    // Q fragments ("split" over head_dim): lane (query l32, half) holds half*D/2 .. +D/2.
    frag qf[QB][C::NS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int t = q0 + qb * 32 + l32;
        if (active && t < a.T) {
            const T* row = qp + (((long long)b * a.T + t) * a.Hq + head) * D + half * (D / 2);
#pragma unroll
            for (int c = 0; c < (D / 2) / C::EPC; ++c) {
                Vec16<T> v = ld16(row + c * C::EPC);
#pragma unroll
                for (int e = 0; e < C::EPC / KPL; ++e) {
                    qf[qb][c * (C::EPC / KPL) + e] =
                        reinterpret_cast<const frag*>(&v.raw)[e];
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < C::NS; ++s) qf[qb][s] = frag{};
        }
    }

    Vec16<T> kreg[C::NCH], vreg[C::NCH];
    auto fetch = [&](int j) {
#pragma unroll
        for (int n = 0; n < C::NCH; ++n) {
            const int c = tid + n * C::NT;
            if (c < BN * C::CPR) {
                const int key = c / C::CPR;
                const int part = c % C::CPR;
                const int s = j * BN + key;
                if (s < a.T) {
                    const long long off =
                        (((long long)b * a.T + s) * a.Hkv + kvh) * D + part * C::EPC;
                    kreg[n] = ld16(kp + off);
                    vreg[n] = ld16(vp + off);
                } else {
                    kreg[n] = zero16<T>();
                    vreg[n] = zero16<T>();
                }
            }
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int n = 0; n < C::NCH; ++n) {
            const int c = tid + n * C::NT;
            if (c < BN * C::CPR) {
                const int key = c / C::CPR;
                const int part = c % C::CPR;
                st16(&Ks[key * C::KS + part * C::EPC], kreg[n]);
                const int slot = (key & ~31) + acc_slot(key & 31);
#pragma unroll
                for (int e = 0; e < C::EPC; ++e) Vt[(part * C::EPC + e) * C::VS + slot] = vreg[n].get(e);
            }
        }
    };

    float m[QB], l[QB];
    f32x16 oacc[QB][C::NDB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -INFINITY;
        l[qb] = 0.0f;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) oacc[qb][db] = zero_acc();
    }

    fetch(0);
    for (int j = 0; j <= jmax; ++j) {
        __syncthreads();
        commit();
        __syncthreads();
        if (j < jmax) fetch(j + 1);
        if (!active || j * BN > qlast) continue;
        const bool diag = (j * BN + BN - 1) > q0;

        // S^T = K Q^T for this tile.
        f32x16 sacc[QB][C::NKB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) sacc[qb][kb] = zero_acc();
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
                const frag af = load_frag<T>(&Ks[(kb * 32 + l32) * C::KS + half * (D / 2) + s * KPL]);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[qb][kb] = M::mma(af, qf[qb][s], sacc[qb][kb]);
            }
        }

        // Online softmax, one query column per lane.
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int tq = q0 + qb * 32 + l32;
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = sacc[qb][kb][r];
                    if (diag) {
                        const int key = j * BN + kb * 32 + acc_row(r, half);
                        if (key > tq) x = -INFINITY;
                    }
                    sacc[qb][kb][r] = x;
                    mx = fmaxf(mx, x);
                }
            }
            mx = fmaxf(mx, xor_shfl32(mx));
            const float mnew = fmaxf(m[qb], mx * a.sl2);
            const float msafe = (mnew == -INFINITY) ? 0.0f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(m[qb] - msafe);
            float rs = 0.0f;
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(sacc[qb][kb][r] * a.sl2 - msafe);
                    sacc[qb][kb][r] = p;
                    rs += p;
                }
            }
            l[qb] = l[qb] * alpha + rs;
            m[qb] = mnew;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
        }

        // O^T += V^T P^T.
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
            for (int ps = 0; ps < C::PS; ++ps) {
                frag pf[QB];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) pf[qb] = acc_to_frag<T>(sacc[qb][kb], ps * KPL);
#pragma unroll
                for (int db = 0; db < C::NDB; ++db) {
                    const frag vf = load_frag<T>(
                        &Vt[(db * 32 + l32) * C::VS + kb * 32 + 16 * half + ps * KPL]);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = M::mma(vf, pf[qb], oacc[qb][db]);
                }
            }
        }
    }

    if (!active) return;
    T* __restrict__ op = static_cast<T*>(a.o);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int tq = q0 + qb * 32 + l32;
        const float lt = l[qb] + xor_shfl32(l[qb]);
        if (tq < a.T) {
            const float inv = 1.0f / lt;
            T* orow = op + (((long long)b * a.T + tq) * a.Hq + head) * D;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int d0 = db * 32 + 8 * a4 + 4 * half;
                    if constexpr (sizeof(T) == 2) {
                        bf16x4 v;
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = (bf16)(oacc[qb][db][4 * a4 + e] * inv);
                        *reinterpret_cast<bf16x4*>(orow + d0) = v;
                    } else {
                        f32x4 v;
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = oacc[qb][db][4 * a4 + e] * inv;
                        *reinterpret_cast<f32x4*>(orow + d0) = v;
                    }
                }
            }
            if (half == 0) a.lse[((long long)b * a.Hq + head) * a.T + tq] = (m[qb] + __log2f(lt)) * kLn2;
        }
    }
}

template <typename T, int D, int QB, int BN, int NW>
hipError_t launch_fwd_cfg(const FwdArgs& a0, int G, int WPH, hipStream_t stream) {
    FwdArgs a = a0;
    const int g = a.Hq / a.Hkv;
    a.G = G;
    a.WPH = WPH;
    a.nhc = g / G;
    const int BM = WPH * 32 * QB;
    a.ntq = (a.T + BM - 1) / BM;
    const long long blocks = (long long)a.ntq * a.B * a.Hkv * a.nhc;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, QB, BN, NW>), dim3((unsigned)blocks), dim3(64 * NW),
                       0, stream, a);
    return hipGetLastError();
}

// Heads per workgroup: the whole group when it has at most four heads, else the largest
// divisor of g that is at most four; heads with fewer siblings get more waves each.
void pick_group(int g, int* G, int* WPH) {
    int G_ = 1;
    for (int c = 4; c >= 1; --c)
        if (g % c == 0) {
            G_ = c;
            break;
        }
    *G = G_;
    *WPH = (G_ == 3) ? 1 : 4 / G_;
}

template <typename T, int D>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
    int G, WPH;
    pick_group(a.Hq / a.Hkv, &G, &WPH);
    constexpr bool big = (sizeof(T) == 4 && D == 128);
    constexpr int QB = big ? 1 : 2;
    constexpr int BN = big ? 32 : 64;
    if (G * WPH == 3) return launch_fwd_cfg<T, D, QB, BN, 3>(a, G, WPH, stream);
    return launch_fwd_cfg<T, D, QB, BN, 4>(a, G, WPH, stream);
}

}  // namespace

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int T, int Hq, int Hkv, int D, float scale, IoType dt,
                           hipStream_t stream) {
    FwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.B = B;
    a.T = T;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.sl2 = scale * kLog2e;
    if (dt == kF32) {
        if (D == 32) return launch_fwd_t<float, 32>(a, stream);
        if (D == 64) return launch_fwd_t<float, 64>(a, stream);
        return launch_fwd_t<float, 128>(a, stream);
    }
    if (D == 32) return launch_fwd_t<bf16, 32>(a, stream);
    if (D == 64) return launch_fwd_t<bf16, 64>(a, stream);
    return launch_fwd_t<bf16, 128>(a, stream);
}

}  // namespace ea
