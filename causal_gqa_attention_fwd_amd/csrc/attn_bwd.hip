// attn_bwd.hip -- causal GQA attention backward on gfx950 (attn_bwd and its stages).
//
// The pages only say that NanoEuler's backward is hand-written and gradient-checked
// ("Show HN: NanoEuler", sections 3 and 4); the algorithm here is the recompute-from-LSE
// backward of tiled attention.  With P_ts = exp(S_ts - LSE_t), dP = dO V^T,
// D_t = sum_d dO_t * O_t (= sum_s P_ts dP_ts) and dS = P (dP - D_t):
//   dV_s = sum_{h in group} sum_{t>=s} P_ts dO_t
//   dK_s = scale * sum_{h in group} sum_{t>=s} dS_ts Q_t
//   dQ_t = scale * sum_{s<=t} dS_ts K_s
// Two launches, no atomics, so every output is deterministic:
//   1. bwd_pre:  D_t for every (b, h, t), into the workspace.
//   then bwd_kernel, whose workgroups take one of two roles (one launch per role, or one
//   launch with both roles interleaved when the problem is small):
//   2. dK/dV role: one workgroup per (64-key tile, K/V head, batch).  K and V stay in
//      registers; the workgroup walks every head of the group and every query tile on or
//      below the diagonal, so dK and dV are group-summed in registers and written once.
//      Q and dO tiles are staged row-major; the Q^T / dO^T operands of dK += dS^T Q and
//      dV += P^T dO are read with gfx950's transposing LDS read.  Large bf16 problems take
//      this role in a launch of its own (bwd_dkdv_kernel), with two 32-row query blocks per
//      wave and, up to head_dim 64, 128-key workgroups.
//   3. dQ role:   one workgroup per (query tile, K/V head, batch) over the G heads of the
//      group, shaped like the forward: Q, dO, LSE and D stay in registers, K/V tiles stream
//      through LDS shared by the group's heads, dQ is written once in the I/O dtype.
// Splitting dQ out costs the S and dP products a second time (14D instead of 10D FLOPs per
// query/key pair) but removes the fp32 atomic traffic of a fused kernel, which on this chip
// costs more than the extra matrix-core work at these sizes.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "ea_common.h"
#include "ea_kernels.h"

namespace ea {
namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------------------
// 1. D_t = sum_d dO * O per row.
// ---------------------------------------------------------------------------------------
// Blocks past dt_blocks fill the RoPE table instead: entry (t, i) = (cos, sin) of the angle of
// pair i at position pos0 + t, [T][D/2] float2, for the inverse RoPE applied on the stores of
// dQ and dK (absent when cs is null).
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ o,
                                                      const T* __restrict__ dout,
                                                      float* __restrict__ dt, long long nrows,
                                                      int T_, int Hq, long long dt_blocks,
                                                      float* __restrict__ cs, int pos0, RopeFreq f) {
    if ((long long)blockIdx.x >= dt_blocks) {
        const long long u = ((long long)blockIdx.x - dt_blocks) * 256 + threadIdx.x;
        if (u < (long long)T_ * (D / 2)) {
            const int t = (int)(u / (D / 2)), i = (int)(u % (D / 2));
            float c, sn;
            rope_cos_sin((double)pos0 + (double)t, f.theta[i], &c, &sn);
            reinterpret_cast<float2*>(cs)[u] = make_float2(c, sn);
        }
        return;
    }
    constexpr int EPC = 16 / sizeof(T);
    constexpr int LPR = D / EPC;       // lanes per row (4 .. 32)
    constexpr int RPB = 256 / LPR;     // rows per block: consecutive positions of one (b, h)
    const int tid = threadIdx.x;
    // Block -> (b, h, block of RPB positions), so that the block's D_t values are contiguous
    // in [B, Hq, T] and each row is read as whole 16-byte chunks.
    const long long tblocks = (T_ + RPB - 1) / RPB;
    const long long bh = (long long)blockIdx.x / tblocks;
    const int t = (int)((long long)blockIdx.x % tblocks) * RPB + tid / LPR;
    const long long b = bh / Hq, h = bh % Hq;
    const int c = tid % LPR;
    const bool ok = t < T_ && bh * T_ < nrows;
    const long long row = (b * T_ + t) * Hq + h;
    // Chunk dot products, then the DPP lane butterfly of group_sum (no LDS access).
    float acc = 0.0f;
    if (ok) acc = dot16(ld16(o + row * D + c * EPC), ld16(dout + row * D + c * EPC));
    acc = group_sum<LPR>(acc);
    if (ok && c == 0) dt[bh * T_ + t] = acc;
}

constexpr int kMaxOrder = 256;  // items per (batch, K/V head) the dispatch table can hold

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* lse;
    const float* dt;
    void* dq;
    void* dk;
    void* dv;
    int B, T, Hq, Hkv;
    int G, WPH, nhc;  // dq role: heads per workgroup, waves per head, head chunks
    int ntk;          // dK/dV role: 64-key tiles
    int ntq;          // dK/dV role: query stages (BM rows each)
    int ntq_dq;       // dq role: query tiles (32 * WPH rows each)
    int roles;        // 1: dK/dV only, 2: dQ only, 3: both in one launch
    int causal;       // 1: key s visible to query t iff s <= t; 0: every key visible
    float sl2;        // scale * log2(e)
    float scale;
    const float* rope_cs;  // (cos, sin) per (t, pair) for the inverse RoPE on dQ / dK, or null
    // Dispatch order of one (batch, K/V head)'s items when both roles share a launch (roles
    // 3): entry m is dK/dV item e (e < 0x8000) or dQ item e - 0x8000.  norder = 0: use the
    // proportional merge instead.
    int norder;
    unsigned short order[kMaxOrder];
};

// ---------------------------------------------------------------------------------------
// 2. dK, dV: KV-stationary.
// ---------------------------------------------------------------------------------------
// x as a 16-byte chunk (hi, mid, lo, 0, 0, 0, 0, 0) of bf16 with hi = bf16(x), mid =
// bf16(x - hi), lo = bf16(x - hi - mid) (each difference exact in fp32): hi + mid + lo is x
// to within 2^-24 |x| or so, which a matrix-core product with (1, 1, 1, 0, ...) adds to an
// fp32 accumulator.
template <typename T>
__device__ inline Vec16<T> pad_parts(float x) {
    Vec16<T> v = zero16<T>();
    if constexpr (sizeof(T) == 2) {
        const T hi = (T)x;
        const float r1 = x - (float)hi;
        const T mid = (T)r1;
        const T lo = (T)(r1 - (float)mid);
        v.set(0, hi);
        v.set(1, mid);
        v.set(2, lo);
    }
    return v;
}

// LDS of the dK/dV epilogue's partials (see dkdv_epilogue).
template <int D>
constexpr int kEpiStride = D + 4;  // floats per partial row (conflict-free 16-byte reads)
template <int D, int NKH, int NQH>
constexpr size_t dkdv_epi_bytes() {
    return D <= 64 ? (size_t)NQH * NKH * 2 * 32 * kEpiStride<D> * sizeof(float)
                   : (size_t)NKH * 2 * (D / 32) * 16 * 64 * sizeof(float);
}

template <typename T, int D, int BM, int QB = 1, int BN_ = 64>
struct DkdvCfg {
    static constexpr int KPL = Mfma<T>::KPL;
    static constexpr int BN = BN_;              // keys per workgroup
    static constexpr int NKH = BN / 32;         // 32-key blocks
    static constexpr int QW = 32 * QB;          // query rows of a wave per iteration
    static constexpr int NQH = BM / QW;         // query blocks per iteration
    static constexpr int NW = NKH * NQH;
    static constexpr int NT = 64 * NW;
    static constexpr int NS = D / (2 * KPL);    // MFMA steps over head_dim
    static constexpr int NDB = D / 32;
    static constexpr int PS = 16 / KPL;         // MFMA steps over a 32-row accumulator
    static constexpr int EPC = 16 / sizeof(T);
    static constexpr int CPR = D / EPC;
    static constexpr int QS = D + EPC;          // row-major Q / dO stride (16 bytes of padding)
    static constexpr int NCH = (BM * CPR + NT - 1) / NT;  // chunks per thread per tensor
    // LDS carve-up of one stage (bytes); two stages.
    static constexpr size_t OFF_Q = 0;
    static constexpr size_t OFF_DO = OFF_Q + sizeof(T) * BM * QS;
    static constexpr size_t OFF_LSE = OFF_DO + sizeof(T) * BM * QS;
    static constexpr size_t OFF_DT = OFF_LSE + sizeof(float) * BM;
    static constexpr size_t STAGE = (OFF_DT + sizeof(float) * BM + 15) & ~(size_t)15;
    static constexpr size_t BYTES = 2 * STAGE;
    // LDS of a workgroup of this role: its stages, or the partials of its epilogue.
    static constexpr size_t LDS = BYTES > dkdv_epi_bytes<D, NKH, NQH>() ? BYTES : dkdv_epi_bytes<D, NKH, NQH>();
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// End of a dK/dV item (up to head_dim 64).  Every wave writes its dK / dV partial (its 32 keys, the query rows it
// took) to LDS row-major, [query block][key block][dK | dV][32 keys][D + 4] floats; then every
// thread takes 16-byte output row segments: it sums the NQH partials of its segment, last
// query block first (fixed order: deterministic), scales dK, applies the inverse RoPE to dK
// with (cos, sin) loaded before the partials were written, and stores.  Wave w holds key block
// kh = w % NKH, query block qh = w / NKH.

template <typename T, int D, int NKH, int NQH, int BN, int NT>
__device__ __forceinline__ void dkdv_epilogue_all(const BwdArgs& a, char* smem, f32x16 (&dkacc)[D / 32],
                                              f32x16 (&dvacc)[D / 32], int j, int kvh, int b) {
    constexpr int NDB = D / 32;
    constexpr int EPC = 16 / sizeof(T);
    constexpr int PS = kEpiStride<D>;
    constexpr int CPRo = D / EPC;          // 16-byte output chunks per row
    constexpr int NCK = BN * CPRo;         // chunks of dK (and of dV)
    constexpr int NDK = (NCK + NT - 1) / NT;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int kh = w % NKH;
    const int qh = w / NKH;
    float* part = reinterpret_cast<float*>(smem);
    __syncthreads();  // every wave is done with the stages in LDS
    {
        float* mine = part + (size_t)(qh * NKH + kh) * 2 * 32 * PS;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int at = acc_row(r, half) * PS + db * 32 + l32;
                mine[at] = dkacc[db][r];
                mine[32 * PS + at] = dvacc[db][r];
            }
    }
    // (cos, sin) of this thread's dK segments: issued once the accumulators are in LDS, in
    // flight across the barrier.
    f32x4 tab[NDK][EPC / 4];
    if (a.rope_cs != nullptr) {
#pragma unroll
        for (int u = 0; u < NDK; ++u) {
            const int c = tid + u * NT;
            const int key = min(j * BN + (c < NCK ? c : 0) / CPRo, a.T - 1);
            const f32x4* src = reinterpret_cast<const f32x4*>(a.rope_cs + ((long long)key * (D / 2) + (c % CPRo) * (EPC / 2)) * 2);
#pragma unroll
            for (int e = 0; e < EPC / 4; ++e) tab[u][e] = src[e];
        }
    }
    __syncthreads();
    T* __restrict__ dkp = static_cast<T*>(a.dk);
    T* __restrict__ dvp = static_cast<T*>(a.dv);
#pragma unroll
    for (int u = 0; u < (2 * NCK + NT - 1) / NT; ++u) {
        const int c = tid + u * NT;
        if (c >= 2 * NCK) break;
        const int tsel = c / NCK;
        const int cc = c % NCK;
        const int kl = cc / CPRo, pt = cc % CPRo;
        const int key = j * BN + kl;
        if (key >= a.T) continue;
        const float* src0 = part + (size_t)(kl >> 5) * 2 * 32 * PS + (size_t)tsel * 32 * PS + (size_t)(kl & 31) * PS + pt * EPC;
        constexpr size_t QSTEP = (size_t)NKH * 2 * 32 * PS;  // floats between query blocks
        float x[EPC];
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
            f32x4 s4 = *reinterpret_cast<const f32x4*>(src0 + (NQH - 1) * QSTEP + e);
#pragma unroll
            for (int o = NQH - 2; o >= 0; --o) {
                const f32x4 p4 = *reinterpret_cast<const f32x4*>(src0 + o * QSTEP + e);
#pragma unroll
                for (int v = 0; v < 4; ++v) s4[v] = p4[v] + s4[v];
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) x[e + v] = tsel == 0 ? s4[v] * a.scale : s4[v];
        }
        if (tsel == 0 && a.rope_cs != nullptr) {
            // dK_raw = R(-phi) dK on each pair (2p, 2p + 1) of the segment.
#pragma unroll
            for (int e = 0; e < EPC; e += 4) {
                const f32x4 wv = tab[u < NDK ? u : 0][e / 4];
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const float x0 = x[e + 2 * v], x1 = x[e + 2 * v + 1];
                    rope_rotate(x0, x1, wv[2 * v], -wv[2 * v + 1], &x[e + 2 * v], &x[e + 2 * v + 1]);
                }
            }
        }
        Vec16<T> out;
#pragma unroll
        for (int e = 0; e < EPC; ++e) out.set(e, from_f32<T>(x[e]));
        T* dst = (tsel == 0 ? dkp : dvp) + (((long long)b * a.T + key) * a.Hkv + kvh) * D + pt * EPC;
        st16(dst, out);
    }
}

// The same end of a dK/dV item for head_dim 128, whose kernels have no registers to spare: the
// partials are summed in NQH - 1 rounds through a region of one query block's size, in the
// same order, and the totals leave through LDS as 16-byte row segments.
template <typename T, int D, int NKH, int NQH, int BN, int NT>
__device__ __forceinline__ void dkdv_epilogue_rounds(const BwdArgs& a, char* smem, f32x16 (&dkacc)[D / 32],
                                              f32x16 (&dvacc)[D / 32], int j, int kvh, int b) {
    constexpr int NDB = D / 32;
    constexpr int EPC = 16 / sizeof(T);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int kh = w % NKH;
    const int qh = w / NKH;
    // Sum the dK/dV partials of the query blocks in LDS, last block first (fixed order:
    // deterministic).  The waves of query block 0 then hold the totals; they write them back
    // row-major per key half ([dK | dV][32 keys][D] floats, dK scaled by `scale`), and every
    // thread stores 16-byte row segments, with the inverse RoPE of dK applied pair by pair.
    float* red = reinterpret_cast<float*>(smem);
    const size_t rbase = (size_t)kh * 2 * NDB * 16 * 64;
    for (int o = NQH - 1; o >= 0; --o) {
        __syncthreads();
        if (qh == o) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const size_t ik = rbase + (size_t)db * 1024 + r * 64 + lane;
                    const size_t iv = ik + (size_t)NDB * 1024;
                    if (o < NQH - 1) {
                        dkacc[db][r] += red[ik];
                        dvacc[db][r] += red[iv];
                    }
                    if (o > 0) {
                        red[ik] = dkacc[db][r];
                        red[iv] = dvacc[db][r];
                    }
                }
        }
    }
    __syncthreads();  // every partial read
    if (qh == 0) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const size_t at = rbase + (size_t)acc_row(r, half) * D + db * 32 + l32;
                red[at] = dkacc[db][r] * a.scale;
                red[at + 32 * D] = dvacc[db][r];
            }
    }
    __syncthreads();
    constexpr int CPRo = D / EPC;       // 16-byte output chunks per row
    constexpr int NCHO = 2 * BN * CPRo;    // chunks of dK and dV
    T* __restrict__ dkp = static_cast<T*>(a.dk);
    T* __restrict__ dvp = static_cast<T*>(a.dv);
    for (int c = tid; c < NCHO; c += NT) {
        const int tsel = c / (BN * CPRo);
        const int cc = c % (BN * CPRo);
        const int kl = cc / CPRo, part = cc % CPRo;
        const int key = j * BN + kl;
        if (key >= a.T) continue;
        const float* src = red + (size_t)(kl >> 5) * 2 * NDB * 1024 + (size_t)tsel * 32 * D +
                           (size_t)(kl & 31) * D + part * EPC;
        float x[EPC];
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
            const f32x4 v4 = *reinterpret_cast<const f32x4*>(src + e);
#pragma unroll
            for (int u = 0; u < 4; ++u) x[e + u] = v4[u];
        }
        if (tsel == 0 && a.rope_cs != nullptr) {
            // dK_raw = R(-phi) dK on each pair (2p, 2p + 1) of the chunk.
            const float* tab = a.rope_cs + ((long long)key * (D / 2) + part * (EPC / 2)) * 2;
#pragma unroll
            for (int e = 0; e < EPC; e += 4) {
                const f32x4 w = *reinterpret_cast<const f32x4*>(tab + e);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const float x0 = x[e + 2 * u], x1 = x[e + 2 * u + 1];
                    rope_rotate(x0, x1, w[2 * u], -w[2 * u + 1], &x[e + 2 * u], &x[e + 2 * u + 1]);
                }
            }
        }
        Vec16<T> out;
#pragma unroll
        for (int e = 0; e < EPC; ++e) out.set(e, from_f32<T>(x[e]));
        T* dst = (tsel == 0 ? dkp : dvp) + (((long long)b * a.T + key) * a.Hkv + kvh) * D + part * EPC;
        st16(dst, out);
    }
}

template <typename T, int D, int NKH, int NQH, int BN, int NT>
__device__ __forceinline__ void dkdv_epilogue(const BwdArgs& a, char* smem, f32x16 (&dkacc)[D / 32],
                                              f32x16 (&dvacc)[D / 32], int j, int kvh, int b) {
    if constexpr (D <= 64)
        dkdv_epilogue_all<T, D, NKH, NQH, BN, NT>(a, smem, dkacc, dvacc, j, kvh, b);
    else
        dkdv_epilogue_rounds<T, D, NKH, NQH, BN, NT>(a, smem, dkacc, dvacc, j, kvh, b);
}

// One workgroup of the dK/dV role: key tile j of K/V head kvh in batch b.  Each wave takes
// 32 keys and QB blocks of 32 query rows per iteration; with QB = 2 the two blocks' products
// and exponentials are independent chains that the scheduler interleaves.
template <typename T, int D, int BM, int QB = 1, int BN_ = 64>
__device__ __forceinline__ void dkdv_role(const BwdArgs& a, char* smem, int j, int kvh, int b) {
    using C = DkdvCfg<T, D, BM, QB, BN_>;
    using M = Mfma<T>;
    using frag = typename M::frag;
    constexpr int KPL = C::KPL;
    constexpr int BN = C::BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int kh = w % C::NKH;
    const int qh = w / C::NKH;
    const int g = a.Hq / a.Hkv;

    const T* __restrict__ qp = static_cast<const T*>(a.q);
    const T* __restrict__ kp = static_cast<const T*>(a.k);
    const T* __restrict__ vp = static_cast<const T*>(a.v);
    const T* __restrict__ dop = static_cast<const T*>(a.dout);

    // Stationary K_j / V_j fragments ("split" over head_dim) for this wave's 32 keys.
    const int mykey = j * BN + kh * 32 + l32;
    frag kf[C::NS], vf[C::NS];
    {
        const bool ok = mykey < a.T;
        const long long off = (((long long)b * a.T + mykey) * a.Hkv + kvh) * D + half * (D / 2);
#pragma unroll
        for (int c = 0; c < (D / 2) / C::EPC; ++c) {
            const Vec16<T> kv = ok ? ld16(kp + off + c * C::EPC) : zero16<T>();
            const Vec16<T> vv = ok ? ld16(vp + off + c * C::EPC) : zero16<T>();
#pragma unroll
            for (int e = 0; e < C::EPC / KPL; ++e) {
                kf[c * (C::EPC / KPL) + e] = reinterpret_cast<const frag*>(&kv.raw)[e];
                vf[c * (C::EPC / KPL) + e] = reinterpret_cast<const frag*>(&vv.raw)[e];
            }
        }
    }

    f32x16 dkacc[C::NDB], dvacc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
        dkacc[db] = zero_acc();
        dvacc[db] = zero_acc();
    }
    // bf16 head_dim 128: the per-row -LSE/scale and -D ride in the 16-byte padding chunk of
    // each staged Q and dO row as three bf16 parts (pad_parts), and an extra matrix-core step
    // multiplies them by this fragment: (1, 1, 1, 0, ...) in the lower half's slots, zero in
    // the upper half's (whose lanes read the same chunk).  That replaces eight 16-byte LDS
    // reads per block (the rows' LSE and D, the same for every lane of a half) by two, for two
    // more matrix-core steps: measured 5.6% faster at head_dim 128 (eight steps per chain),
    // slower at head_dim 64 (four).
    constexpr bool FOLD = sizeof(T) == 2 && D >= 128;
    [[maybe_unused]] frag ones3{};
    if constexpr (FOLD) {
        const T one = (T)(half == 0 ? 1.0f : 0.0f);
        reinterpret_cast<T*>(&ones3)[0] = one;
        reinterpret_cast<T*>(&ones3)[1] = one;
        reinterpret_cast<T*>(&ones3)[2] = one;
    }

    // Iterations: every head of the group x every query tile on or below the diagonal (every
    // query tile without the causal mask).
    const int i0 = a.causal ? (j * BN) / BM : 0;
    const int nq = a.ntq - i0;
    const int niter = g * nq;

    // Staging of Q_i / dO_i (16-byte chunks, row-major), LSE and D: HBM -> registers -> LDS,
    // through NSET register sets (two for bf16 up to head_dim 64 with one query block per wave:
    // each stage's loads then have two iterations to land; one for fp32, for head_dim 128 and
    // for two query blocks per wave, whose registers are already spent on wider fragments and
    // accumulators).
    constexpr int NSET = (sizeof(T) == 2 && D < 128 && QB == 1) ? 2 : 1;
    struct Stg {
        Vec16<T> q[C::NCH], d[C::NCH];
        float l, t;
    };
    Stg sa;
    [[maybe_unused]] Stg sb;
    auto fetch = [&](Stg& st, int it) {
        Vec16<T>* qreg = st.q;
        Vec16<T>* dreg = st.d;
        const int head = kvh * g + it / nq;
        const int i = i0 + it % nq;
#pragma unroll
        for (int n = 0; n < C::NCH; ++n) {
            const int c = tid + n * C::NT;
            if (BM * C::CPR % C::NT == 0 || c < BM * C::CPR) {
                const int row = c / C::CPR, part = c % C::CPR;
                // Rows past the end load a real row instead: their P is 0 (LSE = +inf below),
                // so they contribute nothing, and the loads need no branch.
                const int t = min(i * BM + row, a.T - 1);
                const long long off = (((long long)b * a.T + t) * a.Hq + head) * D + part * C::EPC;
                qreg[n] = ld16(qp + off);
                dreg[n] = ld16(dop + off);
            }
        }
        if (tid < BM) {
            const int t = i * BM + tid;
            const long long ro = ((long long)b * a.Hq + head) * a.T;
            if constexpr (FOLD) {
                // -LSE / scale (rows past the end: a finite -2^100, so that P = 0 without an
                // infinity meeting the zero operands of the padding step).
                st.l = (t < a.T) ? -a.lse[ro + t] / a.scale : -0x1p100f;
                st.t = (t < a.T) ? -a.dt[ro + t] : 0.0f;
            } else {
                st.l = (t < a.T) ? a.lse[ro + t] * kLog2e : INFINITY;
                st.t = (t < a.T) ? -a.dt[ro + t] : 0.0f;  // staged negated: the dP accumulator starts from it
            }
        }
    };
    auto commit = [&](const Stg& st, int stage) {
        const Vec16<T>* qreg = st.q;
        const Vec16<T>* dreg = st.d;
        char* base = smem + stage * C::STAGE;
        T* Qs = reinterpret_cast<T*>(base + C::OFF_Q);
        T* dOs = reinterpret_cast<T*>(base + C::OFF_DO);
#pragma unroll
        for (int n = 0; n < C::NCH; ++n) {
            const int c = tid + n * C::NT;
            if (c < BM * C::CPR) {
                const int row = c / C::CPR, part = c % C::CPR;
                st16(&Qs[row * C::QS + part * C::EPC], qreg[n]);
                st16(&dOs[row * C::QS + part * C::EPC], dreg[n]);
            }
        }
        if (tid < BM) {
            if constexpr (FOLD) {
                st16(&Qs[tid * C::QS + D], pad_parts<T>(st.l));
                st16(&dOs[tid * C::QS + D], pad_parts<T>(st.t));
            } else {
                reinterpret_cast<float*>(base + C::OFF_LSE)[tid] = st.l;
                reinterpret_cast<float*>(base + C::OFF_DT)[tid] = st.t;
            }
        }
    };

    auto compute = [&](int it, int stage, auto masked) {
        constexpr bool MASK = decltype(masked)::value;
        const int i = i0 + it % nq;
        const char* base = smem + stage * C::STAGE;
        const T* Qs = reinterpret_cast<const T*>(base + C::OFF_Q);
        const T* dOs = reinterpret_cast<const T*>(base + C::OFF_DO);
        const float* lse2s = reinterpret_cast<const float*>(base + C::OFF_LSE);
        const float* ndts = reinterpret_cast<const float*>(base + C::OFF_DT);  // -D per row
        // S = Q K^T and dP - D = dO V^T - D on this wave's QB 32 x 32 blocks (lanes = keys).
        // FOLD: one more step per chain multiplies each row's padding chunk (the parts of
        // -LSE/scale, resp. -D) by (1, 1, 1, 0, ...), so S - LSE/scale and dP - D come out of
        // the matrix core.  Otherwise the dP accumulator starts from -D of its rows, read from
        // LDS straight into it (four 16-byte reads per block, rows acc_row(4 r4 + c, half)).
        // Either way dS = P (dP - D) is one multiply.
        f32x16 sacc[QB], dpacc[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            sacc[qb] = zero_acc();
            if constexpr (FOLD) {
                dpacc[qb] = zero_acc();
            } else {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(&ndts[qh * C::QW + qb * 32 + 8 * r4 + 4 * half]);
#pragma unroll
                    for (int c = 0; c < 4; ++c) dpacc[qb][4 * r4 + c] = d4[c];
                }
            }
        }
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int ro = (qh * C::QW + qb * 32 + l32) * C::QS + half * (D / 2) + s * KPL;
                sacc[qb] = M::mma(load_frag<T>(&Qs[ro]), kf[s], sacc[qb]);
                dpacc[qb] = M::mma(load_frag<T>(&dOs[ro]), vf[s], dpacc[qb]);
            }
        }
        if constexpr (FOLD) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int ro = (qh * C::QW + qb * 32 + l32) * C::QS + D;
                sacc[qb] = M::mma(load_frag<T>(&Qs[ro]), ones3, sacc[qb]);
                dpacc[qb] = M::mma(load_frag<T>(&dOs[ro]), ones3, dpacc[qb]);
            }
        }
        // P = exp(S - LSE) (masked where key > query); dS = P (dP - D), the second factor
        // being the dP accumulator itself.
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int lq0 = qh * C::QW + qb * 32 + 8 * r4 + 4 * half;
                [[maybe_unused]] f32x4 l4;
                if constexpr (!FOLD) l4 = *reinterpret_cast<const f32x4*>(&lse2s[lq0]);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int r = 4 * r4 + c;
                    float p = FOLD ? __builtin_amdgcn_exp2f(sacc[qb][r] * a.sl2)
                                   : __builtin_amdgcn_exp2f(sacc[qb][r] * a.sl2 - l4[c]);
                    if constexpr (MASK) {
                        if (mykey > i * BM + lq0 + c) p = 0.0f;
                    }
                    sacc[qb][r] = p;
                    dpacc[qb][r] = p * dpacc[qb][r];
                }
            }
        }
        // dV += P^T dO and dK += dS^T Q (contraction over this wave's queries).
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
            for (int ps = 0; ps < C::PS; ++ps) {
                const frag pf = acc_to_frag<T>(sacc[qb], ps * KPL);
                const frag dsf = acc_to_frag<T>(dpacc[qb], ps * KPL);
#pragma unroll
                for (int db = 0; db < C::NDB; ++db) {
                    const int r0 = qh * C::QW + qb * 32;
                    dvacc[db] = M::mma(pf, load_rows_frag<T>(dOs, C::QS, r0, ps, db * 32), dvacc[db]);
                    dkacc[db] = M::mma(dsf, load_rows_frag<T>(Qs, C::QS, r0, ps, db * 32), dkacc[db]);
                }
            }
        }
    };

    // Stage s sits in register set s % NSET until it is committed, at the start of iteration
    // s - 1; the set is then refilled with stage s + NSET.
    if (niter > 0) {
        fetch(sa, 0);
        commit(sa, 0);
    }
    // The K_j / V_j loads were issued before stage 0's, which the commit has waited for.
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
        settle(kf[s]);
        settle(vf[s]);
    }
    if constexpr (NSET == 2) {
        if (niter > 1) fetch(sb, 1);
        if (niter > 2) fetch(sa, 2);
    } else {
        if (niter > 1) fetch(sa, 1);
    }
    auto iteration = [&](int it, Stg& nxt) {
        __syncthreads();  // stage it&1 visible; stage (it+1)&1 free
        if (it + 1 < niter) {
            commit(nxt, (it + 1) & 1);
            if (it + 1 + NSET < niter) fetch(nxt, it + 1 + NSET);
        }
        const int i = i0 + it % nq;
        // Skip blocks whose keys all follow their queries; mask blocks crossing the diagonal.
        // Without the causal mask nothing is masked: keys past the end have K = V = 0 and
        // their dK / dV are never stored; queries past the end have P = 0 (LSE = +inf).
        const int kfirst = j * BN + kh * 32, qfirst = i * BM + qh * C::QW;
        if (a.causal && kfirst > qfirst + C::QW - 1) return;
        if (a.causal && kfirst + 31 > qfirst)
            compute(it, it & 1, std::true_type{});
        else
            compute(it, it & 1, std::false_type{});
    };
    if constexpr (NSET == 2) {
        for (int it = 0; it < niter; it += 2) {
            iteration(it, sb);
            if (it + 1 < niter) iteration(it + 1, sa);
        }
    } else {
        for (int it = 0; it < niter; ++it) iteration(it, sa);
    }

    dkdv_epilogue<T, D, C::NKH, C::NQH, BN, C::NT>(a, smem, dkacc, dvacc, j, kvh, b);
}

// ---------------------------------------------------------------------------------------
// 2b. dK, dV for bf16 head_dim 64: Q / dO stages copied HBM -> LDS by the load unit.
// ---------------------------------------------------------------------------------------
// The same item as dkdv_role, but each stage of Q and dO rows goes from global memory straight
// into LDS (global_load_lds_dwordx4: each instruction fills 1 KB, lane l at byte 16 l) with no
// register staging and no LDS stores of those rows.  Rows are 128 bytes, unpadded, with their
// 16-byte chunks permuted by swz64 so that both kinds of read are free of bank conflicts:
//  * the 16-byte "split" reads (lanes 0-15: the same logical chunk of 16 consecutive rows)
//    land on 16 distinct 16-byte bank groups;
//  * the transposing reads (32 lanes: 4 consecutive rows x 64 bytes) land on 4 distinct
//    64-byte bank groups.
// LSE (times log2 e) and -D of a stage go through registers: loaded by every thread in the
// iteration that issues the stage's copies, stored to LDS by the first BM threads at its end.
// The compiler's wait for those loads is a wait for every vector-memory operation (it does not
// count the copies into LDS as later operations), so a stage's copies have one compute phase
// to land, as with register staging: NST = 2 buffers suffice.  The waits before the barriers
// are explicit (the compiler's own would be placed at every LDS access).

// Stored chunk of logical chunk c in row r is c ^ swz64(r) (a permutation of bits 1-3 of r).
__device__ __host__ constexpr inline int swz64(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

typedef __attribute__((address_space(3))) void lds_void;

template <int BM, int QB, int BN_, int NST_>
struct DkdvDmaCfg {
    static constexpr int D = 64;
    static constexpr int NST = NST_;
    static constexpr int BN = BN_;
    static constexpr int NKH = BN / 32;
    static constexpr int QW = 32 * QB;
    static constexpr int NQH = BM / QW;
    static constexpr int NW = NKH * NQH;
    static constexpr int NT = 64 * NW;
    static constexpr int NS = 4;      // MFMA steps over head_dim
    static constexpr int NDB = 2;
    static constexpr int TILE = BM * 128;
    static constexpr size_t OFF_Q = 0;
    static constexpr size_t OFF_DO = TILE;
    static constexpr size_t OFF_LSE = 2 * (size_t)TILE;
    static constexpr size_t OFF_DT = OFF_LSE + sizeof(float) * BM;
    static constexpr size_t STAGE = OFF_DT + sizeof(float) * BM;
    static constexpr size_t BYTES = NST * STAGE;
    static constexpr int NPIECE = BM / 8;          // 1 KB copies per tile
    static constexpr int PPW = NPIECE / NW;        // copies per wave per tile
    static constexpr size_t LDS = BYTES > dkdv_epi_bytes<D, NKH, NQH>() ? BYTES : dkdv_epi_bytes<D, NKH, NQH>();
    static_assert(NPIECE % NW == 0, "every wave issues the same number of copies");
    static_assert(STAGE % 16 == 0, "stage alignment");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// s_waitcnt vmcnt(N) lgkmcnt(0), then s_barrier: this wave's vector-memory operations but the
// last N have completed (its copies into LDS included), and so have its LDS accesses.  Written
// as one asm statement so that no memory access moves across it.
template <int N>
__device__ inline void vm_wait_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Operand fragment from two transposing reads (rows r .. r+3, then r+8 .. r+11).
__device__ inline bf16x8 tr_join(i16x4 x, i16x4 y) {
    bf16x8 f;
    const bf16x4 a = __builtin_bit_cast(bf16x4, x);
    const bf16x4 c = __builtin_bit_cast(bf16x4, y);
    f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
    f[4] = c[0]; f[5] = c[1]; f[6] = c[2]; f[7] = c[3];
    return f;
}

// The transposing reads of one 16-row step of a 32-row block, for both head_dim halves of Q
// (at LDS byte addresses lo[db] / hi[db]) and of dO (OFF bytes further): eight reads in one asm
// statement that also waits for them.  (Issued through the builtin, each transposing read makes
// the compiler wait for every copy into LDS still in flight, the later stages' included; here
// the wait covers LDS accesses only.)
template <int OFF>
__device__ inline void tr_reads8(const unsigned (&lo)[2], const unsigned (&hi)[2], bf16x8 (&qt)[2], bf16x8 (&dt)[2]) {
    i16x4 q0, q1, q2, q3, d0, d1, d2, d3;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %6, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(q0), "=&v"(q1), "=&v"(q2), "=&v"(q3), "=&v"(d0), "=&v"(d1), "=&v"(d2), "=&v"(d3)
        : "v"(lo[0]), "v"(hi[0]), "v"(lo[1]), "v"(hi[1]), "n"(OFF)
        : "memory");
    qt[0] = tr_join(q0, q1);
    qt[1] = tr_join(q2, q3);
    dt[0] = tr_join(d0, d1);
    dt[1] = tr_join(d2, d3);
}

template <int BM, int QB, int BN_, int NST>
__device__ __forceinline__ void dkdv_role_dma(const BwdArgs& a, char* smem, int j, int kvh, int b) {
    using C = DkdvDmaCfg<BM, QB, BN_, NST>;
    using T = bf16;
    using M = Mfma<T>;
    using frag = typename M::frag;
    constexpr int D = 64;
    constexpr int KPL = 8;
    constexpr int BN = C::BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int kh = w % C::NKH;
    const int qh = w / C::NKH;
    const int g = a.Hq / a.Hkv;

    const T* __restrict__ qp = static_cast<const T*>(a.q);
    const T* __restrict__ kp = static_cast<const T*>(a.k);
    const T* __restrict__ vp = static_cast<const T*>(a.v);
    const T* __restrict__ dop = static_cast<const T*>(a.dout);

    // Stationary K_j / V_j fragments ("split" over head_dim) for this wave's 32 keys.
    const int mykey = j * BN + kh * 32 + l32;
    frag kf[C::NS], vf[C::NS];
    {
        const bool ok = mykey < a.T;
        const long long off = (((long long)b * a.T + mykey) * a.Hkv + kvh) * D + half * (D / 2);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const Vec16<T> kv = ok ? ld16(kp + off + c * 8) : zero16<T>();
            const Vec16<T> vv = ok ? ld16(vp + off + c * 8) : zero16<T>();
            kf[c] = reinterpret_cast<const frag*>(&kv.raw)[0];
            vf[c] = reinterpret_cast<const frag*>(&vv.raw)[0];
        }
    }
    f32x16 dkacc[C::NDB], dvacc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
        dkacc[db] = zero_acc();
        dvacc[db] = zero_acc();
    }

    const int i0 = a.causal ? (j * BN) / BM : 0;
    const int nq = a.ntq - i0;
    const int niter = g * nq;

    // Copies of stage it into buffer buf (this wave's PPW pieces of Q and of dO): piece n covers
    // rows 8n .. 8n+7; lane l fills row 8n + l/8, stored chunk l%8, i.e. logical chunk
    // (l%8) ^ swz64(row).  Rows past the end copy row T-1 instead (their P is 0: LSE = +inf).
    auto dma = [&](int it, int buf) {
        const int head = kvh * g + it / nq;
        const int i = i0 + it % nq;
        char* base = smem + buf * C::STAGE;
#pragma unroll
        for (int u = 0; u < C::PPW; ++u) {
            const int n = w * C::PPW + u;
            const int row = 8 * n + (lane >> 3);
            const int c = (lane & 7) ^ swz64(row);
            const int t = min(i * BM + row, a.T - 1);
            const long long off = (((long long)b * a.T + t) * a.Hq + head) * D + c * 8;
            __builtin_amdgcn_global_load_lds(qp + off, (lds_void*)(base + C::OFF_Q + n * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(dop + off, (lds_void*)(base + C::OFF_DO + n * 1024), 16, 0, 0);
        }
    };
    // LSE and D of the stage's rows, loaded raw by every thread (row tid % BM) and stored by the
    // first BM threads as LSE * log2(e) and -D (+inf and 0 past the end).  The loads and copies
    // of a stage are issued unconditionally (past the last stage, the last one is copied again
    // into the free buffer), so that every iteration runs the same straight-line sequence.
    auto fetch_ld = [&](int it, float& l, float& d) {
        const int head = kvh * g + it / nq;
        const int t = min((i0 + it % nq) * BM + (tid % BM), a.T - 1);
        const long long ro = ((long long)b * a.Hq + head) * a.T;
        l = a.lse[ro + t];
        d = a.dt[ro + t];
    };
    // (The two LDS stores are written in asm: for an LDS store it can see, the compiler would
    // first wait for every copy into LDS in flight.)
    auto commit_ld = [&](int it, int buf, float l, float d) {
        if (tid < BM) {
            const bool in = (i0 + it % nq) * BM + tid < a.T;
            const float lv = in ? l * kLog2e : INFINITY;
            const float dv = in ? -d : 0.0f;
            const unsigned at = (unsigned)(uintptr_t)(smem + buf * C::STAGE + C::OFF_LSE) + 4 * tid;
            asm volatile("ds_write_b32 %0, %1\n\tds_write_b32 %0, %2 offset:%3" ::"v"(at), "v"(lv), "v"(dv),
                         "n"(4 * BM)
                         : "memory");
        }
    };

    // Lane offsets of the reads.  Split: row l32 of a 32-row block, logical chunk 4 half + s.
    // Transposing: rows 4 half + (jj >> 2) (and + 8) of a 16-row block, logical chunk
    // 4 db + 2 grp + ((jj >> 1) & 1), byte 8 (jj & 1) of it.
    int soff[C::NS];
#pragma unroll
    for (int s = 0; s < C::NS; ++s) soff[s] = l32 * 128 + (((4 * half + s) ^ swz64(l32)) << 4);
    unsigned tlo[C::NDB], thi[C::NDB];
    {
        const int jj = lane & 15, grp = (lane >> 4) & 1;
        const int r = 4 * half + (jj >> 2);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            const int c = 4 * db + 2 * grp + ((jj >> 1) & 1);
            tlo[db] = r * 128 + ((c ^ swz64(r)) << 4) + 8 * (jj & 1);
            thi[db] = (r + 8) * 128 + ((c ^ swz64(r + 8)) << 4) + 8 * (jj & 1);
        }
    }

    auto compute = [&](int it, auto masked) {
        constexpr bool MASK = decltype(masked)::value;
        const int i = i0 + it % nq;
        const char* base = smem + (it % NST) * C::STAGE;
        const char* qb0 = base + C::OFF_Q + (size_t)qh * C::QW * 128;  // this wave's first row
        const float* lse2s = reinterpret_cast<const float*>(base + C::OFF_LSE);
        const float* ndts = reinterpret_cast<const float*>(base + C::OFF_DT);
        f32x16 sacc[QB], dpacc[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            sacc[qb] = zero_acc();
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(&ndts[qh * C::QW + qb * 32 + 8 * r4 + 4 * half]);
#pragma unroll
                for (int c = 0; c < 4; ++c) dpacc[qb][4 * r4 + c] = d4[c];
            }
        }
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const char* p = qb0 + qb * 32 * 128 + soff[s];
                sacc[qb] = M::mma(*reinterpret_cast<const frag*>(p), kf[s], sacc[qb]);
                dpacc[qb] = M::mma(*reinterpret_cast<const frag*>(p + C::TILE), vf[s], dpacc[qb]);
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int lq0 = qh * C::QW + qb * 32 + 8 * r4 + 4 * half;
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2s[lq0]);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int r = 4 * r4 + c;
                    float p = __builtin_amdgcn_exp2f(sacc[qb][r] * a.sl2 - l4[c]);
                    if constexpr (MASK) {
                        if (mykey > i * BM + lq0 + c) p = 0.0f;
                    }
                    sacc[qb][r] = p;
                    dpacc[qb][r] = p * dpacc[qb][r];
                }
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
            for (int ps = 0; ps < 2; ++ps) {
                const frag pf = acc_to_frag<T>(sacc[qb], ps * KPL);
                const frag dsf = acc_to_frag<T>(dpacc[qb], ps * KPL);
                const unsigned rb = (unsigned)(uintptr_t)(qb0 + (qb * 32 + 16 * ps) * 128);
                const unsigned lo[2] = {rb + tlo[0], rb + tlo[1]};
                const unsigned hi[2] = {rb + thi[0], rb + thi[1]};
                frag qt[2], dt[2];
                tr_reads8<C::TILE>(lo, hi, qt, dt);
#pragma unroll
                for (int db = 0; db < C::NDB; ++db) {
                    dvacc[db] = M::mma(pf, dt[db], dvacc[db]);
                    dkacc[db] = M::mma(dsf, qt[db], dkacc[db]);
                }
            }
        }
    };

    if (niter <= 0) {
        dkdv_epilogue<T, D, C::NKH, C::NQH, BN, C::NT>(a, smem, dkacc, dvacc, j, kvh, b);
        return;
    }
    // Prologue: stage 0.
    static_assert(NST == 2, "the loop below is written for two stages");
    {
        float l0, d0;
        fetch_ld(0, l0, d0);
        dma(0, 0);
        commit_ld(0, 0, l0, d0);
    }
    // The K_j / V_j loads were issued first; wait for them here, once.
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
        settle(kf[s]);
        settle(vf[s]);
    }
    for (int it = 0; it < niter; ++it) {
        // This wave's copies of stage it complete, then the barrier: every wave's copies of
        // stage it have landed, and every wave is done with iteration it - 1, whose buffer the
        // copies of stage it + 1 refill.
        vm_wait_barrier<0>();
        const int nx = min(it + 1, niter - 1);
        const int nbuf = (it + 1) % NST;
        float lreg, dreg;
        fetch_ld(nx, lreg, dreg);
        dma(nx, nbuf);
        const int i = i0 + it % nq;
        const int kfirst = j * BN + kh * 32, qfirst = i * BM + qh * C::QW;
        if (!(a.causal && kfirst > qfirst + C::QW - 1)) {
            if (a.causal && kfirst + 31 > qfirst)
                compute(it, std::true_type{});
            else
                compute(it, std::false_type{});
        }
        commit_ld(nx, nbuf, lreg, dreg);
    }
    // The copies of the repeated last stage may still be in flight: the reduction reuses the LDS.
    vm_wait_barrier<0>();
    dkdv_epilogue<T, D, C::NKH, C::NQH, BN, C::NT>(a, smem, dkacc, dvacc, j, kvh, b);
}

// ---------------------------------------------------------------------------------------
// 3. dQ: Q-stationary, shaped like the forward.
// ---------------------------------------------------------------------------------------
// A stage holds SUB consecutive key tiles of BN keys: one barrier per stage, the tiles of a
// stage taken one after the other by every wave.
template <typename T, int D, int BN, int NW, int SUB = 1>
struct DqCfg {
    static constexpr int KPL = Mfma<T>::KPL;
    static constexpr int NS = D / (2 * KPL);
    static constexpr int NKB = BN / 32;
    static constexpr int NDB = D / 32;
    static constexpr int PS = 16 / KPL;
    static constexpr int EPC = 16 / sizeof(T);
    static constexpr int CPR = D / EPC;
    static constexpr int KS = D + EPC;   // row-major K / V stride (16 bytes of padding)
    static constexpr int NT = 64 * NW;
    static constexpr int SK = SUB * BN;  // keys per stage
    static constexpr int NCH = (SK * CPR + NT - 1) / NT;  // chunks per thread per tensor
    static constexpr int KBUF = SK * KS;
    static constexpr int STAGE = 2 * KBUF;  // K, V row-major
    // Up to head_dim 64 the (cos, sin) rows of the workgroup's query rows (inverse RoPE of dQ)
    // are staged once in LDS behind the two stages; TAB_ROWS is the most query rows a
    // workgroup takes (32 per wave of a head, at most four waves per head).
    static constexpr bool TAB = D <= 64;
    static constexpr int TAB_ROWS = 128;
    static constexpr size_t TAB_OFF = 2 * (size_t)STAGE * sizeof(T);
    static constexpr size_t BYTES = TAB_OFF + (TAB ? (size_t)TAB_ROWS * D * sizeof(float) : 0);
};

// One workgroup of the dQ role: item it (0 = the longest query tile) of K/V head kvh in
// batch b.  Waves beyond G * WPH stay in the staging loop but never compute.
template <typename T, int D, int BN, int NW, int SUB = 1>
__device__ __forceinline__ void dq_role(const BwdArgs& a, char* smem_raw, int it, int kvh, int b) {
    using C = DqCfg<T, D, BN, NW, SUB>;
    using M = Mfma<T>;
    using frag = typename M::frag;
    constexpr int KPL = C::KPL;

    T* smem = reinterpret_cast<T*>(smem_raw);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int half = lane >> 5;
    const int l32 = lane & 31;

    const int tile = a.ntq_dq - 1 - it / a.nhc;
    const int hc = it % a.nhc;
    const int g = a.Hq / a.Hkv;
    const int BM = a.WPH * 32;
    const bool wave_used = w < a.G * a.WPH;
    const int hs = wave_used ? w / a.WPH : 0;
    const int sub = wave_used ? w % a.WPH : 0;
    const int head = kvh * g + hc * a.G + hs;
    const int q0 = tile * BM + sub * 32;
    const bool active = wave_used && q0 < a.T;
    const int wg_last = min(tile * BM + BM, a.T) - 1;
    const int jmax = (a.causal ? wg_last : a.T - 1) / C::SK;  // last stage
    const int tq = q0 + l32;  // this lane's query
    const int lim = a.causal ? tq : a.T - 1;  // last key it sees

    const T* __restrict__ qp = static_cast<const T*>(a.q);
    const T* __restrict__ kp = static_cast<const T*>(a.k);
    const T* __restrict__ vp = static_cast<const T*>(a.v);
    const T* __restrict__ dop = static_cast<const T*>(a.dout);
    const long long kv_row0 = (long long)b * a.T;

    // Q and dO fragments ("split" over head_dim), LSE and D of this lane's query.
    constexpr int NC = (D / 2) / C::EPC;  // chunks per half row
    frag qf[C::NS], df[C::NS];
    float lse2 = INFINITY, dtv = 0.0f;
    if (active && tq < a.T) {
        const long long off = (((long long)b * a.T + tq) * a.Hq + head) * D + half * (D / 2);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const Vec16<T> qv = ld16(qp + off + c * C::EPC);
            const Vec16<T> dv = ld16(dop + off + c * C::EPC);
#pragma unroll
            for (int e = 0; e < C::EPC / KPL; ++e) {
                qf[c * (C::EPC / KPL) + e] = reinterpret_cast<const frag*>(&qv.raw)[e];
                df[c * (C::EPC / KPL) + e] = reinterpret_cast<const frag*>(&dv.raw)[e];
            }
        }
        const long long ro = ((long long)b * a.Hq + head) * a.T + tq;
        lse2 = a.lse[ro] * kLog2e;
        dtv = a.dt[ro];
    } else {
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
            qf[s] = frag{};
            df[s] = frag{};
        }
    }

    // Staging of one K/V tile, row-major 16-byte chunks, through NSET register sets (two for
    // bf16 up to head_dim 64, so that each tile's loads have two iterations to land; one for
    // head_dim 128, which keeps the kernel within 256 registers).
    constexpr int NSET = (sizeof(T) == 2 && D < 128 && SUB == 1) ? 2 : 1;
    struct Stg {
        Vec16<T> k[C::NCH], v[C::NCH];
    };
    Stg sa;
    [[maybe_unused]] Stg sb;
    auto fetch = [&](Stg& st, int j) {
        Vec16<T>* kreg = st.k;
        Vec16<T>* vreg = st.v;
#pragma unroll
        for (int n = 0; n < C::NCH; ++n) {
            const int c = tid + n * C::NT;
            if (c < C::SK * C::CPR) {
                const int key = c / C::CPR, part = c % C::CPR;
                const int s = j * C::SK + key;
                // Keys past the end load a real row instead: they only occur in diagonal
                // tiles, where the mask zeroes them, and the loads need no branch.
                const long long off = ((kv_row0 + min(s, a.T - 1)) * a.Hkv + kvh) * D + part * C::EPC;
                kreg[n] = ld16(kp + off);
                vreg[n] = ld16(vp + off);
            }
        }
    };
    auto commit = [&](const Stg& st, int stage) {
        const Vec16<T>* kreg = st.k;
        const Vec16<T>* vreg = st.v;
        T* Ks = smem + stage * C::STAGE;
        T* Vs = Ks + C::KBUF;
#pragma unroll
        for (int n = 0; n < C::NCH; ++n) {
            const int c = tid + n * C::NT;
            if (c < C::SK * C::CPR) {
                const int key = c / C::CPR, part = c % C::CPR;
                st16(&Ks[key * C::KS + part * C::EPC], kreg[n]);
                st16(&Vs[key * C::KS + part * C::EPC], vreg[n]);
            }
        }
    };

    f32x16 dqacc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) dqacc[db] = zero_acc();

    // One key tile: keys j * BN .. + BN - 1, at row u * BN of the stage in LDS.
    auto compute = [&](int j, int stage, int u, auto masked) {
        constexpr bool MASK = decltype(masked)::value;
        const T* Ks = smem + stage * C::STAGE + u * BN * C::KS;
        const T* Vs = smem + stage * C::STAGE + C::KBUF + u * BN * C::KS;
        // The dP accumulator starts from -D of the lane's query where registers allow (16 more
        // live before the products; the twelve-wave and head_dim-128 shapes would spill), so
        // that dS = P (dP - D) is one multiply; elsewhere D is subtracted afterwards.
        constexpr bool DINIT = (sizeof(T) == 2 && D <= 64 && NW <= 8) || (sizeof(T) == 4 && D <= 32);
        f32x16 sacc[C::NKB], pacc[C::NKB];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
            sacc[kb] = zero_acc();
            if constexpr (DINIT) {
#pragma unroll
                for (int r = 0; r < 16; ++r) pacc[kb][r] = -dtv;
            } else {
                pacc[kb] = zero_acc();
            }
        }
        // S^T = K Q^T and dP^T (- D) = V dO^T (- D) (lanes = queries, registers = keys).
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
                const int ro = (kb * 32 + l32) * C::KS + half * (D / 2) + s * KPL;
                sacc[kb] = M::mma(load_frag<T>(&Ks[ro]), qf[s], sacc[kb]);
                pacc[kb] = M::mma(load_frag<T>(&Vs[ro]), df[s], pacc[kb]);
            }
        }
        // dS^T = P^T (dP^T - D), P^T = exp(S^T - LSE).
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = __builtin_amdgcn_exp2f(sacc[kb][r] * a.sl2 - lse2);
                if constexpr (MASK) {
                    if (j * BN + kb * 32 + acc_row(r, half) > lim) p = 0.0f;
                }
                pacc[kb][r] = DINIT ? p * pacc[kb][r] : p * (pacc[kb][r] - dtv);
            }
        }
        // dQ^T += K^T dS^T.
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
            for (int ps = 0; ps < C::PS; ++ps) {
                const frag dsf = acc_to_frag<T>(pacc[kb], ps * KPL);
#pragma unroll
                for (int db = 0; db < C::NDB; ++db) {
                    const frag kt = load_rows_frag<T>(Ks, C::KS, kb * 32, ps, db * 32);
                    dqacc[db] = M::mma(kt, dsf, dqacc[db]);
                }
            }
        }
    };

    // The (cos, sin) rows of this workgroup's query rows, [BM][D] floats, staged in LDS by
    // 16-byte pieces while tile 0 is in flight (used only after the loop).
    constexpr int TPT = C::TAB ? (C::TAB_ROWS * D / 4 + C::NT - 1) / C::NT : 0;  // pieces per thread
    [[maybe_unused]] f32x4 tabv[TPT > 0 ? TPT : 1];
    const bool stage_tab = C::TAB && a.rope_cs != nullptr && BM <= C::TAB_ROWS;
    if (stage_tab) {
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
            const int c = tid + u * C::NT;  // piece: row c / (D / 4), floats 4 (c % (D / 4)) ..
            const int t = min(tile * BM + min(c / (D / 4), BM - 1), a.T - 1);
            tabv[u] = *reinterpret_cast<const f32x4*>(a.rope_cs + (long long)t * D + 4 * (c % (D / 4)));
        }
    }
    // Tile s sits in register set s % NSET until it is committed at the start of iteration
    // s - 1; the set is then refilled with tile s + NSET.
    fetch(sa, 0);
    commit(sa, 0);
    if (stage_tab) {
        float* tabs = reinterpret_cast<float*>(smem_raw + C::TAB_OFF);
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
            const int c = tid + u * C::NT;
            if (c < BM * D / 4) *reinterpret_cast<f32x4*>(tabs + 4 * c) = tabv[u];
        }
    }
    // The LSE / D loads were issued before tile 0's, which the commit has waited for.
    settle(lse2);
    settle(dtv);
    if constexpr (NSET == 2) {
        if (jmax >= 1) fetch(sb, 1);
        if (jmax >= 2) fetch(sa, 2);
    } else {
        if (jmax >= 1) fetch(sa, 1);
    }
    const int qlast = min(q0 + 32, a.T) - 1;
    // Causal: tiles from the diagonal's on are masked.  Otherwise only a ragged last tile.
    const int jfirst_masked = a.causal ? q0 / BN : ((a.T % BN) ? (a.T - 1) / BN : INT_MAX);
    auto iteration = [&](int j, Stg& nxt) {
        __syncthreads();
        if (j + 1 <= jmax) {
            commit(nxt, (j + 1) & 1);
            if (j + 1 + NSET <= jmax) fetch(nxt, j + 1 + NSET);
        }
        if (!active) return;
#pragma unroll 1
        for (int u = 0; u < SUB; ++u) {
            const int jt = j * SUB + u;  // key tile
            if ((a.causal && jt * BN > qlast) || jt * BN >= a.T) break;
            if (jt >= jfirst_masked)
                compute(jt, j & 1, u, std::true_type{});
            else
                compute(jt, j & 1, u, std::false_type{});
        }
    };
    if constexpr (NSET == 2) {
        for (int j = 0; j <= jmax; j += 2) {
            iteration(j, sb);
            if (j + 1 <= jmax) iteration(j + 1, sa);
        }
    } else {
        for (int j = 0; j <= jmax; ++j) iteration(j, sa);
    }

    if (!active || tq >= a.T) return;
    if (a.rope_cs != nullptr) {
        // dQ_raw = R(-phi) dQ.  Pair (d, d+1) sits in registers (r, r+1), r even, of this lane;
        // one 16-byte table read gives (cos, sin) of two consecutive pairs.
        const float4* cs = stage_tab ? reinterpret_cast<const float4*>(smem_raw + C::TAB_OFF) + (tq - tile * BM) * (D / 4)
                                     : reinterpret_cast<const float4*>(a.rope_cs + (long long)tq * D);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const float4 w = cs[(db * 32 + 8 * a4 + 4 * half) / 4];
                f32x16& x = dqacc[db];
                const int r = 4 * a4;
                const float x0 = x[r], x1 = x[r + 1], x2 = x[r + 2], x3 = x[r + 3];
                float y0, y1, y2, y3;
                rope_rotate(x0, x1, w.x, -w.y, &y0, &y1);
                rope_rotate(x2, x3, w.z, -w.w, &y2, &y3);
                x[r] = y0;
                x[r + 1] = y1;
                x[r + 2] = y2;
                x[r + 3] = y3;
            }
    }
    T* __restrict__ dqp = static_cast<T*>(a.dq);
    T* row = dqp + (((long long)b * a.T + tq) * a.Hq + head) * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
            const int d0 = db * 32 + 8 * a4 + 4 * half;
            if constexpr (sizeof(T) == 2) {
                bf16x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (bf16)(dqacc[db][4 * a4 + e] * a.scale);
                *reinterpret_cast<bf16x4*>(row + d0) = v;
            } else {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = dqacc[db][4 * a4 + e] * a.scale;
                *reinterpret_cast<f32x4*>(row + d0) = v;
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// One launch for both roles.  Items are numbered per (batch, K/V head): dK/dV items
// j = 0 .. ntk-1 (key tile j, heaviest first) and dQ items i = 0 .. nqi-1 (heaviest first).
// With both roles, the items are dispatched in decreasing order of their estimated cost
// (longest first, from a table the host sorts), so the longest items start first and the
// short ones fill in behind them; when a (batch, K/V head) has more items than the table
// holds, the two lists are merged by relative position (j/ntk vs i/nqi) instead.
// ---------------------------------------------------------------------------------------
struct Sched {
    int ntk, nqi;
};

__device__ inline int dkdv_rank(int j, const Sched& s) {  // merged position of dK/dV item j
    return j + (int)(((long long)j * s.nqi + s.ntk - 1) / s.ntk);
}

// bf16 head_dim 64 takes the dK/dV role with direct copies into LDS (dkdv_role_dma).
template <typename T, int D>
constexpr bool kDkdvDma = sizeof(T) == 2 && D == 64;
// One 32-row query block per wave in the shared launch (two, over 256-row stages, measured
// slower at T=1024); two LDS stages (three measured 1-2% slower).
constexpr int kDmaQbShared = 1;      // query blocks per wave, shared launch
constexpr int kDmaStagesShared = 2;  // LDS stages of the shared launch's dK/dV role
constexpr int kDmaStagesSolo = 2;    // and of the separate dK/dV kernel

template <typename T, int D, int NW>
struct BwdKernelCfg {
    // dK/dV role: 2 key halves x NW/2 query blocks of 32 (or 64) rows
    static constexpr int BM = (kDkdvDma<T, D> ? 16 * kDmaQbShared : 16) * NW;
    static constexpr int BNQ = (D == 128) ? 32 : 64;  // dQ role key tile
    using Dk = DkdvCfg<T, D, 16 * NW>;
    using Dq = DqCfg<T, D, BNQ, NW>;
    static constexpr size_t DQ_BYTES = Dq::BYTES;
    static constexpr size_t DK_BYTES = kDkdvDma<T, D> ? DkdvDmaCfg<BM, kDmaQbShared, 64, kDmaStagesShared>::LDS : Dk::LDS;
    static constexpr size_t BYTES = DK_BYTES > DQ_BYTES ? DK_BYTES : DQ_BYTES;
    static_assert(Dk::NW == NW, "dK/dV role must use every wave");
    static_assert(!kDkdvDma<T, D> || DkdvDmaCfg<BM, kDmaQbShared, 64, kDmaStagesShared>::NW == NW, "waves");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <typename T, int D, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_kernel(BwdArgs a) {
    using K = BwdKernelCfg<T, D, NW>;
    __shared__ __attribute__((aligned(16))) char smem[K::BYTES];
    const int HB = a.B * a.Hkv;
    const int m = blockIdx.x / HB;
    const int rem = blockIdx.x % HB;
    const int kvh = rem % a.Hkv;
    const int b = rem / a.Hkv;
    const int nqi = a.ntq_dq * a.nhc;
    bool is_dkdv;
    int item;
    if (a.roles == 1) {
        is_dkdv = true;
        item = m;
    } else if (a.roles == 2) {
        is_dkdv = false;
        item = m;
    } else if (a.norder > 0) {
        const int e = a.order[m];
        is_dkdv = e < 0x8000;
        item = is_dkdv ? e : e - 0x8000;
    } else {
        // Largest j with dkdv_rank(j) <= m (dkdv_rank is increasing, dkdv_rank(0) = 0).
        const Sched sc{a.ntk, nqi};
        int lo = 0, hi = a.ntk - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (dkdv_rank(mid, sc) <= m) lo = mid;
            else hi = mid - 1;
        }
        is_dkdv = dkdv_rank(lo, sc) == m;
        item = is_dkdv ? lo : m - (lo + 1);
    }
    if (is_dkdv) {
        if constexpr (kDkdvDma<T, D>)
            dkdv_role_dma<K::BM, kDmaQbShared, 64, kDmaStagesShared>(a, smem, item, kvh, b);
        else
            dkdv_role<T, D, K::BM>(a, smem, item, kvh, b);
    } else
        dq_role<T, D, K::BNQ, NW>(a, smem, item, kvh, b);
}

// The dQ role alone, with only its own LDS; NW may exceed the dK/dV role's wave count.
template <typename T, int D, int NW>
// bf16 head_dim 128 (32-key tiles, one staging register set) fits 256 registers: two
// workgroups per CU, two waves per SIMD.  Twelve waves (three per SIMD, 168 registers) take
// 32-key tiles too: with 64-key tiles the kernel spills.
// The twelve-wave kernel stages four 32-key tiles per barrier (measured at T=8192: 8% faster
// than one tile per barrier, two tiles halfway).
__global__ __launch_bounds__(64 * NW, (sizeof(T) == 2 && D >= 128) ? 2 : 1) void bwd_dq_kernel(BwdArgs a) {
    constexpr int BNQ = (D == 128 || NW == 12) ? 32 : 64;
    constexpr int SUB = (sizeof(T) == 2 && NW == 12) ? 4 : 1;
    using Dq = DqCfg<T, D, BNQ, NW, SUB>;
    __shared__ __attribute__((aligned(16))) char smem[Dq::BYTES];
    const int HB = a.B * a.Hkv;
    const int m = blockIdx.x / HB;
    const int rem = blockIdx.x % HB;
    dq_role<T, D, BNQ, NW, SUB>(a, smem, m, rem % a.Hkv, rem / a.Hkv);
}

// The dK/dV role in a launch of its own (bf16, large problems): waves of 32 keys x two 32-row
// query blocks (two independent chains for the scheduler) over 128-row stages.  Up to head_dim
// 64 a workgroup takes 128 keys as eight waves, so each staged Q / dO tile feeds twice as many
// keys as in the shared launch's 64-key workgroups (half the load traffic per product); head
// dim 128 takes 64 keys as four waves (460 registers: one wave per SIMD, 139 KB of LDS).
template <typename T, int D>
struct DkdvSolo {
    static constexpr int BN = D <= 64 ? 128 : 64;
    using Cfg = DkdvCfg<T, D, 128, 2, BN>;
    static constexpr int NT = 64 * Cfg::NW;
    static constexpr size_t BYTES = kDkdvDma<T, D> ? DkdvDmaCfg<128, 2, BN, kDmaStagesSolo>::LDS : Cfg::LDS;
};
template <typename T, int D>
__global__ __launch_bounds__((DkdvSolo<T, D>::NT), 1) void bwd_dkdv_kernel(BwdArgs a) {
    using S = DkdvSolo<T, D>;
    __shared__ __attribute__((aligned(16))) char smem[S::BYTES];
    const int HB = a.B * a.Hkv;
    const int m = blockIdx.x / HB;
    const int rem = blockIdx.x % HB;
    if constexpr (kDkdvDma<T, D>)
        dkdv_role_dma<128, 2, S::BN, kDmaStagesSolo>(a, smem, m, rem % a.Hkv, rem / a.Hkv);
    else
        dkdv_role<T, D, 128, 2, S::BN>(a, smem, m, rem % a.Hkv, rem / a.Hkv);
}

template <typename T, int D>
hipError_t launch_pre_t(const void* o, const void* dout, float* dtbuf, int B, int seq, int Hq,
                        float* cs, const RopeArgs* rope, hipStream_t stream) {
    const long long nrows = (long long)B * seq * Hq;
    constexpr int LPR = D / (16 / sizeof(T));
    const long long rows_per_block = 256 / LPR;
    const long long dt_blocks = (long long)B * Hq * ((seq + rows_per_block - 1) / rows_per_block);
    RopeFreq f;
    fill_rope_freq(&f, D, rope ? rope->base : 2.0);
    const long long tab_blocks = rope ? ((long long)seq * (D / 2) + 255) / 256 : 0;
    const long long blocks = dt_blocks + tab_blocks;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const T*>(o), static_cast<const T*>(dout), dtbuf, nrows, seq, Hq,
                       dt_blocks, cs, rope ? rope->pos0 : 0, f);
    return hipGetLastError();
}

// Heads per dQ workgroup: the largest divisor G of g that is at most four, with two waves
// per head (four when G <= 2) for head_dim <= 64, i.e. 4, 6 or 8 waves; for head_dim 128
// one wave per head (G >= 3) or 4/G, in a 4-wave workgroup.
template <int D>
void pick_dq_shape(int g, int* G, int* WPH) {
    int G_ = 1;
    for (int c = 4; c >= 1; --c)
        if (g % c == 0) {
            G_ = c;
            break;
        }
    *G = G_;
    if (D >= 128)
        *WPH = (G_ >= 3) ? 1 : 4 / G_;
    else
        *WPH = (G_ <= 2) ? 4 : 2;
}

// Waves of a dK/dV workgroup (2 key halves x NW/2 query blocks of 32 rows).
template <typename T, int D>
constexpr int dkdv_waves() {
    return (D >= 128 || (sizeof(T) == 4 && D == 64)) ? 4 : 8;
}

// Longest-first dispatch table of one (batch, K/V head)'s items for the shared launch.  Cost
// of an item = its iterations x the MFMA work of one iteration (8 D FLOPs per pair for the
// dK/dV role: S, dP, dV, dK; 6 D for the dQ role: S, dP, dQ).  Both roles' lists are already
// in non-increasing cost order, so one merge sorts them; ties keep dK/dV items first.
template <typename K>
void fill_order(BwdArgs& a) {
    const int nqi = a.ntq_dq * a.nhc;
    if (a.ntk + nqi > kMaxOrder) return;
    const int g = a.Hq / a.Hkv;
    const int BN = K::Dk::BN, BMq = a.WPH * 32, BNq = K::BNQ;
    auto cost_dkdv = [&](int j) {
        const int stages = a.causal ? a.ntq - (j * BN) / K::BM : a.ntq;
        return (long long)g * stages * (BN * K::BM * 8);
    };
    auto cost_dq = [&](int i) {
        const int tile = a.ntq_dq - 1 - i / a.nhc;
        const int last = a.causal ? std::min(tile * BMq + BMq, a.T) - 1 : a.T - 1;
        return (long long)(last / BNq + 1) * (BMq * a.G * BNq * 6);
    };
    int j = 0, i = 0, n = 0;
    while (j < a.ntk || i < nqi) {
        if (i >= nqi || (j < a.ntk && cost_dkdv(j) >= cost_dq(i)))
            a.order[n++] = (unsigned short)j++;
        else
            a.order[n++] = (unsigned short)(0x8000 + i++);
    }
    a.norder = n;
}

template <typename T, int D, int NW>
hipError_t launch_bwd_cfg(const BwdArgs& a0, int G, int WPH, int roles, hipStream_t stream) {
    using K = BwdKernelCfg<T, D, NW>;
    BwdArgs a = a0;
    a.G = G;
    a.WPH = WPH;
    a.nhc = (a.Hq / a.Hkv) / G;
    a.ntk = (a.T + K::Dk::BN - 1) / K::Dk::BN;
    a.ntq = (a.T + K::BM - 1) / K::BM;
    a.ntq_dq = (a.T + WPH * 32 - 1) / (WPH * 32);
    a.roles = roles;
    a.norder = 0;
    if (roles == 3) fill_order<K>(a);
    long long items = 0;
    if (roles & 1) items += a.ntk;
    if (roles & 2) items += (long long)a.ntq_dq * a.nhc;
    const long long blocks = items * a.B * a.Hkv;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_kernel<T, D, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int D, int NW>
hipError_t launch_dq_cfg(const BwdArgs& a0, int G, int WPH, hipStream_t stream) {
    BwdArgs a = a0;
    a.G = G;
    a.WPH = WPH;
    a.nhc = (a.Hq / a.Hkv) / G;
    a.ntq_dq = (a.T + WPH * 32 - 1) / (WPH * 32);
    a.roles = 2;
    a.norder = 0;
    const long long blocks = (long long)a.ntq_dq * a.nhc * a.B * a.Hkv;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dkdv_only(const BwdArgs& a0, hipStream_t stream) {
    using S = DkdvSolo<T, D>;
    BwdArgs a = a0;
    a.ntk = (a.T + S::BN - 1) / S::BN;
    a.ntq = (a.T + 127) / 128;
    a.roles = 1;
    a.norder = 0;
    const long long blocks = (long long)a.ntk * a.B * a.Hkv;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D>), dim3((unsigned)blocks), dim3(S::NT), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dq_only(const BwdArgs& a, int G, int WPH, hipStream_t stream) {
    if constexpr (D >= 128) {
        return launch_dq_cfg<T, D, 4>(a, G, WPH, stream);
    } else {
        // Three heads: 12 waves (three per SIMD) instead of 6 (two SIMDs with one wave more
        // than the others), when the launch still has two workgroups per CU.
        if constexpr (sizeof(T) == 2)
            if (G == 3 && (long long)((a.T + 127) / 128) * (a.Hq / a.Hkv / 3) * a.B * a.Hkv >= 512)
                return launch_dq_cfg<T, D, 12>(a, G, 4, stream);
        const int nw = G * WPH;
        if (nw == 6) return launch_dq_cfg<T, D, 6>(a, G, WPH, stream);
        if (nw == 4) return launch_dq_cfg<T, D, 4>(a, G, WPH, stream);
        return launch_dq_cfg<T, D, 8>(a, G, WPH, stream);
    }
}

// Both roles share one launch when the dK/dV role alone has at most two workgroups per CU
// (then each role's causal tail overlaps the other's work) and the dQ role's workgroup fits
// the dK/dV role's wave count.
template <typename T, int D>
bool shared_launch(const BwdArgs& a) {
    int G, WPH;
    pick_dq_shape<D>(a.Hq / a.Hkv, &G, &WPH);
    const long long dkdv_blocks = (long long)((a.T + 63) / 64) * a.B * a.Hkv;
    return dkdv_blocks <= 512 && G * WPH <= dkdv_waves<T, D>();
}

// roles: 1 = dK/dV, 2 = dQ, 3 = both; both roles in one launch when shared_launch holds,
// otherwise two launches, each with its own workgroup shape.
template <typename T, int D>
hipError_t launch_bwd_t(const BwdArgs& a, int roles, hipStream_t stream) {
    constexpr int NWK = dkdv_waves<T, D>();
    int G, WPH;
    pick_dq_shape<D>(a.Hq / a.Hkv, &G, &WPH);
    const long long dkdv_blocks = (long long)((a.T + 63) / 64) * a.B * a.Hkv;
    const bool small = dkdv_blocks <= 512;
    if (roles == 3 && shared_launch<T, D>(a)) return launch_bwd_cfg<T, D, NWK>(a, G, WPH, 3, stream);
    if (roles & 1) {
        // The separate dK/dV kernel pays once the 64-key launch would have more than two
        // workgroups per CU; below that the role of the shared launch is used, so that the
        // dK/dV entry point and the shared launch give bitwise the same dK and dV.
        hipError_t e;
        if constexpr (sizeof(T) == 2) {
            if (!small)
                e = launch_dkdv_only<T, D>(a, stream);
            else
                e = launch_bwd_cfg<T, D, NWK>(a, G, WPH, 1, stream);
        } else {
            e = launch_bwd_cfg<T, D, NWK>(a, G, WPH, 1, stream);
        }
        if (e != hipSuccess) return e;
    }
    if (roles & 2) return launch_dq_only<T, D>(a, G, WPH, stream);
    return hipSuccess;
}

template <typename T>
hipError_t launch_bwd_roles(const BwdArgs& a, int D, int roles, hipStream_t stream) {
    if (D == 32) return launch_bwd_t<T, 32>(a, roles, stream);
    if (D == 64) return launch_bwd_t<T, 64>(a, roles, stream);
    return launch_bwd_t<T, 128>(a, roles, stream);
}

float* ws_dt(void* ws) { return static_cast<float*>(ws); }
size_t dt_bytes(int B, int T, int Hq) { return align256((size_t)B * Hq * T * sizeof(float)); }
float* ws_rope(void* ws, int B, int T, int Hq) {
    return reinterpret_cast<float*>(static_cast<char*>(ws) + dt_bytes(B, T, Hq));
}

BwdArgs make_args(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, void* workspace, int B, int T, int Hq, int Hkv,
                  float scale, bool rope = false, bool causal = true) {
    BwdArgs a{};
    a.causal = causal ? 1 : 0;
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.lse = lse;
    a.dt = ws_dt(workspace);
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.B = B;
    a.T = T;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.sl2 = scale * kLog2e;
    a.scale = scale;
    a.rope_cs = rope ? ws_rope(workspace, B, T, Hq) : nullptr;
    return a;
}

}  // namespace

size_t bwd_workspace_bytes(int B, int T, int Hq, int D, bool rope) {
    return dt_bytes(B, T, Hq) + (rope ? align256((size_t)T * (D / 2) * 2 * sizeof(float)) : 0);
}

hipError_t launch_bwd_pre(const void* o, const void* dout, void* workspace, int B, int T, int Hq,
                          int D, IoType dt, const RopeArgs* rope, hipStream_t stream) {
    float* dtb = ws_dt(workspace);
    float* cs = rope ? ws_rope(workspace, B, T, Hq) : nullptr;
    if (dt == kF32) {
        if (D == 32) return launch_pre_t<float, 32>(o, dout, dtb, B, T, Hq, cs, rope, stream);
        if (D == 64) return launch_pre_t<float, 64>(o, dout, dtb, B, T, Hq, cs, rope, stream);
        return launch_pre_t<float, 128>(o, dout, dtb, B, T, Hq, cs, rope, stream);
    }
    if (D == 32) return launch_pre_t<bf16, 32>(o, dout, dtb, B, T, Hq, cs, rope, stream);
    if (D == 64) return launch_pre_t<bf16, 64>(o, dout, dtb, B, T, Hq, cs, rope, stream);
    return launch_pre_t<bf16, 128>(o, dout, dtb, B, T, Hq, cs, rope, stream);
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                           const void* dout, void* dk, void* dv, void* workspace, int B, int T,
                           int Hq, int Hkv, int D, float scale, IoType dt, hipStream_t stream) {
    const BwdArgs a = make_args(q, k, v, lse, dout, nullptr, dk, dv, workspace, B, T, Hq, Hkv, scale);
    return dt == kF32 ? launch_bwd_roles<float>(a, D, 1, stream) : launch_bwd_roles<bf16>(a, D, 1, stream);
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                         const void* dout, void* dq, void* workspace, int B, int T, int Hq,
                         int Hkv, int D, float scale, IoType dt, hipStream_t stream) {
    const BwdArgs a = make_args(q, k, v, lse, dout, dq, nullptr, nullptr, workspace, B, T, Hq, Hkv, scale);
    return dt == kF32 ? launch_bwd_roles<float>(a, D, 2, stream) : launch_bwd_roles<bf16>(a, D, 2, stream);
}

hipError_t launch_bwd_main(const void* q, const void* k, const void* v, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, void* workspace, int B,
                           int T, int Hq, int Hkv, int D, float scale, IoType dt, bool rope,
                           bool causal, hipStream_t stream) {
    const BwdArgs a = make_args(q, k, v, lse, dout, dq, dk, dv, workspace, B, T, Hq, Hkv, scale, rope,
                                causal);
    return dt == kF32 ? launch_bwd_roles<float>(a, D, 3, stream) : launch_bwd_roles<bf16>(a, D, 3, stream);
}

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           void* workspace, int B, int T, int Hq, int Hkv, int D, float scale,
                           IoType dt, const RopeArgs* rope, bool causal, hipStream_t stream) {
    hipError_t e = launch_bwd_pre(o, dout, workspace, B, T, Hq, D, dt, rope, stream);
    if (e != hipSuccess) return e;
    return launch_bwd_main(q, k, v, lse, dout, dq, dk, dv, workspace, B, T, Hq, Hkv, D, scale, dt,
                           rope != nullptr, causal, stream);
}

}  // namespace ea
