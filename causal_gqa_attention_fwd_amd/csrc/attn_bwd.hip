// attn_bwd.hip -- causal GQA attention backward on gfx950 (attn_bwd).
//
// The pages only say that NanoEuler's backward is hand-written and gradient-checked
// ("Show HN: NanoEuler", sections 3 and 4); the algorithm here is the standard
// recompute-from-LSE backward of tiled attention.  With P_ts = exp(S_ts - LSE_t),
// dP = dO V^T, D_t = sum_d dO_t * O_t (= sum_s P_ts dP_ts), dS = P (dP - D_t):
//   dV_s = sum_{h in group} sum_{t>=s} P_ts dO_t
//   dK_s = scale * sum_{h in group} sum_{t>=s} dS_ts Q_t
//   dQ_t = scale * sum_{s<=t} dS_ts K_s
// Three launches:
//   1. bwd_pre:  D_t for every (b, h, t) and a zeroed fp32 dQ accumulator.
//   2. bwd_main: one workgroup per (64-key tile j, K/V head, batch).  K_j and V_j stay in
//      registers; the workgroup walks every head of the group and every query tile on or
//      below the diagonal, so dK_j and dV_j are group-summed in registers and written once
//      (deterministic).  dQ contributions are added to the fp32 accumulator with hardware
//      float atomics.
//   3. dq_convert: dQ = scale * accumulator, in the I/O dtype.
//
// gfx950 layout of bwd_main (4 waves; wave w owns keys 32*(w&1).. and queries 32*(w>>1)..
// of the current 64 x 64 (query x key) tile):
//   S = Q K^T and dP = dO V^T are 32x32 MFMA tiles whose lanes hold one key column and 16
//   query rows, which is exactly the A-operand shape of dV += P^T dO and dK += dS^T Q, so P
//   and dS go from accumulator to operand without leaving registers.  Q and dO are staged
//   in LDS twice (row-major for S/dP, transposed in "slot" order for dV/dK); dS goes
//   through LDS once so that dQ = dS K can take it in query-row form.
#include <cmath>

#include "ea_common.h"
#include "ea_kernels.h"

namespace ea {
namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------------------
// 1. D_t = sum_d dO * O per row, and zero the dQ accumulator.
// ---------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ o,
                                                      const T* __restrict__ dout,
                                                      float* __restrict__ dt,
                                                      float* __restrict__ dqacc, long long nrows,
                                                      long long nacc4, int T_, int Hq) {
    constexpr int EPC = 16 / sizeof(T);
    constexpr int LPR = D / EPC;  // lanes per row (4 .. 32)
    const int tid = threadIdx.x;
    const long long row = (long long)blockIdx.x * (256 / LPR) + tid / LPR;
    const int c = tid % LPR;
    float acc = 0.0f;
    if (row < nrows) {
        const Vec16<T> a = ld16(o + row * D + c * EPC);
        const Vec16<T> d = ld16(dout + row * D + c * EPC);
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc += to_f32(a.get(e)) * to_f32(d.get(e));
    }
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (row < nrows && c == 0) {
        const long long h = row % Hq;
        const long long bt = row / Hq;
        const long long t = bt % T_;
        const long long b = bt / T_;
        dt[(b * Hq + h) * T_ + t] = acc;
    }
    const long long gid = (long long)blockIdx.x * 256 + tid;
    const long long nth = (long long)gridDim.x * 256;
    f32x4* acc4 = reinterpret_cast<f32x4*>(dqacc);
    for (long long i = gid; i < nacc4; i += nth) acc4[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ---------------------------------------------------------------------------------------
// 3. dQ = scale * accumulator.
// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc,
                                                         T* __restrict__ dq, long long n8,
                                                         float scale) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const f32x4 a0 = reinterpret_cast<const f32x4*>(acc)[2 * i];
    const f32x4 a1 = reinterpret_cast<const f32x4*>(acc)[2 * i + 1];
    if constexpr (sizeof(T) == 2) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = (bf16)(a0[e] * scale);
            v[4 + e] = (bf16)(a1[e] * scale);
        }
        reinterpret_cast<bf16x8*>(dq)[i] = v;
    } else {
        reinterpret_cast<f32x4*>(dq)[2 * i] = a0 * scale;
        reinterpret_cast<f32x4*>(dq)[2 * i + 1] = a1 * scale;
    }
}

// ---------------------------------------------------------------------------------------
// 2. Main backward kernel.
// ---------------------------------------------------------------------------------------
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* lse;
    const float* dt;
    float* dqacc;
    void* dk;
    void* dv;
    int B, T, Hq, Hkv;
    int ntk;  // key tiles
    int ntq;  // query tiles
    float sl2;    // scale * log2(e)
    float scale;
};

template <typename T, int D, int BM>
struct BwdCfg {
    static constexpr int KPL = Mfma<T>::KPL;
    static constexpr int BN = 64;               // keys per workgroup
    static constexpr int NKH = BN / 32;         // key halves
    static constexpr int NQH = BM / 32;         // query blocks per iteration
    static constexpr int NW = NKH * NQH;
    static constexpr int NT = 64 * NW;
    static constexpr int NS = D / (2 * KPL);    // MFMA steps over head_dim
    static constexpr int NDB = D / 32;
    static constexpr int PS = 16 / KPL;         // MFMA steps over a 32-row accumulator
    static constexpr int NSK = BN / (2 * KPL);  // MFMA steps over the tile's keys (dQ)
    static constexpr int EPC = 16 / sizeof(T);
    static constexpr int CPR = D / EPC;
    static constexpr int QS = D + EPC;          // row-major Q / dO stride
    static constexpr int QTS = BM + EPC;        // transposed Q / dO stride
    static constexpr int KTS = BN + EPC;        // transposed K stride
    static constexpr int DSS = BN + EPC;        // dS stride
    static constexpr int NCHQ = (BM * CPR + NT - 1) / NT;
    static constexpr int NCHK = (BN * CPR + NT - 1) / NT;
    // LDS carve-up (bytes).
    static constexpr size_t OFF_Q = 0;
    static constexpr size_t OFF_DO = OFF_Q + sizeof(T) * BM * QS;
    static constexpr size_t OFF_QT = OFF_DO + sizeof(T) * BM * QS;
    static constexpr size_t OFF_DOT = OFF_QT + sizeof(T) * D * QTS;
    static constexpr size_t OFF_KT = OFF_DOT + sizeof(T) * D * QTS;
    static constexpr size_t OFF_DS = OFF_KT + sizeof(T) * D * KTS;
    static constexpr size_t OFF_LSE = OFF_DS + sizeof(T) * BM * DSS;
    static constexpr size_t OFF_DT = OFF_LSE + sizeof(float) * BM;
    static constexpr size_t BYTES = OFF_DT + sizeof(float) * BM;
    // dK/dV partials of the waves with query block > 0, reduced at the end (reuses the
    // Q / dO / Q^T / dO^T region).
    static constexpr size_t RED_BYTES = (size_t)(NQH - 1) * NKH * 2 * NDB * 16 * 64 * sizeof(float);
    static_assert(RED_BYTES <= OFF_KT, "reduction buffer must fit in the staging region");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <typename T, int D, int BM>
__global__ __launch_bounds__((64 * BwdCfg<T, D, BM>::NW)) void attn_bwd_kernel(BwdArgs a) {
    using C = BwdCfg<T, D, BM>;
    using M = Mfma<T>;
    using frag = typename M::frag;
    constexpr int KPL = C::KPL;
    constexpr int BN = C::BN;

    __shared__ __attribute__((aligned(16))) char smem[C::BYTES];
    T* Qs = reinterpret_cast<T*>(smem + C::OFF_Q);
    T* dOs = reinterpret_cast<T*>(smem + C::OFF_DO);
    T* QTs = reinterpret_cast<T*>(smem + C::OFF_QT);
    T* dOTs = reinterpret_cast<T*>(smem + C::OFF_DOT);
    T* KTs = reinterpret_cast<T*>(smem + C::OFF_KT);
    T* dSs = reinterpret_cast<T*>(smem + C::OFF_DS);
    float* lse2s = reinterpret_cast<float*>(smem + C::OFF_LSE);
    float* dts = reinterpret_cast<float*>(smem + C::OFF_DT);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int kh = w % C::NKH;
    const int qh = w / C::NKH;

    const int HB = a.B * a.Hkv;
    const int j = blockIdx.x / HB;
    const int rem = blockIdx.x % HB;
    const int kvh = rem % a.Hkv;
    const int b = rem / a.Hkv;
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
    // K_j^T in LDS (identity key order) for dQ = dS K.
#pragma unroll
    for (int n = 0; n < C::NCHK; ++n) {
        const int c = tid + n * C::NT;
        if (c < BN * C::CPR) {
            const int key = c / C::CPR;
            const int part = c % C::CPR;
            const int s = j * BN + key;
            const Vec16<T> kv = (s < a.T)
                ? ld16(kp + (((long long)b * a.T + s) * a.Hkv + kvh) * D + part * C::EPC)
                : zero16<T>();
#pragma unroll
            for (int e = 0; e < C::EPC; ++e) KTs[(part * C::EPC + e) * C::KTS + key] = kv.get(e);
        }
    }

    f32x16 dkacc[C::NDB], dvacc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
        dkacc[db] = zero_acc();
        dvacc[db] = zero_acc();
    }

    const int i0 = (j * BN) / BM;
    for (int hs = 0; hs < g; ++hs) {
        const int head = kvh * g + hs;
        const float* lse_row = a.lse + ((long long)b * a.Hq + head) * a.T;
        const float* dt_row = a.dt + ((long long)b * a.Hq + head) * a.T;
        for (int i = i0; i < a.ntq; ++i) {
            __syncthreads();  // previous iteration is done with the staging buffers
            // Stage Q_i and dO_i: row-major and transposed ("slot" order per 32 rows).
#pragma unroll
            for (int n = 0; n < C::NCHQ; ++n) {
                const int c = tid + n * C::NT;
                if (c < BM * C::CPR) {
                    const int qr = c / C::CPR;
                    const int part = c % C::CPR;
                    const int t = i * BM + qr;
                    Vec16<T> qv = zero16<T>(), dv = zero16<T>();
                    if (t < a.T) {
                        const long long off = (((long long)b * a.T + t) * a.Hq + head) * D + part * C::EPC;
                        qv = ld16(qp + off);
                        dv = ld16(dop + off);
                    }
                    st16(&Qs[qr * C::QS + part * C::EPC], qv);
                    st16(&dOs[qr * C::QS + part * C::EPC], dv);
                    const int slot = (qr & ~31) + acc_slot(qr & 31);
#pragma unroll
                    for (int e = 0; e < C::EPC; ++e) {
                        QTs[(part * C::EPC + e) * C::QTS + slot] = qv.get(e);
                        dOTs[(part * C::EPC + e) * C::QTS + slot] = dv.get(e);
                    }
                }
            }
            for (int qr = tid; qr < BM; qr += C::NT) {
                const int t = i * BM + qr;
                lse2s[qr] = (t < a.T) ? lse_row[t] * kLog2e : INFINITY;
                dts[qr] = (t < a.T) ? dt_row[t] : 0.0f;
            }
            __syncthreads();

            // S = Q K^T and dP = dO V^T on this wave's 32 x 32 block.
            f32x16 sacc = zero_acc(), dpacc = zero_acc();
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                const int ro = (qh * 32 + l32) * C::QS + half * (D / 2) + s * KPL;
                sacc = M::mma(load_frag<T>(&Qs[ro]), kf[s], sacc);
                dpacc = M::mma(load_frag<T>(&dOs[ro]), vf[s], dpacc);
            }
            // P = exp(S - LSE), masked on blocks crossing the diagonal; dS = P (dP - D).
            const bool diag = (j * BN + kh * 32 + 31) > (i * BM + qh * 32);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lq = qh * 32 + acc_row(r, half);
                float p = __builtin_amdgcn_exp2f(sacc[r] * a.sl2 - lse2s[lq]);
                if (diag && mykey > i * BM + lq) p = 0.0f;
                sacc[r] = p;
                dpacc[r] = p * (dpacc[r] - dts[lq]);
            }
            // dV += P^T dO and dK += dS^T Q (contraction over this wave's 32 queries).
#pragma unroll
            for (int ps = 0; ps < C::PS; ++ps) {
                const frag pf = acc_to_frag<T>(sacc, ps * KPL);
                const frag dsf = acc_to_frag<T>(dpacc, ps * KPL);
#pragma unroll
                for (int db = 0; db < C::NDB; ++db) {
                    const int ro = (db * 32 + l32) * C::QTS + qh * 32 + 16 * half + ps * KPL;
                    dvacc[db] = M::mma(pf, load_frag<T>(&dOTs[ro]), dvacc[db]);
                    dkacc[db] = M::mma(dsf, load_frag<T>(&QTs[ro]), dkacc[db]);
                }
            }
            // dS to LDS in query-row form.
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dSs[(qh * 32 + acc_row(r, half)) * C::DSS + kh * 32 + l32] = from_f32<T>(dpacc[r]);
            __syncthreads();
            // dQ_i += dS K_j ("split" over the tile's keys), one 32x32 block per wave turn.
            for (int blk = w; blk < C::NQH * C::NDB; blk += C::NW) {
                const int qb = blk / C::NDB;
                const int db = blk % C::NDB;
                f32x16 acc = zero_acc();
#pragma unroll
                for (int s = 0; s < C::NSK; ++s) {
                    const frag af = load_frag<T>(&dSs[(qb * 32 + l32) * C::DSS + half * (BN / 2) + s * KPL]);
                    const frag bk = load_frag<T>(&KTs[(db * 32 + l32) * C::KTS + half * (BN / 2) + s * KPL]);
                    acc = M::mma(af, bk, acc);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int t = i * BM + qb * 32 + acc_row(r, half);
                    if (t < a.T)
                        unsafeAtomicAdd(&a.dqacc[(((long long)b * a.T + t) * a.Hq + head) * D + db * 32 + l32], acc[r]);
                }
            }
        }
    }

    // Reduce the dK/dV partials of the query blocks and store (dK scaled by `scale`).
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
    if (qh > 0) {
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const size_t base = ((((size_t)(qh - 1) * C::NKH + kh) * 2) * C::NDB + db) * 16 * 64;
                red[base + r * 64 + lane] = dkacc[db][r];
                red[base + (size_t)C::NDB * 16 * 64 + r * 64 + lane] = dvacc[db][r];
            }
    }
    __syncthreads();
    if (qh > 0) return;
    for (int o = 1; o < C::NQH; ++o) {
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const size_t base = ((((size_t)(o - 1) * C::NKH + kh) * 2) * C::NDB + db) * 16 * 64;
                dkacc[db][r] += red[base + r * 64 + lane];
                dvacc[db][r] += red[base + (size_t)C::NDB * 16 * 64 + r * 64 + lane];
            }
    }
    T* __restrict__ dkp = static_cast<T*>(a.dk);
    T* __restrict__ dvp = static_cast<T*>(a.dv);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int key = j * BN + kh * 32 + acc_row(r, half);
        if (key < a.T) {
            const long long off = (((long long)b * a.T + key) * a.Hkv + kvh) * D + l32;
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
                dkp[off + db * 32] = from_f32<T>(dkacc[db][r] * a.scale);
                dvp[off + db * 32] = from_f32<T>(dvacc[db][r]);
            }
        }
    }
}

template <typename T, int D>
hipError_t launch_pre_t(const void* o, const void* dout, float* dqacc, float* dtbuf, int B, int seq,
                        int Hq, hipStream_t stream) {
    const long long nrows = (long long)B * seq * Hq;
    const long long nacc = nrows * D;
    constexpr int LPR = D / (16 / sizeof(T));
    const long long rows_per_block = 256 / LPR;
    const long long blocks = (nrows + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const T*>(o), static_cast<const T*>(dout), dtbuf, dqacc, nrows,
                       nacc / 4, seq, Hq);
    return hipGetLastError();
}

template <typename T, int D, int BM>
hipError_t launch_main_t(const BwdArgs& a0, hipStream_t stream) {
    BwdArgs a = a0;
    using C = BwdCfg<T, D, BM>;
    a.ntk = (a.T + C::BN - 1) / C::BN;
    a.ntq = (a.T + BM - 1) / BM;
    const long long blocks = (long long)a.ntk * a.B * a.Hkv;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_bwd_kernel<T, D, BM>), dim3((unsigned)blocks), dim3(C::NT), 0, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_convert_t(const float* dqacc, void* dq, long long nacc, float scale,
                            hipStream_t stream) {
    const long long n8 = nacc / 8;
    const long long blocks = (n8 + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((dq_convert_kernel<T>), dim3((unsigned)blocks), dim3(256), 0, stream, dqacc,
                       static_cast<T*>(dq), n8, scale);
    return hipGetLastError();
}

float* ws_dqacc(void* ws) { return static_cast<float*>(ws); }

float* ws_dt(void* ws, int B, int T, int Hq, int D) {
    return reinterpret_cast<float*>(static_cast<char*>(ws) + align256((size_t)B * T * Hq * D * sizeof(float)));
}

}  // namespace

size_t bwd_workspace_bytes(int B, int T, int Hq, int D) {
    return align256((size_t)B * T * Hq * D * sizeof(float)) + align256((size_t)B * Hq * T * sizeof(float));
}

hipError_t launch_bwd_pre(const void* o, const void* dout, void* workspace, int B, int T, int Hq,
                          int D, IoType dt, hipStream_t stream) {
    float* acc = ws_dqacc(workspace);
    float* dtb = ws_dt(workspace, B, T, Hq, D);
    if (dt == kF32) {
        if (D == 32) return launch_pre_t<float, 32>(o, dout, acc, dtb, B, T, Hq, stream);
        if (D == 64) return launch_pre_t<float, 64>(o, dout, acc, dtb, B, T, Hq, stream);
        return launch_pre_t<float, 128>(o, dout, acc, dtb, B, T, Hq, stream);
    }
    if (D == 32) return launch_pre_t<bf16, 32>(o, dout, acc, dtb, B, T, Hq, stream);
    if (D == 64) return launch_pre_t<bf16, 64>(o, dout, acc, dtb, B, T, Hq, stream);
    return launch_pre_t<bf16, 128>(o, dout, acc, dtb, B, T, Hq, stream);
}

hipError_t launch_bwd_main(const void* q, const void* k, const void* v, const float* lse,
                           const void* dout, void* dk, void* dv, void* workspace, int B, int T,
                           int Hq, int Hkv, int D, float scale, IoType dt, hipStream_t stream) {
    BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.lse = lse;
    a.dt = ws_dt(workspace, B, T, Hq, D);
    a.dqacc = ws_dqacc(workspace);
    a.dk = dk;
    a.dv = dv;
    a.B = B;
    a.T = T;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.sl2 = scale * kLog2e;
    a.scale = scale;
    if (dt == kF32) {
        if (D == 32) return launch_main_t<float, 32, 64>(a, stream);
        if (D == 64) return launch_main_t<float, 64, 64>(a, stream);
        return launch_main_t<float, 128, 32>(a, stream);
    }
    if (D == 32) return launch_main_t<bf16, 32, 64>(a, stream);
    if (D == 64) return launch_main_t<bf16, 64, 64>(a, stream);
    return launch_main_t<bf16, 128, 64>(a, stream);
}

hipError_t launch_bwd_dq_finalize(const void* workspace, void* dq, int B, int T, int Hq, int D,
                                  float scale, IoType dt, hipStream_t stream) {
    const float* acc = static_cast<const float*>(workspace);
    const long long nacc = (long long)B * T * Hq * D;
    if (dt == kF32) return launch_convert_t<float>(acc, dq, nacc, scale, stream);
    return launch_convert_t<bf16>(acc, dq, nacc, scale, stream);
}

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           void* workspace, int B, int T, int Hq, int Hkv, int D, float scale,
                           IoType dt, hipStream_t stream) {
    hipError_t e = launch_bwd_pre(o, dout, workspace, B, T, Hq, D, dt, stream);
    if (e != hipSuccess) return e;
    e = launch_bwd_main(q, k, v, lse, dout, dk, dv, workspace, B, T, Hq, Hkv, D, scale, dt, stream);
    if (e != hipSuccess) return e;
    return launch_bwd_dq_finalize(workspace, dq, B, T, Hq, D, scale, dt, stream);
}

}  // namespace ea
