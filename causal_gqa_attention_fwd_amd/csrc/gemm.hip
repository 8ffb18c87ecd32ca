// gemm.hip -- C = op(A) op(B) on the matrix cores (gfx950), for the projections on either
// side of the attention: the QKV projection (with RoPE on Q and K applied in the epilogue)
// and the output projection, forward and backward.
//
// The pages do these steps with a matrix library ("Show HN: NanoEuler", section 4; "Tiny
// Hackable CUDA Language Model Implementation", sections 1 and 3: the attention result is
// projected back to the model dimension, matrix products go to BLAS).  Here they are the
// library's own kernels, tiled for 64-wide wavefronts and LDS.
//
// Layout: every matrix is row-major with a leading dimension.  op(A) is [M, K]: A stored as
// [M, K] (trans_a = 0) or [K, M] (trans_a = 1); op(B) is [K, N]: B stored as [K, N]
// (trans_b = 0) or [N, K] (trans_b = 1).  C is [M, N], fp32 accumulation, one rounding to
// the I/O dtype.  A may be split along K, and B and C along N, into up to three segments,
// each with its own base pointer and leading dimension: the QKV projection writes Q, K and
// V as three separate [B, T, H, D] tensors from one product, and its backward reads the
// three gradients as one operand.
//
// Work split: a workgroup computes a BM x BN tile of C with WM x WN waves; each wave owns
// (BM/WM) x (BN/WN) as 32 x 32 matrix-core blocks.  The MFMA computes C^T = op(B)^T op(A)^T,
// so a lane holds one row m of C and 16 of its columns in groups of four consecutive
// columns: stores are 8 (bf16) or 16 (fp32) bytes, and the two columns of a RoPE pair sit
// in one lane.  The contraction index of a 32-deep block follows the accumulator order
// (ea_common.h): an operand whose rows are K-contiguous is read with two 8-byte LDS reads
// per fragment, an operand whose rows run along K is read with the transposing LDS read.
// Tiles go HBM -> registers -> LDS through two register sets (bf16) and a double-buffered
// LDS, one barrier per K tile.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>

#include "ea_common.h"
#include "ea_kernels.h"

namespace ea {
namespace {

constexpr int kXcds = 8;  // workgroups are dealt to the XCDs round-robin

struct Seg {
    const void* p;
    long long ld;  // leading dimension in elements
    int start;     // first index (along K for A, along N for B and C) of this segment
};

struct GemmArgs {
    Seg a[kGemmMaxSeg];  // A segments along K (trans_a = 0); unused segments start at INT_MAX
    Seg b[kGemmMaxSeg];  // B segments along N (trans_b = 0)
    Seg c[kGemmMaxSeg];  // C segments along N
    int M, N, K;
    int tiles_m, tiles_n;  // ceil(M / BM), ceil(N / BN)
    int rope_mask;       // bit s: rotate the column pairs of C segment s (heads of rope_D)
    int rope_T, rope_D, rope_pos0;
    int ksplit;          // split-K: slices of the K range (1: none)
    float* part;         // split-K: fp32 partial tiles, [tile][slice][BM * BN] in register order
    RopeFreq f;
};

// Segments as plain values (no array indexed at run time, which would live in scratch).
template <typename T>
struct SegV {
    const T* p0;
    const T* p1;
    const T* p2;
    long long ld0, ld1, ld2;
    int st1, st2;
    __device__ inline explicit SegV(const Seg* s)
        : p0(static_cast<const T*>(s[0].p)), p1(static_cast<const T*>(s[1].p)),
          p2(static_cast<const T*>(s[2].p)), ld0(s[0].ld), ld1(s[1].ld), ld2(s[2].ld),
          st1(s[1].start), st2(s[2].start) {}
    // Address of element (r, x) where x runs along the split dimension and r across it (every
    // segment's address is formed and one is selected; the load that uses it is unconditional).
    __device__ inline const T* at(long long r, int x) const {
        const T* a0 = p0 + r * ld0 + x;
        const T* a1 = p1 + r * ld1 + (x - st1);
        const T* a2 = p2 + r * ld2 + (x - st2);
        return x >= st2 ? a2 : (x >= st1 ? a1 : a0);
    }
    __device__ inline int index(int x) const { return (x >= st1 ? 1 : 0) + (x >= st2 ? 1 : 0); }
};

// Fragment of KPL contraction elements from a row whose elements run along K (p points at
// the start of a 32-deep block): element e <-> k = acc_row(ps * KPL + e, half).
template <typename T>
__device__ inline typename Mfma<T>::frag load_k_frag(const T* p, int ps);

template <>
__device__ inline bf16x8 load_k_frag<bf16>(const bf16* p, int ps) {
    const int h = __lane_id() >> 5;
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p + 16 * ps + 4 * h);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16 * ps + 8 + 4 * h);
    bf16x8 f;
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
    return f;
}

template <>
__device__ inline float load_k_frag<float>(const float* p, int ps) {
    return p[acc_row(ps, __lane_id() >> 5)];
}

template <typename T, int TA, int TB, int BM, int BN, int WM, int WN>
struct GemmCfg {
    static constexpr int KPL = Mfma<T>::KPL;
    static constexpr int EPC = 16 / sizeof(T);
    static constexpr int BK = sizeof(T) == 2 ? 64 : 32;
    static constexpr int NW = WM * WN;
    static constexpr int NT = 64 * NW;
    static constexpr int MB = BM / WM / 32;  // 32-row blocks per wave
    static constexpr int NB = BN / WN / 32;  // 32-column blocks per wave
    static constexpr int PS = 16 / KPL;      // MFMA steps per 32-deep block
    static constexpr int KB = BK / 32;
    // A tile: [BM][BK] (trans_a = 0, row = m) or [BK][BM] (trans_a = 1, row = k); likewise B:
    // [BK][BN] (trans_b = 0, row = k) or [BN][BK] (trans_b = 1, row = n).  16 bytes of padding
    // per row.
    static constexpr int A_ROWS = TA ? BK : BM, A_COLS = TA ? BM : BK;
    static constexpr int B_ROWS = TB ? BN : BK, B_COLS = TB ? BK : BN;
    static constexpr int A_STRIDE = A_COLS + EPC, B_STRIDE = B_COLS + EPC;
    static constexpr int A_SIZE = A_ROWS * A_STRIDE, B_SIZE = B_ROWS * B_STRIDE;
    static constexpr int A_CPR = A_COLS / EPC, B_CPR = B_COLS / EPC;  // chunks per tile row
    static constexpr int NCA = (A_ROWS * A_CPR + NT - 1) / NT;       // chunks per thread
    static constexpr int NCB = (B_ROWS * B_CPR + NT - 1) / NT;
    static constexpr size_t LDS_BYTES = 2 * (size_t)(A_SIZE + B_SIZE) * sizeof(T);
    static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tiling");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// MODE 0: C = op(A) op(B).  Split-K (a few output tiles, a long K): MODE 1 computes slice s of
// the K range of a tile and stores its fp32 partial; MODE 2 then sums a tile's partials in slice
// order (deterministic) and runs the epilogue.
template <typename T, int TA, int TB, int BM, int BN, int WM, int WN, int MODE = 0>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmArgs g) {
    using C = GemmCfg<T, TA, TB, BM, BN, WM, WN>;
    using M_ = Mfma<T>;
    using frag = typename M_::frag;
    constexpr int EPC = C::EPC;

    __shared__ __attribute__((aligned(16))) T As[2 * C::A_SIZE];
    __shared__ __attribute__((aligned(16))) T Bs[2 * C::B_SIZE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int wm = w / WN, wn = w % WN;
    // XCD-aware tile order: workgroup L runs on XCD L % 8, and XCD x takes a contiguous run of
    // tiles (row-major over the tile grid), so the A rows and B columns its workgroups share
    // are fetched into its own L2 rather than into all eight.
    // With split-K (MODE 1) the units are (tile, slice), the slices of a tile adjacent.
    const int ntiles = g.tiles_m * g.tiles_n;
    const int nunits = MODE == 1 ? ntiles * g.ksplit : ntiles;
    const int xcd = blockIdx.x % kXcds, jx = blockIdx.x / kXcds;
    const int q8 = nunits / kXcds, r8 = nunits % kXcds;
    const int unit = xcd < r8 ? xcd * (q8 + 1) + jx : r8 * (q8 + 1) + (xcd - r8) * q8 + jx;
    const int tile = MODE == 1 ? unit / g.ksplit : unit;
    const int slice = MODE == 1 ? unit % g.ksplit : 0;
    const int tm = tile / g.tiles_n, tn = tile % g.tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = g.M, N = g.N, K = g.K;
    const int nk_all = (K + C::BK - 1) / C::BK;
    // K tiles [kt0, kt0 + nk) of this workgroup.
    const int kt0 = MODE == 1 ? (int)((long long)slice * nk_all / g.ksplit) : 0;
    const int nk = MODE == 1 ? (int)((long long)(slice + 1) * nk_all / g.ksplit) - kt0 : (MODE == 2 ? 0 : nk_all);
    const SegV<T> sa_(g.a), sb_(g.b);

    // Staging of one K tile (HBM -> registers), then registers -> LDS.  Every load is
    // unconditional, from a clamped address, so that the loads of later tiles stay in flight
    // while earlier ones are committed.  Rows past M or N load a real row: they only feed
    // outputs that are never stored.  Chunks past K load a real chunk too and are replaced
    // by zeros at commit (bit n of ok clear), as they would otherwise enter valid outputs.
    // Register sets of staged K tiles in flight: two for bf16 (a third set for the 64 x 64 tiles
    // measured slower), one for fp32.
    constexpr int NSET = sizeof(T) != 2 ? 1 : 2;
    static_assert(C::NCA + C::NCB <= 32, "chunk mask");
    struct Stg {
        Vec16<T> a[C::NCA], b[C::NCB];
        uint32_t ok;
    };
    Stg sets[NSET];
    // Per-chunk source addresses that do not change along K, computed once (the K loop only
    // adds its offset): A row / column bases (unless A is split along K, which takes the
    // general path below), B bases with their segment's leading dimension.
    const bool a_split_k = TA == 0 && sa_.st1 != INT_MAX;
    const T* abase[C::NCA];
    int aoff[C::NCA];
    const T* bbase[C::NCB];
    long long bld[C::NCB];
    int boff[C::NCB];
#pragma unroll
    for (int n = 0; n < C::NCA; ++n) {
        const int u = tid + n * C::NT;
        const int row = u / C::A_CPR, cc = u % C::A_CPR;
        if constexpr (TA == 0) {
            abase[n] = sa_.p0 + (long long)min(m0 + row, M - 1) * sa_.ld0;
            aoff[n] = cc * EPC;
        } else {
            abase[n] = sa_.p0 + min(m0 + cc * EPC, M - EPC);
            aoff[n] = row;
        }
    }
#pragma unroll
    for (int n = 0; n < C::NCB; ++n) {
        const int u = tid + n * C::NT;
        const int row = u / C::B_CPR, cc = u % C::B_CPR;
        if constexpr (TB == 0) {
            const int nn = min(n0 + cc * EPC, N - EPC);
            bbase[n] = sb_.at(0, nn);
            bld[n] = nn >= sb_.st2 ? sb_.ld2 : (nn >= sb_.st1 ? sb_.ld1 : sb_.ld0);
            boff[n] = row;
        } else {
            bbase[n] = sb_.p0 + (long long)min(n0 + row, N - 1) * sb_.ld0;
            bld[n] = 1;
            boff[n] = cc * EPC;
        }
    }
    auto fetch_fast = [&](Stg& st, int kt) {
        const int k0 = kt * C::BK;
        uint32_t ok = 0;
#pragma unroll
        for (int n = 0; n < C::NCA; ++n) {
            const int k = k0 + aoff[n];
            ok |= (k < K ? 1u : 0u) << n;
            if constexpr (TA == 0)
                st.a[n] = ld16(abase[n] + min(k, K - EPC));
            else
                st.a[n] = ld16(abase[n] + (long long)min(k, K - 1) * sa_.ld0);
        }
#pragma unroll
        for (int n = 0; n < C::NCB; ++n) {
            const int k = k0 + boff[n];
            ok |= (k < K ? 1u : 0u) << (C::NCA + n);
            if constexpr (TB == 0)
                st.b[n] = ld16(bbase[n] + (long long)min(k, K - 1) * bld[n]);
            else
                st.b[n] = ld16(bbase[n] + min(k, K - EPC));
        }
        st.ok = ok;
    };
    auto fetch_general = [&](Stg& st, int kt) {
        const int k0 = kt * C::BK;
        uint32_t ok = 0;
#pragma unroll
        for (int n = 0; n < C::NCA; ++n) {
            const int u = tid + n * C::NT;
            if ((C::A_ROWS * C::A_CPR) % C::NT == 0 || u < C::A_ROWS * C::A_CPR) {
                const int row = u / C::A_CPR, cc = u % C::A_CPR;
                int m, k;
                if constexpr (TA == 0) {
                    m = min(m0 + row, M - 1);
                    k = k0 + cc * EPC;
                } else {
                    k = k0 + row;
                    m = min(m0 + cc * EPC, M - EPC);
                }
                ok |= (k < K ? 1u : 0u) << n;
                if constexpr (TA == 0) {
                    st.a[n] = ld16(sa_.at(m, min(k, K - EPC)));
                } else {
                    st.a[n] = ld16(sa_.p0 + (long long)min(k, K - 1) * sa_.ld0 + m);
                }
            }
        }
#pragma unroll
        for (int n = 0; n < C::NCB; ++n) {
            const int u = tid + n * C::NT;
            if ((C::B_ROWS * C::B_CPR) % C::NT == 0 || u < C::B_ROWS * C::B_CPR) {
                const int row = u / C::B_CPR, cc = u % C::B_CPR;
                int nn, k;
                if constexpr (TB == 0) {
                    k = k0 + row;
                    nn = min(n0 + cc * EPC, N - EPC);
                } else {
                    nn = min(n0 + row, N - 1);
                    k = k0 + cc * EPC;
                }
                ok |= (k < K ? 1u : 0u) << (C::NCA + n);
                if constexpr (TB == 0) {
                    st.b[n] = ld16(sb_.at(min(k, K - 1), nn));
                } else {
                    st.b[n] = ld16(sb_.p0 + (long long)nn * sb_.ld0 + min(k, K - EPC));
                }
            }
        }
        st.ok = ok;
    };
    // Whole K tiles (all but a ragged last one) load through running per-chunk pointers that
    // advance by one K tile per fetch (the fetches come in K order), which costs one 64-bit add
    // per chunk instead of re-forming the address (a 64-bit product for the K-major operands)
    // and the tail mask.
    static_assert((C::A_ROWS * C::A_CPR) % C::NT == 0 && (C::B_ROWS * C::B_CPR) % C::NT == 0,
                  "every staged chunk lies inside the tile (no unclamped spare chunks)");
    const T* ap[C::NCA];
    const T* bp[C::NCB];
    long long bst[C::NCB];
    const long long ast = TA == 0 ? (long long)C::BK : (long long)C::BK * sa_.ld0;
#pragma unroll
    for (int n = 0; n < C::NCA; ++n) {
        if constexpr (TA == 0)
            ap[n] = abase[n] + aoff[n] + (long long)kt0 * C::BK;
        else
            ap[n] = abase[n] + (long long)(kt0 * C::BK + aoff[n]) * sa_.ld0;
    }
#pragma unroll
    for (int n = 0; n < C::NCB; ++n) {
        if constexpr (TB == 0) {
            bp[n] = bbase[n] + (long long)(kt0 * C::BK + boff[n]) * bld[n];
            bst[n] = (long long)C::BK * bld[n];
        } else {
            bp[n] = bbase[n] + boff[n] + (long long)kt0 * C::BK;
            bst[n] = C::BK;
        }
    }
    auto fetch_run = [&](Stg& st) {
#pragma unroll
        for (int n = 0; n < C::NCA; ++n) {
            st.a[n] = ld16(ap[n]);
            ap[n] += ast;
        }
#pragma unroll
        for (int n = 0; n < C::NCB; ++n) {
            st.b[n] = ld16(bp[n]);
            bp[n] += bst[n];
        }
    };
    auto fetch = [&](Stg& st, int kt) {
        if (a_split_k)
            fetch_general(st, kt0 + kt);
        else if (K % C::BK != 0 && kt0 + kt == nk_all - 1)
            fetch_fast(st, kt0 + kt);  // the ragged last tile: clamped addresses and the zero mask
        else
            fetch_run(st);
    };
    // tail: this is the last K tile and K is not a multiple of BK (chunks past K -> zeros).
    auto commit = [&](Stg& st, int buf, bool tail) {
        if (tail) {
#pragma unroll
            for (int n = 0; n < C::NCA; ++n) {
                const uint32_t mk = 0u - ((st.ok >> n) & 1u);
                st.a[n].raw &= u32x4{mk, mk, mk, mk};
            }
#pragma unroll
            for (int n = 0; n < C::NCB; ++n) {
                const uint32_t mk = 0u - ((st.ok >> (C::NCA + n)) & 1u);
                st.b[n].raw &= u32x4{mk, mk, mk, mk};
            }
        }
#pragma unroll
        for (int n = 0; n < C::NCA; ++n) {
            const int u = tid + n * C::NT;
            if (u < C::A_ROWS * C::A_CPR) {
                const int row = u / C::A_CPR, cc = u % C::A_CPR;
                st16(&As[buf * C::A_SIZE + row * C::A_STRIDE + cc * EPC], st.a[n]);
            }
        }
#pragma unroll
        for (int n = 0; n < C::NCB; ++n) {
            const int u = tid + n * C::NT;
            if (u < C::B_ROWS * C::B_CPR) {
                const int row = u / C::B_CPR, cc = u % C::B_CPR;
                st16(&Bs[buf * C::B_SIZE + row * C::B_STRIDE + cc * EPC], st.b[n]);
            }
        }
    };
    const bool k_ragged = K % C::BK != 0 && kt0 + nk == nk_all;  // this range ends on a ragged tile

    f32x16 acc[C::MB][C::NB];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) acc[mb][nb] = zero_acc();

    const int wrow = wm * (BM / WM), wcol = wn * (BN / WN);
    auto compute = [&](int buf) {
        const T* at = As + buf * C::A_SIZE;
        const T* bt = Bs + buf * C::B_SIZE;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
            for (int ps = 0; ps < C::PS; ++ps) {
                frag fa[C::MB], fb[C::NB];
#pragma unroll
                for (int mb = 0; mb < C::MB; ++mb) {
                    if constexpr (TA == 0)
                        fa[mb] = load_k_frag<T>(at + (wrow + mb * 32 + l32) * C::A_STRIDE + kb * 32, ps);
                    else
                        fa[mb] = load_rows_frag<T>(at, C::A_STRIDE, kb * 32, ps, wrow + mb * 32);
                }
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) {
                    if constexpr (TB == 1)
                        fb[nb] = load_k_frag<T>(bt + (wcol + nb * 32 + l32) * C::B_STRIDE + kb * 32, ps);
                    else
                        fb[nb] = load_rows_frag<T>(bt, C::B_STRIDE, kb * 32, ps, wcol + nb * 32);
                }
#pragma unroll
                for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < C::NB; ++nb) acc[mb][nb] = M_::mma(fb[nb], fa[mb], acc[mb][nb]);
            }
        }
    };

    // K tile s sits in register set s % NSET until it is committed at the start of step
    // s - 1; the set is then refilled with tile s + NSET.
    if (nk > 0) {
        fetch(sets[0], 0);
        commit(sets[0], 0, k_ragged && nk == 1);
    }
#pragma unroll
    for (int j = 1; j <= NSET; ++j)
        if (j < nk) fetch(sets[j % NSET], j);
    auto step = [&](int kt, Stg& nxt) {
        __syncthreads();  // tile kt visible in buffer kt&1; buffer (kt+1)&1 free
        if (kt + 1 < nk) {
            commit(nxt, (kt + 1) & 1, k_ragged && kt + 2 == nk);
            if (kt + 1 + NSET < nk) fetch(nxt, kt + 1 + NSET);
        }
        compute(kt & 1);
    };
    // Step kt commits tile kt + 1 from set (kt + 1) % NSET (the loop is unrolled NSET times so
    // that the set is a constant).
    for (int kt = 0; kt < nk; kt += NSET) {
#pragma unroll
        for (int j = 0; j < NSET; ++j)
            if (kt + j < nk) step(kt + j, sets[(j + 1) % NSET]);
    }

    // Split-K: partials in register order, [tile][slice][(mb, nb, r)][thread] (coalesced).
    constexpr int PART = C::MB * C::NB * 16 * C::NT;  // floats per partial tile
    if constexpr (MODE == 1) {
        float* dst = g.part + ((size_t)tile * g.ksplit + slice) * PART + tid;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) dst[((mb * C::NB + nb) * 16 + r) * C::NT] = acc[mb][nb][r];
        return;
    }
    if constexpr (MODE == 2) {
        const float* src = g.part + (size_t)tile * g.ksplit * PART + tid;
        for (int sl = 0; sl < g.ksplit; ++sl) {
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float v = src[(size_t)sl * PART + ((mb * C::NB + nb) * 16 + r) * C::NT];
                        acc[mb][nb][r] = sl == 0 ? v : acc[mb][nb][r] + v;
                    }
        }
    }

    // Epilogue: lane = row m, registers 4*a4 .. 4*a4+3 of block nb = columns
    // wcol + nb*32 + 8*a4 + 4*h + 0..3.
    const SegV<T> sc_(g.c);
    const int rope_mask = g.rope_mask;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
        const int m = m0 + wrow + mb * 32 + l32;
        if (m >= M) continue;
        const int t = rope_mask ? m % g.rope_T : 0;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int n = n0 + wcol + nb * 32 + 8 * a4 + 4 * h;
                if (n >= N) continue;
                const int s = sc_.index(n);
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = acc[mb][nb][4 * a4 + e];
                if ((rope_mask >> s) & 1) {
                    // Pairs (d, d+1), d even, of the head containing column n.
                    const int d0 = (n - (s == 2 ? sc_.st2 : (s == 1 ? sc_.st1 : 0))) % g.rope_D;
#pragma unroll
                    for (int e = 0; e < 4; e += 2) {
                        float co, sn;
                        rope_cos_sin((double)g.rope_pos0 + (double)t, g.f.theta[(d0 + e) >> 1], &co, &sn);
                        const float x0 = x[e], x1 = x[e + 1];
                        rope_rotate(x0, x1, co, sn, &x[e], &x[e + 1]);
                    }
                }
                T* cp = const_cast<T*>(sc_.at(m, n));
                if constexpr (sizeof(T) == 2) {
                    bf16x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (bf16)x[e];
                    *reinterpret_cast<bf16x4*>(cp) = v;
                } else {
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = x[e];
                    *reinterpret_cast<f32x4*>(cp) = v;
                }
            }
        }
    }
}

// Split-K slices for a grid of `tiles` output tiles and nk K tiles: enough (tile, slice) units
// for two per CU, each slice keeping at least 8 K tiles; 1 (no split) when the tiles already
// fill the chip or K is short.
inline int pick_ksplit(long long tiles, int nk) {
    if (tiles >= 256 || nk < 16) return 1;
    const int want = (int)((512 + tiles - 1) / tiles);
    return std::max(1, std::min(std::min(want, nk / 8), 8));
}

template <typename T, int TA, int TB, int BM, int BN, int WM, int WN>
hipError_t launch_cfg(GemmArgs g, float* ws, size_t ws_bytes, hipStream_t stream) {
    g.tiles_n = (g.N + BN - 1) / BN;
    g.tiles_m = (g.M + BM - 1) / BM;
    const long long blocks = (long long)g.tiles_m * g.tiles_n;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    using C = GemmCfg<T, TA, TB, BM, BN, WM, WN>;
    // Only the 64 x 64 tiles split (the 128 x 128 ones are chosen when the tiles fill the chip).
    if constexpr (BM == 64 && BN == 64) {
        const int ks = ws ? pick_ksplit(blocks, (g.K + C::BK - 1) / C::BK) : 1;
        const size_t need = (size_t)blocks * ks * BM * BN * sizeof(float);
        if (ks > 1 && need <= ws_bytes && blocks * ks <= 0x7fffffffLL) {
            g.ksplit = ks;
            g.part = ws;
            hipLaunchKernelGGL((gemm_kernel<T, TA, TB, BM, BN, WM, WN, 1>), dim3((unsigned)(blocks * ks)),
                               dim3(64 * WM * WN), 0, stream, g);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((gemm_kernel<T, TA, TB, BM, BN, WM, WN, 2>), dim3((unsigned)blocks),
                               dim3(64 * WM * WN), 0, stream, g);
            return hipGetLastError();
        }
    }
    g.ksplit = 1;
    g.part = nullptr;
    hipLaunchKernelGGL((gemm_kernel<T, TA, TB, BM, BN, WM, WN>), dim3((unsigned)blocks),
                       dim3(64 * WM * WN), 0, stream, g);
    return hipGetLastError();
}

template <typename T, int BM, int BN, int WM, int WN>
size_t ws_cfg(int M, int N, int K) {
    constexpr int BK = GemmCfg<T, 0, 0, BM, BN, WM, WN>::BK;
    const long long blocks = (long long)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int ks = pick_ksplit(blocks, (K + BK - 1) / BK);
    return ks > 1 ? (size_t)blocks * ks * BM * BN * sizeof(float) : 0;
}

// Tile shape: 128 x 128 (4 waves of 64 x 64) when that still gives every CU two tiles, or one
// tile and a long K; else 64 x 64 (4 waves of 32 x 32) for more, smaller workgroups.
inline bool big_tiles(int M, int N, int K) {
    const long long t = (long long)((M + 127) / 128) * ((N + 127) / 128);
    return t >= 512 || (t >= 256 && K >= 2048);
}

template <typename T, int TA, int TB>
hipError_t launch_t(const GemmArgs& g, float* ws, size_t ws_bytes, hipStream_t stream) {
    if (big_tiles(g.M, g.N, g.K)) return launch_cfg<T, TA, TB, 128, 128, 2, 2>(g, ws, ws_bytes, stream);
    return launch_cfg<T, TA, TB, 64, 64, 2, 2>(g, ws, ws_bytes, stream);
}

template <typename T>
hipError_t launch_dt(const GemmArgs& g, int ta, int tb, float* ws, size_t ws_bytes, hipStream_t stream) {
    if (ta == 0 && tb == 0) return launch_t<T, 0, 0>(g, ws, ws_bytes, stream);
    if (ta == 0 && tb == 1) return launch_t<T, 0, 1>(g, ws, ws_bytes, stream);
    if (ta == 1 && tb == 0) return launch_t<T, 1, 0>(g, ws, ws_bytes, stream);
    return hipErrorInvalidValue;
}

void fill_segs(Seg* dst, const GemmSeg* src, int n) {
    for (int s = 0; s < kGemmMaxSeg; ++s) {
        if (s < n) {
            dst[s].p = src[s].p;
            dst[s].ld = src[s].ld;
            dst[s].start = src[s].start;
        } else {
            dst[s].p = src[0].p;
            dst[s].ld = src[0].ld;
            dst[s].start = INT_MAX;
        }
    }
}

}  // namespace

size_t gemm_splitk_bytes(int M, int N, int K, IoType dt) {
    if (big_tiles(M, N, K)) return 0;
    return dt == kF32 ? ws_cfg<float, 64, 64, 2, 2>(M, N, K) : ws_cfg<bf16, 64, 64, 2, 2>(M, N, K);
}

hipError_t launch_gemm(const GemmSeg* a, int na, const GemmSeg* b, int nb, const GemmSeg* c,
                       int nc, int M, int N, int K, int trans_a, int trans_b, IoType dt,
                       const GemmRope* rope, hipStream_t stream, void* splitk_ws, size_t splitk_bytes) {
    GemmArgs g{};
    fill_segs(g.a, a, na);
    fill_segs(g.b, b, nb);
    fill_segs(g.c, c, nc);
    g.M = M;
    g.N = N;
    g.K = K;
    g.rope_mask = 0;
    g.rope_T = 1;
    g.rope_D = 2;
    if (rope != nullptr) {
        g.rope_mask = rope->mask;
        g.rope_T = rope->T;
        g.rope_D = rope->D;
        g.rope_pos0 = rope->pos0;
        fill_rope_freq(&g.f, rope->D, rope->base);
    }
    float* ws = static_cast<float*>(splitk_ws);
    return dt == kF32 ? launch_dt<float>(g, trans_a, trans_b, ws, splitk_bytes, stream)
                      : launch_dt<bf16>(g, trans_a, trans_b, ws, splitk_bytes, stream);
}

}  // namespace ea
