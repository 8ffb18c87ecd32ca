// attn_decode.hip -- causal GQA attention of a few new query rows against a KV cache on
// gfx950 (attn_decode).
//
// What it computes: the causal attention of the pages ("Tiny Hackable CUDA Language Model
// Implementation", section 1; shared K/V heads, "Show HN: NanoEuler", section 2) for the
// last Tq positions of a Tk-long sequence, the step of generation with a cache (one token,
// or the K tokens of multi-token speculative decoding, "Show HN: NanoEuler", section 2):
// query row i sits at position Tk - Tq + i and attends to the keys s <= Tk - Tq + i.
//
// The work is HBM-bound (every key and value row of the cache is read once per K/V head, and
// there are few queries to reuse it), so the design is about bytes in flight, not matrix
// cores:
//  * Rows.  The g query heads sharing a K/V head and the Tq tokens form R = g * Tq rows,
//    row r = i * g + hs; each wave takes a block of 32 rows as the columns of its MFMA
//    tiles (S^T = K Q^T, O^T += V^T P^T, as in attn_fwd), so one read of a key row serves
//    every head of the group and every new token.  bf16 at head_dim 64 and 128 uses 16 x 16
//    x 32 products on 16-row halves of the block (a second half only where the block has
//    more than 16 rows), since R is usually 16 or less: half the padding work, half the
//    softmax lanes' values per tile, and far fewer registers when no block needs a second
//    half.
//  * Split over the cache (split-K): each wave streams its own chunk of keys, 32 at a time;
//    K rows go straight from HBM into the operand registers (the "split" layout is 16-byte
//    runs of a key row), V rows through a wave-private LDS tile for the transposing read of
//    V^T.  The next tile's loads are issued before the current tile is computed.  No
//    barriers: each wave is independent.
//  * Each chunk leaves a partial (O_c, LSE_c) in the workspace; a second kernel merges the
//    chunks exactly, LSE = log sum_c e^{LSE_c}, O = sum_c e^{LSE_c - LSE} O_c (or the first
//    kernel writes O and LSE directly when there is one chunk).  Small caches (a few chunks)
//    take one launch instead: one workgroup per row block, a wave per chunk, the same merge
//    through LDS.
#include <cmath>
#include <type_traits>

#include "ea_common.h"
#include "ea_kernels.h"

namespace ea {
namespace {

constexpr int kKT = 32;          // keys per tile
constexpr int kWavesPerWG = 4;

struct DecArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    float* part_o;    // [items][32 rows][D] fp32 (items = B * Hkv * nrb * nsplit)
    float* part_lse;  // [items][32 rows] natural log, -inf for a row with no key in the chunk
    int B, Tq, Tk, Hq, Hkv, g, R, nrb, nsplit, chunk;
    float sl2;  // scale * log2(e)
};

template <typename T, int D>
struct DecCfg {
    static constexpr int KPL = Mfma<T>::KPL;
    static constexpr int NS = D / (2 * KPL);  // MFMA steps over head_dim
    static constexpr int NDB = D / 32;
    static constexpr int PS = 16 / KPL;       // MFMA steps over the 32 keys of a tile
    static constexpr int EPC = 16 / sizeof(T);
    static constexpr int CPR = D / EPC;       // 16-byte chunks per row
    static constexpr int VS = D + EPC;        // V tile row stride in LDS (16 bytes of padding)
    static constexpr int VCH = kKT * CPR / 64;  // V chunks per lane per tile
    static constexpr int KCH = (D / 2) / EPC;   // K chunks per lane per tile
    static_assert(kKT * CPR % 64 == 0, "V tile staging");
};

// One wave: chunk sp of row block rb of K/V head kvh in batch b.  On return oacc holds the
// chunk's output O_c (normalised by its own row sums; lane = row l32, registers = head_dim
// as in the accumulator layout) and lse its LSE_c (natural log, -inf for a row that sees no
// key of the chunk).  Vs: this wave's private V tile in LDS.
template <typename T, int D>
__device__ __forceinline__ void decode_chunk(const DecArgs& a, T* Vs, int b, int kvh, int rb, int sp,
                                             f32x16 (&oacc)[DecCfg<T, D>::NDB], float& lse) {
    using C = DecCfg<T, D>;
    using M = Mfma<T>;
    using frag = typename M::frag;
    constexpr int KPL = C::KPL;

    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;

    const T* __restrict__ qp = static_cast<const T*>(a.q);
    const T* __restrict__ kp = static_cast<const T*>(a.k);
    const T* __restrict__ vp = static_cast<const T*>(a.v);
    const int off = a.Tk - a.Tq;

    // This lane's row (MFMA column): token i, head hs of the group; -1 keys for padding rows.
    const int r = rb * 32 + l32;
    const bool row_ok = r < a.R;
    const int ti = row_ok ? r / a.g : 0;
    const int hs = row_ok ? r % a.g : 0;
    const int head = kvh * a.g + hs;
    const int lastkey = row_ok ? off + ti : -1;
    // Keys of this chunk that any row of the block sees.
    const int rlast = min(a.R, rb * 32 + 32) - 1;
    const int kend_block = off + rlast / a.g + 1;
    const int k0 = sp * a.chunk;
    const int k1 = min(k0 + a.chunk, kend_block);
    const int ntiles = k1 > k0 ? (k1 - k0 + kKT - 1) / kKT : 0;

    frag qf[C::NS];
    if (row_ok) {
        const T* row = qp + (((long long)b * a.Tq + ti) * a.Hq + head) * D + half * (D / 2);
#pragma unroll
        for (int c = 0; c < (D / 2) / C::EPC; ++c) {
            const Vec16<T> v = ld16(row + c * C::EPC);
#pragma unroll
            for (int e = 0; e < C::EPC / KPL; ++e) qf[c * (C::EPC / KPL) + e] = reinterpret_cast<const frag*>(&v.raw)[e];
        }
    } else {
#pragma unroll
        for (int s = 0; s < C::NS; ++s) qf[s] = frag{};
    }

    // Tile loads: K rows straight into the split operand (lane = key l32, half of head_dim),
    // V rows as 16-byte chunks for the LDS tile.  Rows past the chunk read as zero.
    Vec16<T> kreg[C::KCH], vreg[C::VCH];
    const long long kv_row0 = (long long)b * a.Tk;
    auto fetch = [&](int t) {
        const int s = k0 + t * kKT + l32;
        const bool ok = s < k1;
        const T* krow = kp + ((kv_row0 + s) * a.Hkv + kvh) * D + half * (D / 2);
#pragma unroll
        for (int c = 0; c < C::KCH; ++c) kreg[c] = ok ? ld16(krow + c * C::EPC) : zero16<T>();
#pragma unroll
        for (int n = 0; n < C::VCH; ++n) {
            const int u = lane + 64 * n;
            const int key = u / C::CPR, part = u % C::CPR;
            const int sv = k0 + t * kKT + key;
            vreg[n] = (sv < k1) ? ld16(vp + ((kv_row0 + sv) * a.Hkv + kvh) * D + part * C::EPC) : zero16<T>();
        }
    };
    auto wave_sync = [&]() {  // LDS writes of this wave visible to its later reads, and back
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    float mrun = -INFINITY, l = 0.0f;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) oacc[db] = zero_acc();

    if (ntiles > 0) fetch(0);
    for (int t = 0; t < ntiles; ++t) {
        // Commit V of tile t to LDS; take K of tile t from the registers.
        wave_sync();  // the previous tile's V reads are done
#pragma unroll
        for (int n = 0; n < C::VCH; ++n) {
            const int u = lane + 64 * n;
            st16(&Vs[(u / C::CPR) * C::VS + (u % C::CPR) * C::EPC], vreg[n]);
        }
        frag kf[C::NS];
#pragma unroll
        for (int c = 0; c < C::KCH; ++c)
#pragma unroll
            for (int e = 0; e < C::EPC / KPL; ++e) kf[c * (C::EPC / KPL) + e] = reinterpret_cast<const frag*>(&kreg[c].raw)[e];
        wave_sync();
        if (t + 1 < ntiles) fetch(t + 1);

        // S^T = K Q^T (lanes = rows, registers = keys), masked where key > the row's last key.
        f32x16 sacc = zero_acc();
#pragma unroll
        for (int s = 0; s < C::NS; ++s) sacc = M::mma(kf[s], qf[s], sacc);
        const int kbase = k0 + t * kKT;
        float mx = -INFINITY;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            if (kbase + acc_row(rr, half) > lastkey) sacc[rr] = -INFINITY;
            mx = fmaxf(mx, sacc[rr]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * a.sl2;
        const float mnew = fmaxf(mrun, mx);
        const float mbase = (mnew == -INFINITY) ? 0.0f : mnew;  // rows with no key so far
        const float alpha = __builtin_amdgcn_exp2f(mrun - mbase);
        float rs = 0.0f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const float p = __builtin_amdgcn_exp2f(sacc[rr] * a.sl2 - mbase);
            sacc[rr] = p;
            rs += p;
        }
        l = l * alpha + rs;
        mrun = mnew;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) oacc[db][rr] *= alpha;
        // O^T += V^T P^T.
#pragma unroll
        for (int ps = 0; ps < C::PS; ++ps) {
            const frag pf = acc_to_frag<T>(sacc, ps * KPL);
#pragma unroll
            for (int db = 0; db < C::NDB; ++db)
                oacc[db] = M::mma(load_rows_frag<T>(Vs, C::VS, 0, ps, db * 32), pf, oacc[db]);
        }
    }

    // Row totals (the two lane halves hold different keys) and the chunk's result.
    const float lt = l + __shfl_xor(l, 32, 64);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    lse = lt > 0.0f ? (mrun + __log2f(lt)) * kLn2 : -INFINITY;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) oacc[db][rr] *= inv;
}

// bf16: the same chunk on 16 x 16 x 32 products, whose 16 columns hold the rows (the g heads x
// Tq tokens of a group are 16 or fewer in the usual shapes, so the 32-column products of
// decode_chunk compute mostly padding).  Rows rb * 32 + 16 hb + (lane % 16): hb = 0, and hb = 1
// only when the block has more than 16 rows.  Lane groups q = lane / 16 hold, for each 16-key
// block kb, the scores of keys 16 kb + 4 q + 0..3 (the accumulator rows 4 q .. 4 q + 3), so a
// row's 32 keys of a tile sit in the four lanes with the same lane % 16.  For O^T += V^T P^T
// the contraction slots 8 q + e take keys 4 q + e (e < 4) and 16 + 4 q + (e - 4): P^T comes
// straight from the lane's own scores, V^T from two transposing reads of the LDS tile.  On
// return oacc[hb][db][i] is O_c of row 16 hb + lane % 16, head_dim 16 db + 4 q + i (normalised
// by its own row sums) and lse[hb] that row's LSE_c (natural log, -inf with no key).
// Which launches take the 16-row products: bf16 with head_dim 64 and 128 (at head_dim 32 the
// 32-row products measured faster).
template <typename T, int D>
constexpr bool kDec16 = sizeof(T) == 2 && D >= 64;

__device__ inline f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x4 tr4(const bf16* p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    return __builtin_bit_cast(bf16x4, v);
}

// NH: 16-row halves the kernel may meet (1 when every row block has at most 16 rows).
template <int D, int NH>
__device__ __forceinline__ void decode_chunk16(const DecArgs& a, bf16* Vs, int b, int kvh, int rb, int sp,
                                               f32x4 (&oacc)[NH][D / 16], float (&lse)[NH]) {
    using T = bf16;
    using C = DecCfg<T, D>;
    constexpr int NST = D / 32;  // 32-deep steps over head_dim
    constexpr int NDB = D / 16;  // 16-wide head_dim blocks of O
    const int lane = threadIdx.x & 63;
    const int q4 = lane >> 4;
    const int c16 = lane & 15;

    const T* __restrict__ qp = static_cast<const T*>(a.q);
    const T* __restrict__ kp = static_cast<const T*>(a.k);
    const T* __restrict__ vp = static_cast<const T*>(a.v);
    const int off = a.Tk - a.Tq;
    const bool two = NH == 2 && rb * 32 + 16 < a.R;  // uniform: a second 16-row half

    int lastkey[NH];
    bf16x8 qf[NH][NST];
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
        const int r = rb * 32 + 16 * hb + c16;
        const bool row_ok = r < a.R;
        const int ti = row_ok ? r / a.g : 0;
        const int head = kvh * a.g + (row_ok ? r % a.g : 0);
        lastkey[hb] = row_ok ? off + ti : -1;
        const T* row = qp + (((long long)b * a.Tq + ti) * a.Hq + head) * D + 8 * q4;
#pragma unroll
        for (int s = 0; s < NST; ++s) {
            bf16x8 v{};
            if (row_ok && (hb == 0 || two)) v = __builtin_bit_cast(bf16x8, ld16(row + 32 * s).raw);
            qf[hb][s] = v;
        }
    }
    // Keys of this chunk that any row of the block sees.
    const int rlast = min(a.R, rb * 32 + 32) - 1;
    const int kend_block = off + rlast / a.g + 1;
    const int k0 = sp * a.chunk;
    const int k1 = min(k0 + a.chunk, kend_block);
    const int ntiles = k1 > k0 ? (k1 - k0 + kKT - 1) / kKT : 0;

    // A row past the chunk's last key is masked for every row of the block (chunks are whole
    // tiles, so a tile crosses k1 only where k1 is past the block's last row's key).
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) lastkey[hb] = min(lastkey[hb], k1 - 1);

    // Tile loads: K and V rows as 16-byte chunks for the wave's LDS tiles, consecutive lanes on
    // consecutive chunks of a row, so that each load instruction covers whole rows (loading K
    // straight into the product operand would take sixteen half rows per instruction, and the
    // CU's load path, not HBM, bounds the small-batch cases).  Each lane keeps running row
    // pointers, one tile apart per step, instead of forming every address again; a row past
    // the chunk reads the chunk's last row instead, whose key the mask removes (P = 0 there), so
    // no load is conditional.
    Vec16<T> kreg[C::VCH], vreg[C::VCH];
    constexpr int VROWS = 64 / C::CPR;           // rows between a lane's successive chunks
    const long long rs = (long long)a.Hkv * D;  // elements from one cache row to the next
    const long long head0 = ((long long)b * a.Tk * a.Hkv + kvh) * D + (lane % C::CPR) * C::EPC;
    const int vkey = lane / C::CPR;  // this lane's first row within a tile
    const long long klast = max(k1 - 1, 0);
    const T* kcl = kp + head0 + klast * rs;
    const T* vcl = vp + head0 + klast * rs;
    const T* kr = kp + head0 + (k0 + vkey) * rs;
    const T* vr = vp + head0 + (k0 + vkey) * rs;
    auto fetch = [&](int t) {  // called once per tile, in order
        const int lim = k1 - k0 - t * kKT;  // rows of this tile inside the chunk
#pragma unroll
        for (int n = 0; n < C::VCH; ++n) {
            const bool in = vkey + VROWS * n < lim;
            kreg[n] = ld16(in ? kr + VROWS * n * rs : kcl);
            vreg[n] = ld16(in ? vr + VROWS * n * rs : vcl);
        }
        kr += kKT * rs;
        vr += kKT * rs;
    };
    T* const Ks = Vs + kKT * C::VS;  // the K tile, after the V tile
    auto wave_sync = [&]() {  // LDS writes of this wave visible to its later reads, and back
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    auto rowmax = [](float x) {
        x = fmaxf(x, __shfl_xor(x, 16, 64));
        return fmaxf(x, __shfl_xor(x, 32, 64));
    };

    float mrun[NH], l[NH];
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
        mrun[hb] = -INFINITY;
        l[hb] = 0.0f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[hb][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // Transposing-read addresses of V^T (keys 4 q4 + (c16 >> 2), then 16 more; head_dim
    // 16 db + 4 (c16 & 3)).
    const T* vt0 = Vs + (4 * q4 + (c16 >> 2)) * C::VS + 4 * (c16 & 3);

    if (ntiles > 0) fetch(0);
    for (int t = 0; t < ntiles; ++t) {
        // Commit K and V of tile t to LDS, then read K's operand fragments back (lane = key c16
        // of block kb, head_dim 32 s + 8 q4 .. +7).
        wave_sync();  // the previous tile's K and V reads are done
#pragma unroll
        for (int n = 0; n < C::VCH; ++n) {
            const int u = lane + 64 * n;
            st16(&Vs[(u / C::CPR) * C::VS + (u % C::CPR) * C::EPC], vreg[n]);
            st16(&Ks[(u / C::CPR) * C::VS + (u % C::CPR) * C::EPC], kreg[n]);
        }
        wave_sync();
        bf16x8 kf[2][NST];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int st = 0; st < NST; ++st)
                kf[kb][st] = __builtin_bit_cast(bf16x8, ld16(&Ks[(16 * kb + c16) * C::VS + 32 * st + 8 * q4]).raw);
        if (t + 1 < ntiles) fetch(t + 1);

        const int kbase = k0 + t * kKT;
#pragma unroll
        for (int hb = 0; hb < NH; ++hb) {
            if (hb == 1 && !two) break;
            // S^T = K Q^T for the two 16-key blocks, masked where key > the row's last key.
            f32x4 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sacc[kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int st = 0; st < NST; ++st) sacc[kb] = mma16(kf[kb][st], qf[hb][st], sacc[kb]);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (kbase + 16 * kb + 4 * q4 + i > lastkey[hb]) sacc[kb][i] = -INFINITY;
                    mx = fmaxf(mx, sacc[kb][i]);
                }
            mx = rowmax(mx) * a.sl2;
            const float mnew = fmaxf(mrun[hb], mx);
            const float mbase = (mnew == -INFINITY) ? 0.0f : mnew;  // rows with no key so far
            const float alpha = __builtin_amdgcn_exp2f(mrun[hb] - mbase);
            float rs = 0.0f;
            bf16x8 pf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = __builtin_amdgcn_exp2f(sacc[kb][i] * a.sl2 - mbase);
                    rs += p;
                    pf[4 * kb + i] = (bf16)p;
                }
            l[hb] = l[hb] * alpha + rs;  // this lane's share of the row sum
            mrun[hb] = mnew;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                oacc[hb][db] *= alpha;
                const bf16x4 lo = tr4(vt0 + 16 * db);
                const bf16x4 hi = tr4(vt0 + 16 * C::VS + 16 * db);
                bf16x8 vf;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vf[e] = lo[e];
                    vf[4 + e] = hi[e];
                }
                oacc[hb][db] = mma16(vf, pf, oacc[hb][db]);
            }
        }
    }

    // Row totals (four lanes share a row) and the chunk's result.
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
        float lt = l[hb] + __shfl_xor(l[hb], 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        lse[hb] = lt > 0.0f ? (mrun[hb] + __log2f(lt)) * kLn2 : -INFINITY;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[hb][db] *= inv;
    }
}

// The split launch: one wave per (batch, K/V head, row block, chunk); with several chunks the
// partials go to the workspace for decode_merge_kernel, with one chunk straight to O and LSE.
template <typename T, int D, int NH>
__global__ __launch_bounds__(64 * kWavesPerWG) void decode_partial_kernel(DecArgs a) {
    using C = DecCfg<T, D>;
    constexpr int VT = kDec16<T, D> ? 2 * kKT : kKT;  // rows staged per wave (K too on the 16-row path)
    __shared__ __attribute__((aligned(16))) T Vsh[kWavesPerWG * VT * C::VS];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const long long item = (long long)blockIdx.x * kWavesPerWG + w;
    const long long nitems = (long long)a.B * a.Hkv * a.nrb * a.nsplit;
    if (item >= nitems) return;
    const int sp = (int)(item % a.nsplit);
    long long rest = item / a.nsplit;
    const int rb = (int)(rest % a.nrb);
    rest /= a.nrb;
    const int kvh = (int)(rest % a.Hkv);
    const int b = (int)(rest / a.Hkv);

    if constexpr (kDec16<T, D>) {
        f32x4 o16[NH][D / 16];
        float l16[NH];
        decode_chunk16<D, NH>(a, Vsh + w * VT * C::VS, b, kvh, rb, sp, o16, l16);
        const int q4 = lane >> 4, c16 = lane & 15;
#pragma unroll
        for (int hb = 0; hb < NH; ++hb) {
            const int rr = 16 * hb + c16;  // row within the block
            const int r = rb * 32 + rr;
            if (r >= a.R) continue;  // padding rows; the merge reads real rows only
            if (a.nsplit == 1) {
                const int ti = r / a.g, head = kvh * a.g + r % a.g;
                T* orow = static_cast<T*>(a.o) + (((long long)b * a.Tq + ti) * a.Hq + head) * D;
#pragma unroll
                for (int db = 0; db < D / 16; ++db) {
                    bf16x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = from_f32<T>(o16[hb][db][i]);
                    *reinterpret_cast<bf16x4*>(orow + 16 * db + 4 * q4) = v;
                }
                if (q4 == 0) a.lse[((long long)b * a.Hq + head) * a.Tq + ti] = l16[hb];
            } else {
                float* po = a.part_o + item * 32 * D + (long long)rr * D;
#pragma unroll
                for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4*>(po + 16 * db + 4 * q4) = o16[hb][db];
                if (q4 == 0) a.part_lse[item * 32 + rr] = l16[hb];
            }
        }
        return;
    }
    f32x16 oacc[C::NDB];
    float lse;
    decode_chunk<T, D>(a, Vsh + w * VT * C::VS, b, kvh, rb, sp, oacc, lse);

    const int r = rb * 32 + l32;
    if (r >= a.R) return;  // padding rows; the merge reads real rows only
    if (a.nsplit == 1) {
        const int ti = r / a.g, head = kvh * a.g + r % a.g;
        T* orow = static_cast<T*>(a.o) + (((long long)b * a.Tq + ti) * a.Hq + head) * D;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) orow[db * 32 + acc_row(rr, half)] = from_f32<T>(oacc[db][rr]);
        if (half == 0) a.lse[((long long)b * a.Hq + head) * a.Tq + ti] = lse;
        return;
    }
    float* po = a.part_o + item * 32 * D + (long long)l32 * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) po[db * 32 + acc_row(rr, half)] = oacc[db][rr];
    if (half == 0) a.part_lse[item * 32 + l32] = lse;
}

// The single launch for caches of at most NW chunks: one workgroup per (batch, K/V head, row
// block), wave w computing chunk w.  Each wave writes its partial (O_c, LSE_c) to its own LDS
// region as soon as its chunk is done (the partials do not overlap the V tiles, so no wave
// waits for another before writing).  The merge is decode_merge_kernel's, step for step:
// one thread per (row, chunk) forms the weight e^{LSE_c - m}, and every thread then merges
// the output elements it stores (the row's weights summed in chunk order, one reciprocal, the
// chunks' values in order).
// Waves of the single launch, sized so that each wave keeps the split launch's registers
// (four waves per SIMD for bf16 head_dim 32, two for head_dim 64 and fp32 head_dim 32, one
// for head_dim 128).
template <typename T, int D>
constexpr int fused_max_chunks() {
    return D >= 128 ? 4 : (sizeof(T) == 2 && D <= 32) ? 16 : 8;
}

template <typename T, int D, int NH>
__global__ __launch_bounds__((64 * fused_max_chunks<T, D>())) void decode_fused_kernel(DecArgs a) {
    using C = DecCfg<T, D>;
    constexpr int NW = fused_max_chunks<T, D>();
    constexpr int PST = D + 1;  // row stride of a partial (odd: lanes of one column on distinct banks)
    constexpr int VT = kDec16<T, D> ? 2 * kKT : kKT;  // rows staged per wave (K too on the 16-row path)
    constexpr size_t V_BYTES = (size_t)NW * VT * C::VS * sizeof(T);
    constexpr size_t P_BYTES = (size_t)NW * 32 * PST * sizeof(float);
    static_assert(V_BYTES % 16 == 0 && V_BYTES + P_BYTES + 2 * NW * 32 * sizeof(float) <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) char smem[V_BYTES + P_BYTES + 2 * NW * 32 * sizeof(float)];
    float* part = reinterpret_cast<float*>(smem + V_BYTES);
    float* lses = reinterpret_cast<float*>(smem + V_BYTES + P_BYTES);  // LSE_c of (chunk, row)
    float* wts = lses + NW * 32;                                        // its weight

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int ns = a.nsplit;  // == blockDim.x / 64
    const int rb = blockIdx.x % a.nrb;
    const int kvh = (blockIdx.x / a.nrb) % a.Hkv;
    const int b = blockIdx.x / (a.nrb * a.Hkv);

    if constexpr (kDec16<T, D>) {
        f32x4 o16[NH][D / 16];
        float l16[NH];
        decode_chunk16<D, NH>(a, reinterpret_cast<T*>(smem) + w * VT * C::VS, b, kvh, rb, w, o16, l16);
        const int q4 = lane >> 4, c16 = lane & 15;
#pragma unroll
        for (int hb = 0; hb < NH; ++hb) {
            const int rr = 16 * hb + c16;
            float* po = part + (size_t)w * 32 * PST + rr * PST;
#pragma unroll
            for (int db = 0; db < D / 16; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) po[16 * db + 4 * q4 + i] = o16[hb][db][i];
            if (q4 == 0) lses[w * 32 + rr] = l16[hb];
        }
    } else {
        f32x16 oacc[C::NDB];
        float lse;
        decode_chunk<T, D>(a, reinterpret_cast<T*>(smem) + w * VT * C::VS, b, kvh, rb, w, oacc, lse);
        float* po = part + (size_t)w * 32 * PST + l32 * PST;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) po[db * 32 + acc_row(rr, half)] = oacc[db][rr];
        if (half == 0) lses[w * 32 + l32] = lse;
    }
    __syncthreads();
    // Chunk weights e^{LSE_c - m}, one thread per (row, chunk) (m: the row's largest LSE_c;
    // chunk 0 holds key 0, which every row sees, so m is finite).
    const int nrows = min(32, a.R - rb * 32);
    const int wr = tid % 32, wch = tid / 32;
    if (wr < nrows && wch < ns) {
        float m = -INFINITY;
        for (int c = 0; c < ns; ++c) m = fmaxf(m, lses[c * 32 + wr]);
        const float ls = lses[wch * 32 + wr];
        wts[wch * 32 + wr] = (ls == -INFINITY) ? 0.0f : expf(ls - m);
    }
    __syncthreads();
    // Each thread merges the output elements it stores: the row's weights summed in chunk order,
    // one reciprocal, then the chunks' values in order; the thread of column 0 writes the row's
    // LSE = m + log(sum).
    for (int e = tid; e < nrows * D; e += ns * 64) {
        const int rl = e / D, d = e % D;
        float z = 0.0f;
        for (int c = 0; c < ns; ++c) z += wts[c * 32 + rl];
        const float iz = 1.0f / z;
        float acc = 0.0f;
        for (int c = 0; c < ns; ++c) acc += (wts[c * 32 + rl] * iz) * part[((size_t)c * 32 + rl) * PST + d];
        const int r = rb * 32 + rl;
        const int ti = r / a.g, head = kvh * a.g + r % a.g;
        static_cast<T*>(a.o)[(((long long)b * a.Tq + ti) * a.Hq + head) * D + d] = from_f32<T>(acc);
        if (d == 0) {
            float m = -INFINITY;
            for (int c = 0; c < ns; ++c) m = fmaxf(m, lses[c * 32 + rl]);
            a.lse[((long long)b * a.Hq + head) * a.Tq + ti] = m + logf(z);
        }
    }
}

// Merge of the chunks: one wave per row.  The lanes first take the chunks' LSE values (max,
// then weights e^{LSE_c - m} kept in LDS and their sum), then the columns of the row, each
// lane summing its columns over the chunks in chunk order (deterministic).
constexpr int kMaxSplit = 256;

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecArgs a) {
    constexpr int CPL = D >= 64 ? D / 64 : 1;  // columns per lane
    constexpr int NB = 16;                      // chunks whose values are loaded up front
    constexpr int LPL = kMaxSplit / 64;         // LSE values per lane
    __shared__ float wsh[kMaxSplit];
    const int lane = threadIdx.x;
    const long long row = blockIdx.x;  // (b * Hkv + kvh) * R + r
    const int r = (int)(row % a.R);
    const long long bk = row / a.R;
    const int kvh = (int)(bk % a.Hkv);
    const int b = (int)(bk / a.Hkv);
    const int rb = r / 32, rl = r % 32;
    const long long item0 = (bk * a.nrb + rb) * a.nsplit;
    const int ns = a.nsplit;
    const bool cols = lane * CPL < D;
    // Lanes past the row's columns (head_dim 32) read column 0 and store nothing.
    const float* po = a.part_o + (item0 * 32 + rl) * D + (cols ? lane * CPL : 0);
    // Every load that does not depend on another goes out first: the row's LSE_c values (lane
    // sp % 64 holds chunk sp) and this lane's columns of the first NB chunks, so the kernel
    // waits for memory once.
    float lsv[LPL];
#pragma unroll
    for (int k = 0; k < LPL; ++k) {
        const int sp = lane + 64 * k;
        const float v = a.part_lse[(item0 + min(sp, ns - 1)) * 32 + rl];  // clamped: no branch
        lsv[k] = sp < ns ? v : -INFINITY;
    }
    float pv[NB][CPL];  // chunks past the last re-read the last one and are never used
#pragma unroll
    for (int sp = 0; sp < NB; ++sp)
#pragma unroll
        for (int c = 0; c < CPL; ++c) pv[sp][c] = po[(long long)min(sp, ns - 1) * 32 * D + c];
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < LPL; ++k) m = fmaxf(m, lsv[k]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float z = 0.0f;
#pragma unroll
    for (int k = 0; k < LPL; ++k) {
        const int sp = lane + 64 * k;
        if (sp < ns) {
            const float wgt = (lsv[k] == -INFINITY) ? 0.0f : expf(lsv[k] - m);
            wsh[sp] = wgt;
            z += wgt;
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o, 64);
    __syncthreads();
    const int ti = r / a.g, head = kvh * a.g + r % a.g;
    if (cols) {
        float acc[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] = 0.0f;
#pragma unroll
        for (int sp = 0; sp < NB; ++sp) {
            if (sp < ns) {
                const float wgt = wsh[sp];
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[c] += wgt * pv[sp][c];
            }
        }
#pragma unroll 8
        for (int sp = NB; sp < ns; ++sp) {
            const float wgt = wsh[sp];
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c] += wgt * po[(long long)sp * 32 * D + c];
        }
        const float inv = 1.0f / z;  // every row sees key 0, so some chunk has weight 1
        T* orow = static_cast<T*>(a.o) + (((long long)b * a.Tq + ti) * a.Hq + head) * D + lane * CPL;
#pragma unroll
        for (int c = 0; c < CPL; ++c) orow[c] = from_f32<T>(acc[c] * inv);
    }
    if (lane == 0) a.lse[((long long)b * a.Hq + head) * a.Tq + ti] = m + logf(z);
}

// Chunking: enough independent waves to keep HBM busy (about 8 per CU), chunks of whole
// 32-key tiles, at least two tiles each.
struct DecPlan {
    int nrb, nsplit, chunk;
};

DecPlan plan_decode(int B, int Tq, int Tk, int Hq, int Hkv) {
    const int g = Hq / Hkv;
    DecPlan p;
    p.nrb = (g * Tq + 31) / 32;
    const long long base = (long long)B * Hkv * p.nrb;
    const long long target = 2048;
    const int tiles = (Tk + kKT - 1) / kKT;
    long long ns = (target + base - 1) / base;
    ns = std::min<long long>(ns, std::max(1, tiles / 2));
    ns = std::min<long long>(ns, kMaxSplit);
    ns = std::max<long long>(ns, 1);
    const int tiles_per = (int)((tiles + ns - 1) / ns);
    p.chunk = tiles_per * kKT;
    p.nsplit = (Tk + p.chunk - 1) / p.chunk;
    return p;
}

template <typename T, int D, int NH>
hipError_t launch_decode_nh(DecArgs a, hipStream_t stream) {
    // Caches split into at most twice as many chunks as the single launch has waves take the
    // single launch, with fewer, longer chunks: the second launch and the workspace round trip
    // cost more there than the waves the split would add.
    constexpr int F = fused_max_chunks<T, D>();
    if (a.nsplit > 1 && a.nsplit <= 2 * F) {
        const int tiles = (a.Tk + kKT - 1) / kKT;
        const int ns = a.nsplit < F ? a.nsplit : F;
        a.chunk = ((tiles + ns - 1) / ns) * kKT;
        a.nsplit = (a.Tk + a.chunk - 1) / a.chunk;
        const long long blocks = (long long)a.B * a.Hkv * a.nrb;
        if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
        hipLaunchKernelGGL((decode_fused_kernel<T, D, NH>), dim3((unsigned)blocks), dim3(64 * a.nsplit), 0, stream, a);
        return hipGetLastError();
    }
    const long long items = (long long)a.B * a.Hkv * a.nrb * a.nsplit;
    const long long blocks = (items + kWavesPerWG - 1) / kWavesPerWG;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_partial_kernel<T, D, NH>), dim3((unsigned)blocks), dim3(64 * kWavesPerWG), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    const long long rows = (long long)a.B * a.Hkv * a.R;
    if (rows > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)rows), dim3(64), 0, stream, a);
    return hipGetLastError();
}

// bf16 at head_dim 64 and 128 runs the 16-row products; when no row block has more than 16
// rows (R <= 16, the usual decode shapes), kernels without a second half keep fewer registers.
template <typename T, int D>
hipError_t launch_decode_t(DecArgs a, hipStream_t stream) {
    if constexpr (kDec16<T, D>) {
        if (a.R <= 16) return launch_decode_nh<T, D, 1>(a, stream);
    }
    return launch_decode_nh<T, D, 2>(a, stream);
}

}  // namespace

size_t decode_workspace_bytes(int B, int Tq, int Tk, int Hq, int Hkv, int D) {
    const DecPlan p = plan_decode(B, Tq, Tk, Hq, Hkv);
    if (p.nsplit == 1) return 256;
    const size_t items = (size_t)B * Hkv * p.nrb * p.nsplit;
    const size_t ob = (items * 32 * D * sizeof(float) + 255) & ~(size_t)255;
    const size_t lb = (items * 32 * sizeof(float) + 255) & ~(size_t)255;
    return ob + lb;
}

hipError_t launch_attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                              void* workspace, int B, int Tq, int Tk, int Hq, int Hkv, int D,
                              float scale, IoType dt, hipStream_t stream) {
    const DecPlan p = plan_decode(B, Tq, Tk, Hq, Hkv);
    DecArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    const size_t items = (size_t)B * Hkv * p.nrb * p.nsplit;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          ((items * 32 * D * sizeof(float) + 255) & ~(size_t)255));
    a.B = B;
    a.Tq = Tq;
    a.Tk = Tk;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.g = Hq / Hkv;
    a.R = a.g * Tq;
    a.nrb = p.nrb;
    a.nsplit = p.nsplit;
    a.chunk = p.chunk;
    a.sl2 = scale * kLog2e;
    if (dt == kF32) {
        if (D == 32) return launch_decode_t<float, 32>(a, stream);
        if (D == 64) return launch_decode_t<float, 64>(a, stream);
        return launch_decode_t<float, 128>(a, stream);
    }
    if (D == 32) return launch_decode_t<bf16, 32>(a, stream);
    if (D == 64) return launch_decode_t<bf16, 64>(a, stream);
    return launch_decode_t<bf16, 128>(a, stream);
}

}  // namespace ea
