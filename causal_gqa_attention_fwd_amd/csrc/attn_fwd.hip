// attn_fwd.hip -- causal GQA attention forward on gfx950 (attn_fwd).
//
// What it computes: for each query row t of each query head, O_t = softmax(scale * q_t K^T
// over keys s <= t) V and LSE_t ("Tiny Hackable CUDA Language Model Implementation",
// section 1: causal scaled dot-product attention; "Show HN: NanoEuler", section 2: query
// heads share K/V heads).  As the NanoEuler engine does ("Show HN: NanoEuler", section 4;
// the blog's "Tiled FlashAttention" section), keys are consumed tile by tile with an online
// softmax (running max, running sum, rescale of the partial output), so no T x T matrix
// exists anywhere.
//
// gfx950 design:
//  * One workgroup = one query tile of one batch and the G heads of one K/V head group
//    (G * WPH waves, WPH waves per head).  Each K/V tile is read from HBM once into LDS and
//    shared by every head of the group.
//  * Each wave owns 32*QB query rows of one head: their Q fragments, output accumulator and
//    softmax state stay in registers.  Scores are formed transposed, S^T = K Q^T, on 32x32
//    MFMA tiles: a lane then holds one query column and 16 keys per tile, so the row max and
//    row sum are in-lane reductions plus one exchange between the two lane halves.
//    O^T += V^T P^T takes the score registers directly as its B operand.
//  * K and V tiles are staged row-major in LDS.  K feeds S^T = K Q^T with plain 16-byte
//    reads of 16 consecutive rows (16 bytes of row padding keep them on distinct banks); V^T,
//    the A operand of O^T, is read with gfx950's transposing LDS read (ds_read_b64_tr_b16),
//    so no transposed copy is ever written, and V rows are padded to a stride of 16 dwords
//    modulo the 64 banks, which keeps the 4 rows of each transposing read on distinct banks.  Two LDS buffers: tile j+1 is committed from
//    registers while tile j is computed, and tile j+2 is in flight from HBM; one barrier
//    per tile.
//  * The online softmax forms every tile's row max but raises the running max m (and
//    rescales O and l) only when a row's max grows by more than 2^8: P is then at most 2^8,
//    well inside fp32 and bf16 range, and the result is exact either way.  Most tiles skip
//    the rescale of the output accumulator.  (Taking P against a stale m and forming the max
//    only where a tile's sum overflows a bound was measured too: on inputs whose logits jump,
//    such as a workload with a few large key rows, its second pass over the tile costs more
//    than the max it saves.)
//  * Small problems (too few query blocks to fill the chip twice) split each query block's
//    key range over KSPL = 2 waves that take alternate K/V tiles; their (max, sum, output)
//    partials merge exactly through LDS at the end.  This halves the serial work of the
//    longest (last) query blocks, which set the kernel's duration under causal masking.
//  * Tiles strictly above the diagonal are never visited; the causal mask is evaluated only
//    on the one tile that crosses a wave's diagonal.  The launch order puts the longest
//    (latest) query tiles first; workgroups of one K/V head land on the same XCD.
#include <cmath>
#include <type_traits>

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
    int causal;  // 1: key s visible to query t iff s <= t; 0: every key visible
    float sl2;  // scale * log2(e)
    const float* qtab;  // if set: q is pre-RoPE; (cos, sin) per (position, pair) rotate it
    void* q_r;          // ... and the rotated rows are written here
};

constexpr float kRescaleThreshold = 8.0f;  // log2 of the largest P taken against a stale max

template <typename T, int D, int QB, int BN, int NW, int KSPL>
struct FwdCfg {
    static constexpr int KPL = Mfma<T>::KPL;
    static constexpr int NS = D / (2 * KPL);  // MFMA steps over head_dim
    static constexpr int NKB = BN / 32;       // 32-key blocks per tile
    static constexpr int NDB = D / 32;        // 32-row blocks of head_dim
    static constexpr int PS = 16 / KPL;       // MFMA steps per 32-key block
    static constexpr int EPC = 16 / sizeof(T);
    static constexpr int CPR = D / EPC;       // 16-byte chunks per K/V row
    // Row strides (elements) of the K and V tiles.  K is read as 16-byte pieces of 16
    // consecutive rows: a stride of D + 16 bytes puts those rows on distinct banks.  V is read
    // only by the transposing read, 4 rows x 64 bytes per 32 lanes: for bf16 a stride that is
    // 16 dwords modulo the 64 banks puts those 4 rows on distinct banks.
    static constexpr int KSTR = D + EPC;
    static constexpr int VSTR = sizeof(T) == 2 ? (D == 32 ? 32 : D + 32) : D + EPC;
    static_assert(sizeof(T) != 2 || ((VSTR / 2) % 64 == 16 || (VSTR / 2) % 64 == 48), "V stride");
    static constexpr int NT = 64 * NW;
    static constexpr int NCH = (KSPL * BN * CPR + NT - 1) / NT;  // chunks per thread per tensor
    static constexpr int QW = 32 * QB;
    static constexpr int KBUF = BN * KSTR;
    static constexpr int VBUF = BN * VSTR;
    static constexpr int NBUF = 2 * KSPL;     // double buffer per key split
    // Merge area for the key splits' partials (reuses the K tiles after the loop).
    static constexpr int MERGE_FLOATS = (NW / KSPL) * (16 * (D / 32) * QB + 2 * QB) * 64;
    static constexpr int LDS_ELEMS = NBUF * (KBUF + VBUF);
    static_assert(KSPL == 1 || MERGE_FLOATS * 4 <= (int)(LDS_ELEMS * sizeof(T)), "merge area");
};

template <typename T, int D, int QB, int BN, int NW, int KSPL>
// bf16 head_dim 128 with four waves is held to 256 registers (one staging register set), so
// that two workgroups share a CU and each SIMD runs two waves instead of one.
__global__ __launch_bounds__(64 * NW, (sizeof(T) == 2 && D >= 128 && NW == 4) ? 2 : 1) void attn_fwd_kernel(FwdArgs a) {
    using C = FwdCfg<T, D, QB, BN, NW, KSPL>;
    using M = Mfma<T>;
    using frag = typename M::frag;
    constexpr int KPL = C::KPL;

    // K tiles, then V tiles (one array: the key-split merge reuses both).
    __shared__ __attribute__((aligned(16))) T KVs[C::LDS_ELEMS];
    T* const Ks = KVs;
    T* const Vs = KVs + C::NBUF * C::KBUF;

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
    const int nws = a.G * a.WPH;      // waves per key split
    const int ks = w / nws;           // this wave's key split: tiles j with j % KSPL == ks
    const int slot = w % nws;
    const int hs = slot / a.WPH;
    const int sub = slot % a.WPH;
    const int head = kvh * g + hc * a.G + hs;
    const int q0 = tile * BM + sub * C::QW;
    const bool active = q0 < a.T;
    const int qlast = min(q0 + C::QW, a.T) - 1;
    const int wg_last = min(tile * BM + BM, a.T) - 1;
    const int jmax = (a.causal ? wg_last : a.T - 1) / BN;

    const T* __restrict__ qp = static_cast<const T*>(a.q);
    const T* __restrict__ kp = static_cast<const T*>(a.k);
    const T* __restrict__ vp = static_cast<const T*>(a.v);
    const long long kv_row0 = (long long)b * a.T;  // row index of key 0 of this batch

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
                for (int e = 0; e < C::EPC / KPL; ++e)
                    qf[qb][c * (C::EPC / KPL) + e] = reinterpret_cast<const frag*>(&v.raw)[e];
            }
        } else {
#pragma unroll
            for (int s = 0; s < C::NS; ++s) qf[qb][s] = frag{};
        }
    }

    // Staging of one step (KSPL consecutive K/V tiles): HBM -> registers (fetch) -> LDS
    // (commit), 16-byte chunks, consecutive lanes on consecutive chunks of a row, through NSET
    // register sets (two for bf16 with 32-row waves up to head_dim 64, so that each step's
    // loads have two steps to land; 64-row waves, head_dim 128 and the twelve-wave key split,
    // held to 168 registers, have none to spare).
    constexpr int NSET = (sizeof(T) == 2 && QB == 1 && D < 128 && !(KSPL == 2 && NW == 12)) ? 2 : 1;
    struct Stg {
        Vec16<T> k[C::NCH], v[C::NCH];
    };
    Stg sa;
    [[maybe_unused]] Stg sb;
    // Chunk n of this thread: key row tkey (0 .. KSPL * BN - 1 within a step), 16-byte part
    // tpart; its byte offset from the step's first key row is fixed for the whole loop (when
    // it fits 32 bits), so a step's loads are a wave-uniform base plus that offset.
    const long long row_bytes = (long long)a.Hkv * D * sizeof(T);
    // (Head_dim 128 and 64-row waves keep the per-chunk index arithmetic: their register
    // budgets have no room for the offsets.)
    constexpr bool HOIST = D < 128 && QB == 1;
    const bool off32 = HOIST && (long long)KSPL * BN * row_bytes < (1LL << 31);
    // (key row, part) of chunk n; cheap to form again from the thread index where needed.
    auto chunk_key = [&](int n) { const int u = tid + n * C::NT; return (u / (BN * C::CPR)) * BN + (u % (BN * C::CPR)) / C::CPR; };
    auto chunk_part = [&](int n) { return (tid + n * C::NT) % C::CPR; };
    uint32_t toff[C::NCH];
#pragma unroll
    for (int n = 0; n < C::NCH; ++n) toff[n] = HOIST ? (uint32_t)(chunk_key(n) * row_bytes + chunk_part(n) * 16) : 0u;
    auto fetch = [&](Stg& sg, int step) {
        Vec16<T>* kreg = sg.k;
        Vec16<T>* vreg = sg.v;
        const int s0 = step * KSPL * BN;  // first key of the step
        if (HOIST && off32 && s0 + KSPL * BN <= a.T) {
            const long long base = ((kv_row0 + s0) * a.Hkv + kvh) * D;
            const char* kb = reinterpret_cast<const char*>(kp + base);
            const char* vb = reinterpret_cast<const char*>(vp + base);
#pragma unroll
            for (int n = 0; n < C::NCH; ++n) {
                if (tid + n * C::NT < KSPL * BN * C::CPR) {
                    kreg[n] = ld16(reinterpret_cast<const T*>(kb + toff[n]));
                    vreg[n] = ld16(reinterpret_cast<const T*>(vb + toff[n]));
                }
            }
        } else {
#pragma unroll
            for (int n = 0; n < C::NCH; ++n) {
                if (tid + n * C::NT < KSPL * BN * C::CPR) {
                    // Keys past the end (or of a tile past jmax, never computed) load a real
                    // row instead: they only occur in a masked tile (the diagonal, or the ragged
                    // last tile without the causal mask).
                    const int s = min(s0 + chunk_key(n), a.T - 1);
                    const long long off = ((kv_row0 + s) * a.Hkv + kvh) * D + chunk_part(n) * C::EPC;
                    kreg[n] = ld16(kp + off);
                    vreg[n] = ld16(vp + off);
                }
            }
        }
    };
    auto commit = [&](const Stg& sg, int buf) {
        const Vec16<T>* kreg = sg.k;
        const Vec16<T>* vreg = sg.v;
#pragma unroll
        for (int n = 0; n < C::NCH; ++n) {
            if (tid + n * C::NT < KSPL * BN * C::CPR) {
                const int tk = chunk_key(n), sp = tk / BN, key = tk % BN, part = chunk_part(n);
                st16(&Ks[(sp * 2 + buf) * C::KBUF + key * C::KSTR + part * C::EPC], kreg[n]);
                st16(&Vs[(sp * 2 + buf) * C::VBUF + key * C::VSTR + part * C::EPC], vreg[n]);
            }
        }
    };

    float mrun[QB], l[QB];
    f32x16 oacc[QB][C::NDB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        mrun[qb] = -INFINITY;
        l[qb] = 0.0f;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) oacc[qb][db] = zero_acc();
    }

    // One tile: S^T = K Q^T, online softmax, O^T += V^T P^T.
    auto scores = [&](const T* kb, int j, f32x16 (&sacc)[QB][C::NKB], auto masked) {
        constexpr bool MASK = decltype(masked)::value;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb2 = 0; kb2 < C::NKB; ++kb2) sacc[qb][kb2] = zero_acc();
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
#pragma unroll
            for (int kb2 = 0; kb2 < C::NKB; ++kb2) {
                const frag af = load_frag<T>(&kb[(kb2 * 32 + l32) * C::KSTR + half * (D / 2) + s * KPL]);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[qb][kb2] = M::mma(af, qf[qb][s], sacc[qb][kb2]);
            }
        }
        if constexpr (MASK) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                // Last key this lane's query sees.
                const int lim = a.causal ? q0 + qb * 32 + l32 : a.T - 1;
#pragma unroll
                for (int kb2 = 0; kb2 < C::NKB; ++kb2)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (j * BN + kb2 * 32 + acc_row(r, half) > lim) sacc[qb][kb2][r] = -INFINITY;
            }
        }
    };
    // P = exp2(S scale log2(e) - m) in place; returns the row sum of the tile (both halves of
    // the row, in both lanes), accumulated as four independent partial sums.
    auto exp_sum = [&](f32x16 (&sv)[C::NKB], float m) {
        float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb2 = 0; kb2 < C::NKB; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(sv[kb2][r] * a.sl2 - m);
                sv[kb2][r] = p;
                ps[r & 3] += p;
            }
        return half_sum((ps[0] + ps[1]) + (ps[2] + ps[3]));
    };
    // Row max of a tile (both halves of the row), in log2 units.
    auto tile_max = [&](const f32x16 (&sv)[C::NKB]) {
        float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int kb2 = 0; kb2 < C::NKB; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) m4[r & 3] = fmaxf(m4[r & 3], sv[kb2][r]);
        return half_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))) * a.sl2;
    };
    // slot = 2 * (key split) + buffer.
    auto compute = [&](int j, int slot, auto masked) {
        const T* kb = Ks + slot * C::KBUF;
        const T* vb = Vs + slot * C::VBUF;
        f32x16 sacc[QB][C::NKB];
        scores(kb, j, sacc, masked);
        float rs[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float mx = tile_max(sacc[qb]);
            const bool grow = mx > mrun[qb] + kRescaleThreshold;
            if (__builtin_expect(__any(grow), 0)) {
                const float mnew = grow ? mx : mrun[qb];
                const float alpha = __builtin_amdgcn_exp2f(mrun[qb] - mnew);  // 0 on the first tile
                l[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
                mrun[qb] = mnew;
            }
            rs[qb] = exp_sum(sacc[qb], mrun[qb]);
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) l[qb] += rs[qb];
#pragma unroll
        for (int kb2 = 0; kb2 < C::NKB; ++kb2) {
#pragma unroll
            for (int ps = 0; ps < C::PS; ++ps) {
                frag pf[QB];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) pf[qb] = acc_to_frag<T>(sacc[qb][kb2], ps * KPL);
#pragma unroll
                for (int db = 0; db < C::NDB; ++db) {
                    const frag vf = load_rows_frag<T>(vb, C::VSTR, kb2 * 32, ps, db * 32);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = M::mma(vf, pf[qb], oacc[qb][db]);
                }
            }
        }
    };

    const int nsteps = jmax / KSPL + 1;
    // Step s sits in register set s % NSET until it is committed at the start of step s - 1;
    // the set is then refilled with step s + NSET.
    fetch(sa, 0);
    if (a.qtab != nullptr) {
        // Queries given before RoPE: rotate each chunk's pairs (2p, 2p + 1) at its position with
        // the (cos, sin) table and rope_apply's fp32 arithmetic, while the first K/V tile is in
        // flight; the first key split writes the rotated rows out.
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int t = q0 + qb * 32 + l32;
            if (!active || t >= a.T) continue;
            const long long roff = (((long long)b * a.T + t) * a.Hq + head) * D + half * (D / 2);
#pragma unroll
            for (int c = 0; c < (D / 2) / C::EPC; ++c) {
                Vec16<T> v;
#pragma unroll
                for (int e = 0; e < C::EPC / KPL; ++e)
                    reinterpret_cast<frag*>(&v.raw)[e] = qf[qb][c * (C::EPC / KPL) + e];
                const float* tab = a.qtab + ((long long)t * (D / 2) + (half * (D / 2) + c * C::EPC) / 2) * 2;
#pragma unroll
                for (int p = 0; p < C::EPC / 2; ++p) {
                    float y0, y1;
                    rope_rotate(to_f32(v.get(2 * p)), to_f32(v.get(2 * p + 1)), tab[2 * p], tab[2 * p + 1], &y0, &y1);
                    v.set(2 * p, from_f32<T>(y0));
                    v.set(2 * p + 1, from_f32<T>(y1));
                }
#pragma unroll
                for (int e = 0; e < C::EPC / KPL; ++e)
                    qf[qb][c * (C::EPC / KPL) + e] = reinterpret_cast<const frag*>(&v.raw)[e];
                if (ks == 0) st16(static_cast<T*>(a.q_r) + roff + c * C::EPC, v);
            }
        }
    }
    commit(sa, 0);
    if constexpr (NSET == 2) {
        if (nsteps > 1) fetch(sb, 1);
        if (nsteps > 2) fetch(sa, 2);
    } else {
        if (nsteps > 1) fetch(sa, 1);
    }
    // Causal: the diagonal of this wave lies in tile q0 / BN; earlier tiles need no mask.
    // Otherwise only a ragged last tile (keys past the end) is masked.
    const int jfirst_masked = a.causal ? q0 / BN : ((a.T % BN) ? (a.T - 1) / BN : INT_MAX);
    auto step = [&](int st, Stg& nxt) {
        __syncthreads();  // step st visible in buffer st&1; step st-1's buffer is free
        if (st + 1 < nsteps) {
            commit(nxt, (st + 1) & 1);
            if (st + 1 + NSET < nsteps) fetch(nxt, st + 1 + NSET);
        }
        const int j = st * KSPL + ks;
        if (!active || j > jmax || (a.causal && j * BN > qlast)) return;
        if (j >= jfirst_masked)
            compute(j, ks * 2 + (st & 1), std::true_type{});
        else
            compute(j, ks * 2 + (st & 1), std::false_type{});
    };
    if constexpr (NSET == 2) {
        for (int st = 0; st < nsteps; st += 2) {
            step(st, sb);
            if (st + 1 < nsteps) step(st + 1, sa);
        }
    } else {
        for (int st = 0; st < nsteps; ++st) step(st, sa);
    }

    // Output staging region of this wave (16 rows of O at a time, row stride OS): the merge
    // slot of the key-split path, else a slice of the K/V area once every wave is done with it.
    constexpr int OS = D + C::EPC;
    T* ostage;
    if constexpr (KSPL == 1) {
        __syncthreads();  // every wave is done with the K/V tiles
        ostage = Ks + (size_t)w * 16 * OS;
    }

    if constexpr (KSPL == 2) {
        // Merge the two key splits: m = max(m0, m1), a_i = 2^(m_i - m),
        // l = a0 l0 + a1 l1, O = a0 O0 + a1 O1 (per lane; l already holds the whole row).
        constexpr int PER = 16 * C::NDB * QB + 2 * QB;
        float* mb = reinterpret_cast<float*>(Ks) + (size_t)slot * PER * 64;
        ostage = reinterpret_cast<T*>(mb);
        __syncthreads();  // every wave is done with the K/V tiles
        if (ks == 1 && active) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
                for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mb[((qb * C::NDB + db) * 16 + r) * 64 + lane] = oacc[qb][db][r];
                mb[(16 * C::NDB * QB + 2 * qb) * 64 + lane] = mrun[qb];
                mb[(16 * C::NDB * QB + 2 * qb + 1) * 64 + lane] = l[qb];
            }
        }
        __syncthreads();
        if (ks == 1) return;
        if (active) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float m1 = mb[(16 * C::NDB * QB + 2 * qb) * 64 + lane];
                const float l1 = mb[(16 * C::NDB * QB + 2 * qb + 1) * 64 + lane];
                const float m = fmaxf(mrun[qb], m1);  // finite: split 0 always has tile 0
                const float a0 = __builtin_amdgcn_exp2f(mrun[qb] - m);
                const float a1 = __builtin_amdgcn_exp2f(m1 - m);  // 0 when split 1 saw no tile
                l[qb] = l[qb] * a0 + l1 * a1;
                mrun[qb] = m;
#pragma unroll
                for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        oacc[qb][db][r] = oacc[qb][db][r] * a0 + mb[((qb * C::NDB + db) * 16 + r) * 64 + lane] * a1;
            }
        }
    }

    if (!active) return;
    // O leaves through LDS: the lanes of 16 rows write their row (normalised, in the I/O
    // dtype) to the staging region, then the wave stores whole 16-byte row segments, eight
    // lanes per 128-byte row (the accumulator layout alone would give 8-byte pieces).
    T* __restrict__ op = static_cast<T*>(a.o);
    constexpr int CPRo = D / C::EPC;
    auto wave_sync = [&]() {  // this wave's LDS accesses before / after, in order
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int tq = q0 + qb * 32 + l32;
        const float lt = l[qb];  // both halves of the row already summed
        const float inv = 1.0f / lt;
        if (half == 0 && tq < a.T)
            a.lse[((long long)b * a.Hq + head) * a.T + tq] = (mrun[qb] + __log2f(lt)) * kLn2;
#pragma unroll
        for (int hr = 0; hr < 2; ++hr) {
            wave_sync();  // the previous round's reads (or the merge's) are done
            if ((l32 >> 4) == hr) {
                T* srow = ostage + (l32 & 15) * OS;
#pragma unroll
                for (int db = 0; db < C::NDB; ++db)
#pragma unroll
                    for (int a4 = 0; a4 < 4; ++a4) {
                        const int d0 = db * 32 + 8 * a4 + 4 * half;
                        if constexpr (sizeof(T) == 2) {
                            bf16x4 v;
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] = (bf16)(oacc[qb][db][4 * a4 + e] * inv);
                            *reinterpret_cast<bf16x4*>(srow + d0) = v;
                        } else {
                            f32x4 v;
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] = oacc[qb][db][4 * a4 + e] * inv;
                            *reinterpret_cast<f32x4*>(srow + d0) = v;
                        }
                    }
            }
            wave_sync();
            for (int c = lane; c < 16 * CPRo; c += 64) {
                const int row = c / CPRo, part = c % CPRo;
                const int t = q0 + qb * 32 + hr * 16 + row;
                if (t < a.T)
                    st16(op + (((long long)b * a.T + t) * a.Hq + head) * D + part * C::EPC,
                         ld16(ostage + row * OS + part * C::EPC));
            }
        }
    }
}

template <typename T, int D, int QB, int BN, int NW, int KSPL>
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
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, QB, BN, NW, KSPL>), dim3((unsigned)blocks),
                       dim3(64 * NW), 0, stream, a);
    return hipGetLastError();
}

// Heads per workgroup: the largest divisor G of g that is at most four.
// * head_dim <= 64, bf16, few query blocks (B * Hq * T / 32 <= 2048, i.e. fewer than two
//   waves per SIMD): two 32-row blocks per head (one for G = 4) and two key splits, so that
//   three heads make twelve waves, three per SIMD.
// * head_dim <= 64 otherwise: four waves per head when G <= 2 or (bf16) G = 3, else two; no
//   key split; for bf16 head_dim 64 with 6 or 8 waves, each wave then owns 64 query rows
//   (QB = 2) if 512+ workgroups remain.
// * head_dim 128: one wave per head (4/G when G <= 2), no key split (LDS and registers).
// Every shape gives 4, 6, 8 or 12 waves (3 or 4 for head_dim 128).
template <typename T, int D>
void pick_fwd_shape(const FwdArgs& a, int* G, int* WPH, int* KSPL) {
    const int g = a.Hq / a.Hkv;
    int G_ = 1;
    for (int c = 4; c >= 1; --c)
        if (g % c == 0) {
            G_ = c;
            break;
        }
    *G = G_;
    const long long qblocks = (long long)a.B * a.Hq * ((a.T + 31) / 32);
    if (D >= 128) {
        *WPH = (G_ >= 3) ? 1 : 4 / G_;
        *KSPL = 1;
    } else if (sizeof(T) == 2 && qblocks <= 2048) {
        *WPH = (G_ <= 3) ? 2 : 1;
        *KSPL = 2;
    } else {
        *WPH = (G_ <= 2 || (G_ == 3 && sizeof(T) == 2)) ? 4 : 2;
        *KSPL = 1;
    }
}

template <typename T, int D>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
    int G, WPH, KSPL;
    pick_fwd_shape<T, D>(a, &G, &WPH, &KSPL);
    constexpr int QB = 1;
    constexpr int BN = 64;
    const int nw = G * WPH * KSPL;
    if constexpr (D >= 128) {
        if (nw == 3) return launch_fwd_cfg<T, D, QB, BN, 3, 1>(a, G, WPH, stream);
        return launch_fwd_cfg<T, D, QB, BN, 4, 1>(a, G, WPH, stream);
    } else {
        if constexpr (sizeof(T) == 2) {
            if (KSPL == 2) {
                if (nw == 12) return launch_fwd_cfg<T, D, QB, BN, 12, 2>(a, G, WPH, stream);
                if (nw == 6) return launch_fwd_cfg<T, D, QB, BN, 6, 2>(a, G, WPH, stream);
                if (nw == 4) return launch_fwd_cfg<T, D, QB, BN, 4, 2>(a, G, WPH, stream);
                return launch_fwd_cfg<T, D, QB, BN, 8, 2>(a, G, WPH, stream);
            }
        }
        // Without a key split, bf16 head_dim-64 waves own two 32-row query blocks (QB = 2)
        // when that still leaves at least two workgroups per CU: every K / V fragment read
        // from LDS then feeds two matrix-core instructions.  Three heads per workgroup take
        // twelve 32-row waves instead (three per SIMD: six waves would leave two SIMDs with
        // one wave each), which measured faster than six 64-row waves.
        if constexpr (sizeof(T) == 2) {
            if (nw == 12) return launch_fwd_cfg<T, D, QB, BN, 12, 1>(a, G, WPH, stream);
        }
        if constexpr (sizeof(T) == 2 && D == 64) {
            const long long wgs = (long long)a.B * a.Hkv * ((a.Hq / a.Hkv) / G) *
                                  ((a.T + WPH * 64 - 1) / (WPH * 64));
            if (wgs >= 512) {
                if (nw == 6) return launch_fwd_cfg<T, D, 2, BN, 6, 1>(a, G, WPH, stream);
                if (nw == 4) return launch_fwd_cfg<T, D, 2, BN, 4, 1>(a, G, WPH, stream);
                return launch_fwd_cfg<T, D, 2, BN, 8, 1>(a, G, WPH, stream);
            }
        }
        if (nw == 6) return launch_fwd_cfg<T, D, QB, BN, 6, 1>(a, G, WPH, stream);
        if (nw == 4) return launch_fwd_cfg<T, D, QB, BN, 4, 1>(a, G, WPH, stream);
        return launch_fwd_cfg<T, D, QB, BN, 8, 1>(a, G, WPH, stream);
    }
}

}  // namespace

bool fwd_splits_keys(int B, int T, int Hq, int Hkv, int D, IoType dt) {
    FwdArgs a{};
    a.B = B;
    a.T = T;
    a.Hq = Hq;
    a.Hkv = Hkv;
    int G, WPH, KSPL;
    if (dt == kF32) {
        if (D == 32) pick_fwd_shape<float, 32>(a, &G, &WPH, &KSPL);
        else if (D == 64) pick_fwd_shape<float, 64>(a, &G, &WPH, &KSPL);
        else pick_fwd_shape<float, 128>(a, &G, &WPH, &KSPL);
    } else {
        if (D == 32) pick_fwd_shape<bf16, 32>(a, &G, &WPH, &KSPL);
        else if (D == 64) pick_fwd_shape<bf16, 64>(a, &G, &WPH, &KSPL);
        else pick_fwd_shape<bf16, 128>(a, &G, &WPH, &KSPL);
    }
    return KSPL > 1;
}

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int T, int Hq, int Hkv, int D, float scale, IoType dt,
                           bool causal, hipStream_t stream, const float* qtab, void* q_r) {
    FwdArgs a{};
    a.causal = causal ? 1 : 0;
    a.qtab = qtab;
    a.q_r = q_r;
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
