// oracle.cpp -- plain, slow, double-precision CPU reference for causal grouped-query
// attention with rotary position embeddings, forward and analytic backward.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load this
// file or the library built from it; only the test-suite, the smoke check and the
// benchmark's CPU-baseline leg do.  It shares no code, header, table or helper with the
// HIP library: every formula below is written out from its definition.
//
// Sources (the web pages describing NanoEuler and a tiny CUDA language model):
//  * "Show HN: NanoEuler" (aimsg.uk), section 2 "模型组件": rotary embeddings act on
//    queries and keys; query heads share a smaller set of key/value heads (GQA).
//  * "Tiny Hackable CUDA Language Model Implementation", section 1 "架构设计": causal
//    self-attention (a position sees only itself and earlier positions), scaled
//    dot-product scores with a causal mask, rotary encoding on Q and K.
//  * "Show HN: NanoEuler", section 3 "训练管线与验证": every analytic gradient is checked
//    against central finite differences in double precision (the tests do that to
//    this file).
//  * "Show HN: NanoEuler", section 4 "硬件与性能": the CPU engine is C with libm and
//    OpenMP; this oracle follows the same recipe.
//
// Readings where the pages are silent (each is listed with its reason in the design notes):
//  * RoPE pairs adjacent elements (2i, 2i+1) with frequency theta_i = base^(-2i/D) and
//    angle (pos0 + t) * theta_i; the inverse rotates by the negated angle.
//  * Query head h reads key/value head floor(h / g), g = Hq / Hkv (contiguous groups).
//  * The causal mask keeps key s for query t iff s <= t (diagonal included).
//  * LSE is the natural-log log-sum-exp of the scaled, masked scores of one row.
//
// Layouts: Q, O, dO, dQ are [B, T, Hq, D]; K, V, dK, dV are [B, T, Hkv, D]; LSE is
// [B, Hq, T]; all row-major, D fastest, float64.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#include <omp.h>

namespace {

inline long q_index(long b, long t, long h, long d, long T, long H, long D) {
    return ((b * T + t) * H + h) * D + d;
}

}  // namespace

extern "C" {

// Number of OpenMP threads a parallel region of this library would use.
int oracle_num_threads(void) { return omp_get_max_threads(); }

// Threads for the following parallel regions (a timing aid; no effect on any result, since
// every sum in this file runs in one thread in a fixed order).
void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

// RoPE on x [B, T, H, D] -> y (y may equal x).  For every row (b, t, h) and every pair
// i in [0, D/2):  theta_i = base^(-2i/D),  phi = (pos0 + t) * theta_i  (negated when
// inverse != 0), and the pair is rotated by phi:
//     y[2i]   = x[2i] cos(phi) - x[2i+1] sin(phi)
//     y[2i+1] = x[2i] sin(phi) + x[2i+1] cos(phi)
// Returns 0, or 1 when D is odd.
int oracle_rope(const double* x, double* y, long B, long T, long H, long D, double base,
                long pos0, int inverse) {
    if (D % 2 != 0) return 1;
#pragma omp parallel for collapse(2) schedule(static)
    for (long b = 0; b < B; ++b) {
        for (long t = 0; t < T; ++t) {
            for (long i = 0; i < D / 2; ++i) {
                double theta = std::pow(base, -2.0 * (double)i / (double)D);
                double phi = (double)(pos0 + t) * theta;
                if (inverse) phi = -phi;
                double c = std::cos(phi), s = std::sin(phi);
                for (long h = 0; h < H; ++h) {
                    long base_idx = q_index(b, t, h, 2 * i, T, H, D);
                    double x0 = x[base_idx], x1 = x[base_idx + 1];
                    y[base_idx] = x0 * c - x1 * s;
                    y[base_idx + 1] = x0 * s + x1 * c;
                }
            }
        }
    }
    return 0;
}

// Causal GQA attention forward.  For every (b, h, t), with kv = floor(h / g):
//   S_ts  = scale * sum_d Q[b,t,h,d] * K[b,s,kv,d]          for s <= t only
//   M_t   = max_{s<=t} S_ts
//   Z_t   = sum_{s<=t} exp(S_ts - M_t)
//   P_ts  = exp(S_ts - M_t) / Z_t
//   O_t   = sum_{s<=t} P_ts V[b,s,kv,:]
//   LSE_t = M_t + ln Z_t
// Two passes over the whole row; there is no online rescaling here.
// Returns 0, or 1 when Hq is not a multiple of Hkv.
int oracle_attn_fwd(const double* q, const double* k, const double* v, double* o, double* lse,
                    long B, long T, long Hq, long Hkv, long D, double scale) {
    if (Hkv <= 0 || Hq % Hkv != 0) return 1;
    const long g = Hq / Hkv;
#pragma omp parallel
    {
        std::vector<double> srow(T > 0 ? T : 1);
#pragma omp for collapse(3) schedule(dynamic, 8)
        for (long b = 0; b < B; ++b) {
            for (long h = 0; h < Hq; ++h) {
                for (long t = 0; t < T; ++t) {
                    const long kv = h / g;
                    const double* qt = q + q_index(b, t, h, 0, T, Hq, D);
                    double m = -INFINITY;
                    for (long s = 0; s <= t; ++s) {
                        const double* ks = k + q_index(b, s, kv, 0, T, Hkv, D);
                        double acc = 0.0;
                        for (long d = 0; d < D; ++d) acc += qt[d] * ks[d];
                        srow[s] = scale * acc;
                        if (srow[s] > m) m = srow[s];
                    }
                    double z = 0.0;
                    for (long s = 0; s <= t; ++s) z += std::exp(srow[s] - m);
                    double* ot = o + q_index(b, t, h, 0, T, Hq, D);
                    for (long d = 0; d < D; ++d) ot[d] = 0.0;
                    for (long s = 0; s <= t; ++s) {
                        const double p = std::exp(srow[s] - m) / z;
                        const double* vs = v + q_index(b, s, kv, 0, T, Hkv, D);
                        for (long d = 0; d < D; ++d) ot[d] += p * vs[d];
                    }
                    lse[(b * Hq + h) * T + t] = m + std::log(z);
                }
            }
        }
    }
    return 0;
}

// Causal GQA attention of Tq new query rows against a cache of Tk >= Tq key/value rows
// (generation with a KV cache: "Show HN: NanoEuler", section 2 -- the multi-token prediction
// heads used for speculative decoding -- and its key points -- the interactive chat REPL).  The queries are the last Tq positions of
// the sequence, so query row i sits at absolute position (Tk - Tq) + i and, causally, sees the
// keys s <= (Tk - Tq) + i.  Per (b, h, i), kv = h / g, off = Tk - Tq:
//   S_is  = scale * sum_d Q[b,i,h,d] K[b,s,kv,d]       for s <= off + i
//   O_i   = sum_s softmax_s(S_i.) V[b,s,kv,:],  LSE_i = log sum_s exp(S_is)
// Layouts: q, o [B, Tq, Hq, D]; k, v [B, Tk, Hkv, D]; lse [B, Hq, Tq].  With Tq = Tk this is
// the causal self-attention above.  Two passes per row, as oracle_attn_fwd.
// Returns 0, 1 when Hq is not a multiple of Hkv, 2 when Tq > Tk.
int oracle_attn_fwd_kv(const double* q, const double* k, const double* v, double* o, double* lse,
                       long B, long Tq, long Tk, long Hq, long Hkv, long D, double scale) {
    if (Hkv <= 0 || Hq % Hkv != 0) return 1;
    if (Tq > Tk) return 2;
    const long g = Hq / Hkv;
    const long off = Tk - Tq;
#pragma omp parallel
    {
        std::vector<double> srow(Tk > 0 ? Tk : 1);
#pragma omp for collapse(3) schedule(dynamic, 8)
        for (long b = 0; b < B; ++b) {
            for (long h = 0; h < Hq; ++h) {
                for (long i = 0; i < Tq; ++i) {
                    const long kv = h / g;
                    const long last = off + i;  // last visible key
                    const double* qi = q + q_index(b, i, h, 0, Tq, Hq, D);
                    double m = -INFINITY;
                    for (long s = 0; s <= last; ++s) {
                        const double* ks = k + q_index(b, s, kv, 0, Tk, Hkv, D);
                        double acc = 0.0;
                        for (long d = 0; d < D; ++d) acc += qi[d] * ks[d];
                        srow[s] = scale * acc;
                        if (srow[s] > m) m = srow[s];
                    }
                    double z = 0.0;
                    for (long s = 0; s <= last; ++s) z += std::exp(srow[s] - m);
                    double* oi = o + q_index(b, i, h, 0, Tq, Hq, D);
                    for (long d = 0; d < D; ++d) oi[d] = 0.0;
                    for (long s = 0; s <= last; ++s) {
                        const double p = std::exp(srow[s] - m) / z;
                        const double* vs = v + q_index(b, s, kv, 0, Tk, Hkv, D);
                        for (long d = 0; d < D; ++d) oi[d] += p * vs[d];
                    }
                    lse[(b * Hq + h) * Tq + i] = m + std::log(z);
                }
            }
        }
    }
    return 0;
}

// Causal GQA attention backward, analytic, from the fully materialised masked softmax of
// one (b, h) at a time.  Given dO = dL/dO:
//   dP_ts = dO_t . V_s
//   D_t   = sum_{s<=t} P_ts dP_ts
//   dS_ts = P_ts (dP_ts - D_t)
//   dQ_t  = scale * sum_{s<=t} dS_ts K_s
//   dK_s  = scale * sum_{h in group} sum_{t>=s} dS_ts Q_t
//   dV_s  =         sum_{h in group} sum_{t>=s} P_ts dO_t
// dK and dV are overwritten (the group sum is formed here).  P and dS for one (b, h) are
// held as full T x T matrices (zero above the diagonal).
// Returns 0, or 1 when Hq is not a multiple of Hkv.
int oracle_attn_bwd(const double* q, const double* k, const double* v, const double* dout,
                    double* dq, double* dk, double* dv, long B, long T, long Hq, long Hkv,
                    long D, double scale) {
    if (Hkv <= 0 || Hq % Hkv != 0) return 1;
    const long g = Hq / Hkv;
    std::memset(dk, 0, sizeof(double) * (size_t)(B * T * Hkv * D));
    std::memset(dv, 0, sizeof(double) * (size_t)(B * T * Hkv * D));
    std::vector<double> P((size_t)T * (size_t)T), dS((size_t)T * (size_t)T);
    for (long b = 0; b < B; ++b) {
        for (long h = 0; h < Hq; ++h) {
            const long kv = h / g;
            // Rows: softmax, dP, D_t, dS and dQ.
#pragma omp parallel for schedule(dynamic, 8)
            for (long t = 0; t < T; ++t) {
                double* prow = P.data() + (size_t)t * T;
                double* dsrow = dS.data() + (size_t)t * T;
                const double* qt = q + q_index(b, t, h, 0, T, Hq, D);
                const double* dot = dout + q_index(b, t, h, 0, T, Hq, D);
                double m = -INFINITY;
                for (long s = 0; s < T; ++s) {
                    prow[s] = 0.0;
                    dsrow[s] = 0.0;
                }
                for (long s = 0; s <= t; ++s) {
                    const double* ks = k + q_index(b, s, kv, 0, T, Hkv, D);
                    double acc = 0.0;
                    for (long d = 0; d < D; ++d) acc += qt[d] * ks[d];
                    prow[s] = scale * acc;
                    if (prow[s] > m) m = prow[s];
                }
                double z = 0.0;
                for (long s = 0; s <= t; ++s) z += std::exp(prow[s] - m);
                for (long s = 0; s <= t; ++s) prow[s] = std::exp(prow[s] - m) / z;
                double delta = 0.0;
                for (long s = 0; s <= t; ++s) {
                    const double* vs = v + q_index(b, s, kv, 0, T, Hkv, D);
                    double acc = 0.0;
                    for (long d = 0; d < D; ++d) acc += dot[d] * vs[d];
                    dsrow[s] = acc;  // dP_ts for now
                    delta += prow[s] * acc;
                }
                for (long s = 0; s <= t; ++s) dsrow[s] = prow[s] * (dsrow[s] - delta);
                double* dqt = dq + q_index(b, t, h, 0, T, Hq, D);
                for (long d = 0; d < D; ++d) dqt[d] = 0.0;
                for (long s = 0; s <= t; ++s) {
                    const double* ks = k + q_index(b, s, kv, 0, T, Hkv, D);
                    for (long d = 0; d < D; ++d) dqt[d] += dsrow[s] * ks[d];
                }
                for (long d = 0; d < D; ++d) dqt[d] *= scale;
            }
            // Columns: this head's share of dK and dV.
#pragma omp parallel for schedule(dynamic, 8)
            for (long s = 0; s < T; ++s) {
                double* dks = dk + q_index(b, s, kv, 0, T, Hkv, D);
                double* dvs = dv + q_index(b, s, kv, 0, T, Hkv, D);
                for (long t = s; t < T; ++t) {
                    const double ds = dS[(size_t)t * T + s];
                    const double p = P[(size_t)t * T + s];
                    const double* qt = q + q_index(b, t, h, 0, T, Hq, D);
                    const double* dot = dout + q_index(b, t, h, 0, T, Hq, D);
                    for (long d = 0; d < D; ++d) {
                        dks[d] += scale * ds * qt[d];
                        dvs[d] += p * dot[d];
                    }
                }
            }
        }
    }
    return 0;
}

// Non-causal GQA attention: every query row sees every key row (the per-head attention the
// blog prints beside its tiled FlashAttention, "Tiled FlashAttention": rows of Q against all
// rows of K and V).  Per (b, h, t), kv = h / g:
//   S_ts = scale * sum_d Q[b,t,h,d] K[b,s,kv,d],  s = 0 .. T-1
//   O_t = sum_s softmax_s(S_t.) V[b,s,kv,:],  LSE_t = log sum_s exp(S_ts)
// Returns 0, or 1 when Hq is not a multiple of Hkv.
int oracle_attn_fwd_nc(const double* q, const double* k, const double* v, double* o, double* lse,
                       long B, long T, long Hq, long Hkv, long D, double scale) {
    if (Hkv <= 0 || Hq % Hkv != 0) return 1;
    const long g = Hq / Hkv;
#pragma omp parallel
    {
        std::vector<double> srow(T > 0 ? T : 1);
#pragma omp for collapse(3) schedule(dynamic, 8)
        for (long b = 0; b < B; ++b) {
            for (long h = 0; h < Hq; ++h) {
                for (long t = 0; t < T; ++t) {
                    const long kv = h / g;
                    const double* qt = q + q_index(b, t, h, 0, T, Hq, D);
                    double m = -INFINITY;
                    for (long s = 0; s < T; ++s) {
                        const double* ks = k + q_index(b, s, kv, 0, T, Hkv, D);
                        double acc = 0.0;
                        for (long d = 0; d < D; ++d) acc += qt[d] * ks[d];
                        srow[s] = scale * acc;
                        if (srow[s] > m) m = srow[s];
                    }
                    double z = 0.0;
                    for (long s = 0; s < T; ++s) z += std::exp(srow[s] - m);
                    double* ot = o + q_index(b, t, h, 0, T, Hq, D);
                    for (long d = 0; d < D; ++d) ot[d] = 0.0;
                    for (long s = 0; s < T; ++s) {
                        const double p = std::exp(srow[s] - m) / z;
                        const double* vs = v + q_index(b, s, kv, 0, T, Hkv, D);
                        for (long d = 0; d < D; ++d) ot[d] += p * vs[d];
                    }
                    lse[(b * Hq + h) * T + t] = m + std::log(z);
                }
            }
        }
    }
    return 0;
}

// Backward of the non-causal attention above, analytic from the full softmax of one (b, h):
// dP = dO V^T, D_t = sum_s P_ts dP_ts, dS = P (dP - D), dQ = scale dS K,
// dK = scale sum_{h in group} dS^T Q, dV = sum_{h in group} P^T dO (overwritten).
int oracle_attn_bwd_nc(const double* q, const double* k, const double* v, const double* dout,
                       double* dq, double* dk, double* dv, long B, long T, long Hq, long Hkv,
                       long D, double scale) {
    if (Hkv <= 0 || Hq % Hkv != 0) return 1;
    const long g = Hq / Hkv;
    std::memset(dk, 0, sizeof(double) * (size_t)(B * T * Hkv * D));
    std::memset(dv, 0, sizeof(double) * (size_t)(B * T * Hkv * D));
    std::vector<double> P((size_t)T * (size_t)T), dS((size_t)T * (size_t)T);
    for (long b = 0; b < B; ++b) {
        for (long h = 0; h < Hq; ++h) {
            const long kv = h / g;
#pragma omp parallel for schedule(dynamic, 8)
            for (long t = 0; t < T; ++t) {
                double* prow = P.data() + (size_t)t * T;
                double* dsrow = dS.data() + (size_t)t * T;
                const double* qt = q + q_index(b, t, h, 0, T, Hq, D);
                const double* dot = dout + q_index(b, t, h, 0, T, Hq, D);
                double m = -INFINITY;
                for (long s = 0; s < T; ++s) {
                    const double* ks = k + q_index(b, s, kv, 0, T, Hkv, D);
                    double acc = 0.0;
                    for (long d = 0; d < D; ++d) acc += qt[d] * ks[d];
                    prow[s] = scale * acc;
                    if (prow[s] > m) m = prow[s];
                }
                double z = 0.0;
                for (long s = 0; s < T; ++s) z += std::exp(prow[s] - m);
                for (long s = 0; s < T; ++s) prow[s] = std::exp(prow[s] - m) / z;
                double delta = 0.0;
                for (long s = 0; s < T; ++s) {
                    const double* vs = v + q_index(b, s, kv, 0, T, Hkv, D);
                    double acc = 0.0;
                    for (long d = 0; d < D; ++d) acc += dot[d] * vs[d];
                    dsrow[s] = acc;
                    delta += prow[s] * acc;
                }
                for (long s = 0; s < T; ++s) dsrow[s] = prow[s] * (dsrow[s] - delta);
                double* dqt = dq + q_index(b, t, h, 0, T, Hq, D);
                for (long d = 0; d < D; ++d) dqt[d] = 0.0;
                for (long s = 0; s < T; ++s) {
                    const double* ks = k + q_index(b, s, kv, 0, T, Hkv, D);
                    for (long d = 0; d < D; ++d) dqt[d] += dsrow[s] * ks[d];
                }
                for (long d = 0; d < D; ++d) dqt[d] *= scale;
            }
#pragma omp parallel for schedule(dynamic, 8)
            for (long s = 0; s < T; ++s) {
                double* dks = dk + q_index(b, s, kv, 0, T, Hkv, D);
                double* dvs = dv + q_index(b, s, kv, 0, T, Hkv, D);
                for (long t = 0; t < T; ++t) {
                    const double ds = dS[(size_t)t * T + s];
                    const double p = P[(size_t)t * T + s];
                    const double* qt = q + q_index(b, t, h, 0, T, Hq, D);
                    const double* dot = dout + q_index(b, t, h, 0, T, Hq, D);
                    for (long d = 0; d < D; ++d) {
                        dks[d] += scale * ds * qt[d];
                        dvs[d] += p * dot[d];
                    }
                }
            }
        }
    }
    return 0;
}

}  // extern "C"
