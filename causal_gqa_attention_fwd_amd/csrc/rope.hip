// rope.hip -- rotary position embedding on gfx950 (rope_apply).
//
// The pages apply rotary embeddings to queries and keys ("Show HN: NanoEuler", section 2;
// "Tiny Hackable CUDA Language Model Implementation", section 1) without a formula; this
// kernel implements the adjacent-pair reading: pair (2i, 2i+1) of row (b, t, h) turns by
// phi = (pos0 + t) * theta_i, theta_i = base^(-2i/D), and by -phi for the inverse.
//
// Work is HBM-bound (one read and one write of x).  Two tensors that share (B, T, D) --
// Q and K, or dQ and dK -- can be rotated in one launch.  Each thread owns one 16-byte chunk of
// a row (8 bf16 or 4 fp32 elements) for HPT heads of the same position: the angles of its
// pairs are formed once, in float64 (product and reduction modulo 2*pi), and reused for
// every head.  sin/cos of the reduced angle, |r| <= pi, are float32.  Consecutive lanes
// take consecutive chunks of a row, so each wave reads whole 128-byte rows.  Head dims that
// are not a whole number of chunks (any other even D up to 256) take one thread per pair.
#include <cmath>

#include "ea_common.h"
#include "ea_kernels.h"

namespace ea {
namespace {

constexpr int kHeadsPerThread = 4;

// Up to two tensors [B, T, H_k, D] in one launch (Q and K, or dQ and dK): units
// [0, n0) belong to tensor 0, [n0, n0 + n1) to tensor 1.
template <typename T>
struct RopeJob {
    const T* x[2];
    T* y[2];
    int H[2];
    long long n0, ntot;
    float* tab;  // if set: (cos, sin) of every (position, pair), [T][D/2] float2 (forward angles)
};

// I: unsigned index type of the unit decomposition (32-bit whenever the units fit).
template <typename T, typename I>
__global__ __launch_bounds__(256) void rope_kernel(RopeJob<T> job, int seq, int D, int pos0,
                                                   int inverse, RopeFreq f) {
    constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
    constexpr int PPC = EPC / 2;         // pairs per chunk
    I u = (I)blockIdx.x * (I)blockDim.x + (I)threadIdx.x;
    if (u >= (I)job.ntot) return;
    // The tensor is chosen by selects between the two argument sets (loaded as scalars), not by
    // indexing them with a per-lane value, which would load the pointers per lane and make
    // every data load wait for that load first.
    const int which = u < (I)job.n0 ? 0 : 1;
    if (which) u -= (I)job.n0;
    const T* x = which ? job.x[1] : job.x[0];
    T* y = which ? job.y[1] : job.y[0];
    const int H = which ? job.H[1] : job.H[0];
    const I cpr = (I)(D / EPC);  // chunks per row
    const I nhb = (I)((H + kHeadsPerThread - 1) / kHeadsPerThread);
    const int c = (int)(u % cpr);
    const I rest = u / cpr;
    const int hb = (int)(rest % nhb);
    const long long bt = (long long)(rest / nhb);
    const int t = (int)(bt % seq);
    const double pos = (double)pos0 + (double)t;
    const int h0 = hb * kHeadsPerThread;
    const int nh = min(H - h0, kHeadsPerThread);
    const long long off0 = (bt * H + h0) * (long long)D + (long long)c * EPC;

    // Every load of this thread is issued before any store: its chunks are disjoint from
    // every other thread's, so this is also correct in place, and the loads overlap the
    // angle computation instead of waiting behind each other's stores.
    Vec16<T> v[kHeadsPerThread];
#pragma unroll
    for (int k = 0; k < kHeadsPerThread; ++k)
        if (k < nh) v[k] = ld16(x + off0 + (long long)k * D);

    float cs[PPC], sn[PPC];
#pragma unroll
    for (int p = 0; p < PPC; ++p) {
        float s, co;
        rope_cos_sin(pos, f.theta[c * PPC + p], &co, &s);
        cs[p] = co;
        sn[p] = inverse ? -s : s;
    }
    // The threads of batch 0 and head block 0 of the first tensor cover every (position, chunk)
    // once: they write the table entries of their pairs.
    if (job.tab != nullptr && which == 0 && hb == 0 && bt < seq) {
#pragma unroll
        for (int p = 0; p < PPC; ++p)
            reinterpret_cast<float2*>(job.tab)[(long long)t * (D / 2) + c * PPC + p] = make_float2(cs[p], sn[p]);
    }
#pragma unroll
    for (int k = 0; k < kHeadsPerThread; ++k) {
        if (k < nh) {
            Vec16<T> w;
#pragma unroll
            for (int p = 0; p < PPC; ++p) {
                float y0, y1;
                rope_rotate(to_f32(v[k].get(2 * p)), to_f32(v[k].get(2 * p + 1)), cs[p], sn[p], &y0, &y1);
                w.set(2 * p, from_f32<T>(y0));
                w.set(2 * p + 1, from_f32<T>(y1));
            }
            st16(y + off0 + (long long)k * D, w);
        }
    }
}

// Head dims that are not a whole number of 16-byte chunks (D = 2, 6, 10, ... for bf16; D = 2,
// 6, ... for fp32): one thread per pair (2i, 2i+1) of one position, for kHeadsPerThread heads,
// with the same angle and rotation arithmetic as rope_kernel.  A pair is 4 (bf16) or 8 (fp32)
// bytes and always aligned to its size, since D is even.
template <typename T, typename I>
__global__ __launch_bounds__(256) void rope_pair_kernel(RopeJob<T> job, int seq, int D, int pos0,
                                                        int inverse, RopeFreq f) {
    I u = (I)blockIdx.x * (I)blockDim.x + (I)threadIdx.x;
    if (u >= (I)job.ntot) return;
    const int which = u < (I)job.n0 ? 0 : 1;  // selects, as in rope_kernel
    if (which) u -= (I)job.n0;
    const T* x = which ? job.x[1] : job.x[0];
    T* y = which ? job.y[1] : job.y[0];
    const int H = which ? job.H[1] : job.H[0];
    const I ppr = (I)(D / 2);  // pairs per row
    const I nhb = (I)((H + kHeadsPerThread - 1) / kHeadsPerThread);
    const int i = (int)(u % ppr);
    const I rest = u / ppr;
    const int hb = (int)(rest % nhb);
    const long long bt = (long long)(rest / nhb);
    const int t = (int)(bt % seq);
    const int h0 = hb * kHeadsPerThread;
    const int nh = min(H - h0, kHeadsPerThread);
    const long long off0 = (bt * H + h0) * (long long)D + 2LL * i;
    T v[kHeadsPerThread][2];
#pragma unroll
    for (int k = 0; k < kHeadsPerThread; ++k)
        if (k < nh) {
            v[k][0] = x[off0 + (long long)k * D];
            v[k][1] = x[off0 + (long long)k * D + 1];
        }
    float c, s;
    rope_cos_sin((double)pos0 + (double)t, f.theta[i], &c, &s);
    if (inverse) s = -s;
#pragma unroll
    for (int k = 0; k < kHeadsPerThread; ++k)
        if (k < nh) {
            float y0, y1;
            rope_rotate(to_f32(v[k][0]), to_f32(v[k][1]), c, s, &y0, &y1);
            y[off0 + (long long)k * D] = from_f32<T>(y0);
            y[off0 + (long long)k * D + 1] = from_f32<T>(y1);
        }
}

template <typename T>
hipError_t launch_rope_t(const void* x0, void* y0, int H0, const void* x1, void* y1, int H1, int B,
                         int seq, int D, double base, int pos0, int inverse, hipStream_t stream,
                         float* tab = nullptr) {
    constexpr int EPC = 16 / sizeof(T);
    RopeFreq f;
    fill_rope_freq(&f, D, base);
    RopeJob<T> job;
    job.x[0] = static_cast<const T*>(x0);
    job.y[0] = static_cast<T*>(y0);
    job.H[0] = H0;
    job.x[1] = static_cast<const T*>(x1);
    job.y[1] = static_cast<T*>(y1);
    job.H[1] = H1;
    job.tab = tab;
    // Whole 16-byte chunks per row: one thread per chunk; otherwise one thread per pair.
    const bool chunks = D % EPC == 0;
    if (!chunks && tab != nullptr) return hipErrorInvalidValue;  // the table path needs chunks
    const int per_row = chunks ? D / EPC : D / 2;
    auto units = [&](int H) {
        return H > 0 ? (long long)B * seq * ((H + kHeadsPerThread - 1) / kHeadsPerThread) * per_row : 0LL;
    };
    job.n0 = units(H0);
    job.ntot = job.n0 + units(H1);
    const int threads = 256;
    const long long blocks = (job.ntot + threads - 1) / threads;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const bool narrow = blocks * threads <= 0xffffffffLL;
    if (chunks && narrow)
        hipLaunchKernelGGL((rope_kernel<T, uint32_t>), dim3((unsigned)blocks), dim3(threads), 0, stream,
                           job, seq, D, pos0, inverse, f);
    else if (chunks)
        hipLaunchKernelGGL((rope_kernel<T, uint64_t>), dim3((unsigned)blocks), dim3(threads), 0, stream,
                           job, seq, D, pos0, inverse, f);
    else if (narrow)
        hipLaunchKernelGGL((rope_pair_kernel<T, uint32_t>), dim3((unsigned)blocks), dim3(threads), 0, stream,
                           job, seq, D, pos0, inverse, f);
    else
        hipLaunchKernelGGL((rope_pair_kernel<T, uint64_t>), dim3((unsigned)blocks), dim3(threads), 0, stream,
                           job, seq, D, pos0, inverse, f);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const void* x, void* y, int B, int T, int H, int D, IoType dt,
                       double base, int pos0, int inverse, hipStream_t stream) {
    if (dt == kF32) return launch_rope_t<float>(x, y, H, nullptr, nullptr, 0, B, T, D, base, pos0, inverse, stream);
    return launch_rope_t<bf16>(x, y, H, nullptr, nullptr, 0, B, T, D, base, pos0, inverse, stream);
}

hipError_t launch_rope_table(const void* x, void* y, int B, int T, int H, int D, IoType dt,
                             double base, int pos0, float* tab, hipStream_t stream) {
    if (dt == kF32) return launch_rope_t<float>(x, y, H, nullptr, nullptr, 0, B, T, D, base, pos0, 0, stream, tab);
    return launch_rope_t<bf16>(x, y, H, nullptr, nullptr, 0, B, T, D, base, pos0, 0, stream, tab);
}

hipError_t launch_rope_pair(const void* x0, void* y0, int H0, const void* x1, void* y1, int H1,
                            int B, int T, int D, IoType dt, double base, int pos0, int inverse,
                            hipStream_t stream) {
    if (dt == kF32) return launch_rope_t<float>(x0, y0, H0, x1, y1, H1, B, T, D, base, pos0, inverse, stream);
    return launch_rope_t<bf16>(x0, y0, H0, x1, y1, H1, B, T, D, base, pos0, inverse, stream);
}

}  // namespace ea
