// rope.hip -- rotary position embedding on gfx950 (rope_apply).
//
// The pages apply rotary embeddings to queries and keys ("Show HN: NanoEuler", section 2;
// "Tiny Hackable CUDA Language Model Implementation", section 1) without a formula; this
// kernel implements the adjacent-pair reading: pair (2i, 2i+1) of row (b, t, h) turns by
// phi = (pos0 + t) * theta_i, theta_i = base^(-2i/D), and by -phi for the inverse.
//
// Work is HBM-bound (one read and one write of x).  Each thread owns one 16-byte chunk of
// a row (8 bf16 or 4 fp32 elements) for HPT heads of the same position: the angles of its
// pairs are formed once, in float64 (product and reduction modulo 2*pi), and reused for
// every head.  sin/cos of the reduced angle, |r| <= pi, are float32.  Consecutive lanes
// take consecutive chunks of a row, so each wave reads whole 128-byte rows.
#include <cmath>

#include "ea_common.h"
#include "ea_kernels.h"

namespace ea {
namespace {

struct RopeFreq {
    double theta[128];  // base^(-2i/D), i < D/2 <= 128
};

constexpr double kTwoPiHi = 6.283185307179586;       // nearest double to 2*pi
constexpr double kTwoPiLo = 2.4492935982947064e-16;  // 2*pi - kTwoPiHi
constexpr double kInvTwoPi = 0.15915494309189535;
constexpr int kHeadsPerThread = 4;

template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(const T* x, T* y, long long nunits, int seq,
                                                   int H, int D, int pos0, int inverse,
                                                   RopeFreq f) {
    constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
    constexpr int PPC = EPC / 2;         // pairs per chunk
    const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= nunits) return;
    const int cpr = D / EPC;  // chunks per row
    const int nhb = (H + kHeadsPerThread - 1) / kHeadsPerThread;
    const int c = (int)(u % cpr);
    const long long rest = u / cpr;
    const int hb = (int)(rest % nhb);
    const long long bt = rest / nhb;
    const int t = (int)(bt % seq);
    const double pos = (double)pos0 + (double)t;

    float cs[PPC], sn[PPC];
#pragma unroll
    for (int p = 0; p < PPC; ++p) {
        const double phi = pos * f.theta[c * PPC + p];
        const double n = rint(phi * kInvTwoPi);
        double r = fma(-n, kTwoPiHi, phi);
        r = fma(-n, kTwoPiLo, r);
        float s, co;
        sincosf((float)r, &s, &co);
        cs[p] = co;
        sn[p] = inverse ? -s : s;
    }
    const int h_end = min(H, (hb + 1) * kHeadsPerThread);
    for (int h = hb * kHeadsPerThread; h < h_end; ++h) {
        const long long off = (bt * H + h) * (long long)D + (long long)c * EPC;
        Vec16<T> v = ld16(x + off);
        Vec16<T> w;
#pragma unroll
        for (int p = 0; p < PPC; ++p) {
            const float x0 = to_f32(v.get(2 * p));
            const float x1 = to_f32(v.get(2 * p + 1));
            w.set(2 * p, from_f32<T>(x0 * cs[p] - x1 * sn[p]));
            w.set(2 * p + 1, from_f32<T>(x0 * sn[p] + x1 * cs[p]));
        }
        st16(y + off, w);
    }
}

template <typename T>
hipError_t launch_rope_t(const void* x, void* y, int B, int seq, int H, int D, double base,
                         int pos0, int inverse, hipStream_t stream) {
    constexpr int EPC = 16 / sizeof(T);
    RopeFreq f;
    for (int i = 0; i < D / 2; ++i) f.theta[i] = std::pow(base, -2.0 * (double)i / (double)D);
    for (int i = D / 2; i < 128; ++i) f.theta[i] = 0.0;
    const int nhb = (H + kHeadsPerThread - 1) / kHeadsPerThread;
    const long long nunits = (long long)B * seq * nhb * (D / EPC);
    const int threads = 256;
    const long long blocks = (nunits + threads - 1) / threads;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rope_kernel<T>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       static_cast<const T*>(x), static_cast<T*>(y), nunits, seq, H, D, pos0,
                       inverse, f);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const void* x, void* y, int B, int T, int H, int D, IoType dt,
                       double base, int pos0, int inverse, hipStream_t stream) {
    if (dt == kF32) return launch_rope_t<float>(x, y, B, T, H, D, base, pos0, inverse, stream);
    return launch_rope_t<bf16>(x, y, B, T, H, D, base, pos0, inverse, stream);
}

}  // namespace ea
