// api.hip -- the C ABI of libeuler_attn: argument validation and dispatch.
//
// Every entry point validates all of its arguments before anything is enqueued (no HIP
// call happens on an invalid call), then hands off to the internal launchers.  Nothing is
// allocated, freed or synchronised here.  Declarations and the contract: euler_attn.h.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <mutex>

#include "ea_kernels.h"
#include "euler_attn.h"

// Scratch of attn_bwd_noalloc: D_t of one backward call, in a fixed array that each device
// holds for the life of the process.  In host code this name is only a handle for the
// symbol lookup below: kernels receive the per-device address that the lookup returns.
static __device__ __align__(256) unsigned char scratch[EA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range(const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

size_t elem_size(ea_dtype dt) { return dt == EA_F32 ? 4 : 2; }

bool dtype_ok(int dt) { return dt == EA_F32 || dt == EA_BF16; }

bool attn_dim_ok(int D) { return D == 32 || D == 64 || D == 128; }

ea_status from_hip(hipError_t e) { return e == hipSuccess ? EA_OK : EA_ERR_HIP; }

// Shared checks of attn_fwd / attn_bwd sizes.
ea_status check_attn_sizes(int B, int T, int Hq, int Hkv, int D, float scale, int dt) {
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return EA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return EA_ERR_INVALID_ARG;
    if (!dtype_ok(dt) || !attn_dim_ok(D)) return EA_ERR_UNSUPPORTED;
    // The kernels index with 64-bit arithmetic but launch 1-D grids of 32-bit size.
    if ((long long)B * Hq > (1LL << 24) || T > (1 << 28)) return EA_ERR_UNSUPPORTED;
    return EA_OK;
}

ea_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int T, int Hq, int Hkv, int D, float scale, ea_dtype dt, bool causal,
                   hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return EA_ERR_NULL;
    ea_status st = check_attn_sizes(B, T, Hq, Hkv, D, scale, dt);
    if (st != EA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return EA_ERR_ALIGN;
    const size_t es = elem_size(dt);
    const Range rq = range(q, (size_t)B * T * Hq * D * es);
    const Range rk = range(k, (size_t)B * T * Hkv * D * es);
    const Range rv = range(v, (size_t)B * T * Hkv * D * es);
    const Range ro = range(o, (size_t)B * T * Hq * D * es);
    const Range rl = range(lse, (size_t)B * Hq * T * sizeof(float));
    for (Range out : {ro, rl})
        for (Range in : {rq, rk, rv})
            if (overlap(out, in)) return EA_ERR_ALIAS;
    if (overlap(ro, rl)) return EA_ERR_ALIAS;
    return from_hip(ea::launch_attn_fwd(q, k, v, o, lse, B, T, Hq, Hkv, D, scale,
                                        static_cast<ea::IoType>(dt), causal, stream));
}

}  // namespace

extern "C" {

const char* euler_attn_status_string(ea_status s) {
    switch (s) {
        case EA_OK: return "EA_OK: success";
        case EA_ERR_NULL: return "EA_ERR_NULL: a required pointer is NULL";
        case EA_ERR_INVALID_ARG: return "EA_ERR_INVALID_ARG: a size, count, scale, base or flag is out of range";
        case EA_ERR_UNSUPPORTED: return "EA_ERR_UNSUPPORTED: head_dim or dtype not supported";
        case EA_ERR_ALIGN: return "EA_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
        case EA_ERR_ALIAS: return "EA_ERR_ALIAS: an output overlaps an input or another output";
        case EA_ERR_WORKSPACE: return "EA_ERR_WORKSPACE: workspace smaller than attn_bwd_workspace_size()";
        case EA_ERR_HIP: return "EA_ERR_HIP: the HIP runtime reported an error at launch";
        case EA_ERR_SCRATCH:
            return "EA_ERR_SCRATCH: the problem needs more scratch than attn_bwd_noalloc's static "
                   "buffer (EA_NOALLOC_SCRATCH_BYTES) holds";
    }
    return "unknown euler_attn status";
}

int euler_attn_version(void) { return kVersion; }

ea_status rope_apply(const void* x, void* y, int B, int T, int H, int D, ea_dtype dt,
                     double base, int pos0, int inverse, hipStream_t stream) {
    if (x == nullptr || y == nullptr) return EA_ERR_NULL;
    if (B < 1 || T < 1 || H < 1 || D < 2 || (D % 2) != 0 || pos0 < 0) return EA_ERR_INVALID_ARG;
    if (!std::isfinite(base) || !(base > 1.0) || (inverse != 0 && inverse != 1)) return EA_ERR_INVALID_ARG;
    if (!dtype_ok(dt) || D > 256) return EA_ERR_UNSUPPORTED;
    if ((long long)pos0 + T > (1LL << 31)) return EA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(y)) return EA_ERR_ALIGN;
    const size_t bytes = (size_t)B * T * H * D * elem_size(dt);
    if (x != y && overlap(range(x, bytes), range(y, bytes))) return EA_ERR_ALIAS;
    return from_hip(ea::launch_rope(x, y, B, T, H, D, static_cast<ea::IoType>(dt), base, pos0,
                                    inverse, stream));
}

ea_status rope_apply_qk(const void* q, void* q_out, int Hq, const void* k, void* k_out, int Hkv,
                        int B, int T, int D, ea_dtype dt, double base, int pos0, int inverse,
                        hipStream_t stream) {
    if (!q || !q_out || !k || !k_out) return EA_ERR_NULL;
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || D < 2 || (D % 2) != 0 || pos0 < 0) return EA_ERR_INVALID_ARG;
    if (!std::isfinite(base) || !(base > 1.0) || (inverse != 0 && inverse != 1)) return EA_ERR_INVALID_ARG;
    if (!dtype_ok(dt) || D > 256) return EA_ERR_UNSUPPORTED;
    if ((long long)pos0 + T > (1LL << 31)) return EA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(q_out) || !aligned16(k) || !aligned16(k_out)) return EA_ERR_ALIGN;
    const size_t es = elem_size(dt);
    const Range rq = range(q, (size_t)B * T * Hq * D * es), rqo = range(q_out, (size_t)B * T * Hq * D * es);
    const Range rk = range(k, (size_t)B * T * Hkv * D * es), rko = range(k_out, (size_t)B * T * Hkv * D * es);
    // Each output may equal its own input exactly; no other overlap.
    if ((q != q_out && overlap(rq, rqo)) || (k != k_out && overlap(rk, rko))) return EA_ERR_ALIAS;
    if (overlap(rqo, rk) || overlap(rqo, rko) || overlap(rko, rq) || overlap(rq, rk)) return EA_ERR_ALIAS;
    return from_hip(ea::launch_rope_pair(q, q_out, Hq, k, k_out, Hkv, B, T, D,
                                         static_cast<ea::IoType>(dt), base, pos0, inverse, stream));
}

ea_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int T, int Hq, int Hkv, int D, float scale, ea_dtype dt, hipStream_t stream) {
    return fwd_impl(q, k, v, o, lse, B, T, Hq, Hkv, D, scale, dt, true, stream);
}

size_t attn_fwd_rope_workspace_size(int T, int D) {
    if (T < 1 || D < 2 || (D % 2) != 0) return 0;
    return ((size_t)T * (D / 2) * 2 * sizeof(float) + 255) & ~(size_t)255;
}

ea_status attn_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse,
                        void* q_r, void* k_r, void* workspace, size_t workspace_bytes, int B,
                        int T, int Hq, int Hkv, int D, float scale, ea_dtype dt, double base,
                        int pos0, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !q_r || !k_r || !workspace) return EA_ERR_NULL;
    ea_status st = check_attn_sizes(B, T, Hq, Hkv, D, scale, dt);
    if (st != EA_OK) return st;
    if (!std::isfinite(base) || !(base > 1.0) || pos0 < 0 || (long long)pos0 + T > (1LL << 31))
        return EA_ERR_INVALID_ARG;
    const size_t ws_need = attn_fwd_rope_workspace_size(T, D);
    if (workspace_bytes < ws_need) return EA_ERR_WORKSPACE;
    for (const void* p : {q, k, v, static_cast<const void*>(o), static_cast<const void*>(lse),
                          static_cast<const void*>(q_r), static_cast<const void*>(k_r),
                          static_cast<const void*>(workspace)})
        if (!aligned16(p)) return EA_ERR_ALIGN;
    const size_t es = elem_size(dt);
    const Range ins[] = {range(q, (size_t)B * T * Hq * D * es), range(k, (size_t)B * T * Hkv * D * es),
                         range(v, (size_t)B * T * Hkv * D * es)};
    const Range outs[] = {range(o, (size_t)B * T * Hq * D * es), range(lse, (size_t)B * Hq * T * sizeof(float)),
                          range(q_r, (size_t)B * T * Hq * D * es), range(k_r, (size_t)B * T * Hkv * D * es),
                          range(workspace, ws_need)};
    for (const Range& out : outs)
        for (const Range& in : ins)
            if (overlap(out, in)) return EA_ERR_ALIAS;
    for (int i = 0; i < 5; ++i)
        for (int j = i + 1; j < 5; ++j)
            if (overlap(outs[i], outs[j])) return EA_ERR_ALIAS;
    float* tab = static_cast<float*>(workspace);
    const ea::IoType t = static_cast<ea::IoType>(dt);
    if (attn_fwd_rope_fuses_q(B, T, Hq, Hkv, D, dt) == 1) {
        const hipError_t e = ea::launch_rope_table(k, k_r, B, T, Hkv, D, t, base, pos0, tab, stream);
        if (e != hipSuccess) return EA_ERR_HIP;
        return from_hip(ea::launch_attn_fwd(q, k_r, v, o, lse, B, T, Hq, Hkv, D, scale, t, true, stream,
                                            tab, q_r));
    }
    // Short sequences: a query tile's key loop is too short to hide the rotation of its queries
    // in the prologue (and where the forward splits the keys of each query block over two
    // waves, that prologue sits on the longest workgroups), so Q is rotated with K in the first
    // launch (rope_apply_qk's kernel; the same arithmetic, so q_r, k_r, o and lse are bitwise
    // those of the fused form).
    const hipError_t e = ea::launch_rope_pair(q, q_r, Hq, k, k_r, Hkv, B, T, D, t, base, pos0, 0, stream);
    if (e != hipSuccess) return EA_ERR_HIP;
    return from_hip(ea::launch_attn_fwd(q_r, k_r, v, o, lse, B, T, Hq, Hkv, D, scale, t, true, stream));
}

// Measured (bf16, both forms timed on the same inputs): fusing loses 4.6% at T = 1024 with the
// key split and 3.5% at T = 512 without it, and wins 2.3% at T = 4096 (head_dim 128) and 8.6%
// at T = 8192.
constexpr int kFuseQMinT = 2048;

int attn_fwd_rope_fuses_q(int B, int T, int Hq, int Hkv, int D, ea_dtype dt) {
    if (check_attn_sizes(B, T, Hq, Hkv, D, 1.0f, dt) != EA_OK) return -1;
    if (T < kFuseQMinT) return 0;
    return ea::fwd_splits_keys(B, T, Hq, Hkv, D, static_cast<ea::IoType>(dt)) ? 0 : 1;
}

ea_status attn_fwd_noncausal(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int T, int Hq, int Hkv, int D, float scale, ea_dtype dt,
                             hipStream_t stream) {
    return fwd_impl(q, k, v, o, lse, B, T, Hq, Hkv, D, scale, dt, false, stream);
}

size_t attn_bwd_workspace_size(int B, int T, int Hq, int Hkv, int D, ea_dtype dt) {
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D < 1 || !dtype_ok(dt)) return 0;
    return ea::bwd_workspace_bytes(B, T, Hq, D, false);
}

size_t attn_decode_workspace_size(int B, int Tq, int Tk, int Hq, int Hkv, int D, ea_dtype dt) {
    if (B < 1 || Tq < 1 || Tk < Tq || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || !dtype_ok(dt)) return 0;
    if (D != 32 && D != 64 && D != 128) return 0;
    return ea::decode_workspace_bytes(B, Tq, Tk, Hq, Hkv, D);
}

ea_status attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                      void* workspace, size_t workspace_bytes, int B, int Tq, int Tk, int Hq,
                      int Hkv, int D, float scale, ea_dtype dt, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !workspace) return EA_ERR_NULL;
    if (Tq < 1 || Tk < Tq) return EA_ERR_INVALID_ARG;
    ea_status st = check_attn_sizes(B, Tk, Hq, Hkv, D, scale, dt);
    if (st != EA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return EA_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return EA_ERR_ALIGN;
    const size_t need = ea::decode_workspace_bytes(B, Tq, Tk, Hq, Hkv, D);
    if (workspace_bytes < need) return EA_ERR_WORKSPACE;
    const size_t es = elem_size(dt);
    const Range rq = range(q, (size_t)B * Tq * Hq * D * es);
    const Range rk = range(k, (size_t)B * Tk * Hkv * D * es);
    const Range rv = range(v, (size_t)B * Tk * Hkv * D * es);
    const Range ro = range(o, (size_t)B * Tq * Hq * D * es);
    const Range rl = range(lse, (size_t)B * Hq * Tq * sizeof(float));
    const Range rw = range(workspace, need);
    for (Range out : {ro, rl, rw})
        for (Range in : {rq, rk, rv})
            if (overlap(out, in)) return EA_ERR_ALIAS;
    if (overlap(ro, rl) || overlap(ro, rw) || overlap(rl, rw)) return EA_ERR_ALIAS;
    return from_hip(ea::launch_attn_decode(q, k, v, o, lse, workspace, B, Tq, Tk, Hq, Hkv, D, scale,
                                           static_cast<ea::IoType>(dt), stream));
}

size_t attn_bwd_rope_workspace_size(int B, int T, int Hq, int Hkv, int D, ea_dtype dt) {
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D < 2 || !dtype_ok(dt)) return 0;
    return ea::bwd_workspace_bytes(B, T, Hq, D, true);
}

}  // extern "C"

namespace {

struct BwdSizes {
    size_t qb, kb, lseb, ws;
};

BwdSizes bwd_sizes(int B, int T, int Hq, int Hkv, int D, ea_dtype dt, bool rope = false) {
    const size_t es = elem_size(dt);
    return BwdSizes{(size_t)B * T * Hq * D * es, (size_t)B * T * Hkv * D * es,
                    (size_t)B * Hq * T * sizeof(float), ea::bwd_workspace_bytes(B, T, Hq, D, rope)};
}

ea_status check_rope_args(double base, int pos0, int T) {
    if (!std::isfinite(base) || !(base > 1.0) || pos0 < 0) return EA_ERR_INVALID_ARG;
    if ((long long)pos0 + T > (1LL << 31)) return EA_ERR_INVALID_ARG;
    return EA_OK;
}

ea_status check_workspace(const void* ws, size_t bytes, size_t need) {
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return EA_ERR_ALIGN;
    if (bytes < need) return EA_ERR_WORKSPACE;
    return EA_OK;
}

template <size_t NI, size_t NO>
ea_status check_alias(const Range (&ins)[NI], const Range (&outs)[NO]) {
    for (const Range& out : outs)
        for (const Range& in : ins)
            if (overlap(out, in)) return EA_ERR_ALIAS;
    for (size_t a = 0; a < NO; ++a)
        for (size_t c = a + 1; c < NO; ++c)
            if (overlap(outs[a], outs[c])) return EA_ERR_ALIAS;
    return EA_OK;
}

ea_status bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, int B, int T, int Hq, int Hkv, int D, float scale,
                   ea_dtype dt, const ea::RopeArgs* rope, bool causal, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace) return EA_ERR_NULL;
    ea_status st = check_attn_sizes(B, T, Hq, Hkv, D, scale, dt);
    if (st != EA_OK) return st;
    if (rope && (st = check_rope_args(rope->base, rope->pos0, T)) != EA_OK) return st;
    for (const void* p : {q, k, v, o, static_cast<const void*>(lse), dout,
                          static_cast<const void*>(dq), static_cast<const void*>(dk),
                          static_cast<const void*>(dv)})
        if (!aligned16(p)) return EA_ERR_ALIGN;
    const BwdSizes z = bwd_sizes(B, T, Hq, Hkv, D, dt, rope != nullptr);
    if ((st = check_workspace(workspace, workspace_bytes, z.ws)) != EA_OK) return st;
    const Range ins[] = {range(q, z.qb), range(k, z.kb), range(v, z.kb), range(o, z.qb),
                         range(lse, z.lseb), range(dout, z.qb)};
    const Range outs[] = {range(dq, z.qb), range(dk, z.kb), range(dv, z.kb), range(workspace, z.ws)};
    if ((st = check_alias(ins, outs)) != EA_OK) return st;
    return from_hip(ea::launch_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, T, Hq,
                                        Hkv, D, scale, static_cast<ea::IoType>(dt), rope, causal,
                                        stream));
}

ea_status pre_impl(const void* o, const void* dout, void* workspace, size_t workspace_bytes, int B,
                   int T, int Hq, int Hkv, int D, ea_dtype dt, const ea::RopeArgs* rope,
                   hipStream_t stream) {
    if (!o || !dout || !workspace) return EA_ERR_NULL;
    ea_status st = check_attn_sizes(B, T, Hq, Hkv, D, 1.0f, dt);
    if (st != EA_OK) return st;
    if (rope && (st = check_rope_args(rope->base, rope->pos0, T)) != EA_OK) return st;
    if (!aligned16(o) || !aligned16(dout)) return EA_ERR_ALIGN;
    const BwdSizes z = bwd_sizes(B, T, Hq, Hkv, D, dt, rope != nullptr);
    if ((st = check_workspace(workspace, workspace_bytes, z.ws)) != EA_OK) return st;
    const Range ins[] = {range(o, z.qb), range(dout, z.qb)};
    const Range outs[] = {range(workspace, z.ws)};
    if ((st = check_alias(ins, outs)) != EA_OK) return st;
    return from_hip(ea::launch_bwd_pre(o, dout, workspace, B, T, Hq, D,
                                       static_cast<ea::IoType>(dt), rope, stream));
}

ea_status main_impl(const void* q, const void* k, const void* v, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, const void* workspace,
                    size_t workspace_bytes, int B, int T, int Hq, int Hkv, int D, float scale,
                    ea_dtype dt, bool rope, hipStream_t stream) {
    if (!q || !k || !v || !lse || !dout || !dq || !dk || !dv || !workspace) return EA_ERR_NULL;
    ea_status st = check_attn_sizes(B, T, Hq, Hkv, D, scale, dt);
    if (st != EA_OK) return st;
    for (const void* p : {q, k, v, static_cast<const void*>(lse), dout, static_cast<const void*>(dq),
                          static_cast<const void*>(dk), static_cast<const void*>(dv)})
        if (!aligned16(p)) return EA_ERR_ALIGN;
    const BwdSizes z = bwd_sizes(B, T, Hq, Hkv, D, dt, rope);
    if ((st = check_workspace(workspace, workspace_bytes, z.ws)) != EA_OK) return st;
    const Range ins[] = {range(q, z.qb), range(k, z.kb), range(v, z.kb), range(lse, z.lseb),
                         range(dout, z.qb), range(workspace, z.ws)};
    const Range outs[] = {range(dq, z.qb), range(dk, z.kb), range(dv, z.kb)};
    if ((st = check_alias(ins, outs)) != EA_OK) return st;
    return from_hip(ea::launch_bwd_main(q, k, v, lse, dout, dq, dk, dv, const_cast<void*>(workspace),
                                        B, T, Hq, Hkv, D, scale, static_cast<ea::IoType>(dt), rope,
                                        true, stream));
}

}  // namespace

extern "C" {

ea_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, int B, int T, int Hq, int Hkv, int D, float scale,
                   ea_dtype dt, hipStream_t stream) {
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, T, Hq, Hkv,
                    D, scale, dt, nullptr, true, stream);
}

ea_status attn_bwd_noncausal(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, int B, int T, int Hq,
                             int Hkv, int D, float scale, ea_dtype dt, hipStream_t stream) {
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, T, Hq, Hkv,
                    D, scale, dt, nullptr, false, stream);
}

ea_status attn_bwd_rope(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, int B, int T, int Hq, int Hkv,
                        int D, float scale, ea_dtype dt, double base, int pos0,
                        hipStream_t stream) {
    const ea::RopeArgs rope{base, pos0};
    return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, T, Hq, Hkv,
                    D, scale, dt, &rope, true, stream);
}

ea_status attn_bwd_preprocess(const void* o, const void* dout, void* workspace,
                              size_t workspace_bytes, int B, int T, int Hq, int Hkv, int D,
                              ea_dtype dt, hipStream_t stream) {
    return pre_impl(o, dout, workspace, workspace_bytes, B, T, Hq, Hkv, D, dt, nullptr, stream);
}

ea_status attn_bwd_rope_preprocess(const void* o, const void* dout, void* workspace,
                                   size_t workspace_bytes, int B, int T, int Hq, int Hkv, int D,
                                   ea_dtype dt, double base, int pos0, hipStream_t stream) {
    const ea::RopeArgs rope{base, pos0};
    return pre_impl(o, dout, workspace, workspace_bytes, B, T, Hq, Hkv, D, dt, &rope, stream);
}

ea_status attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                        const void* dout, void* dk, void* dv, const void* workspace,
                        size_t workspace_bytes, int B, int T, int Hq, int Hkv, int D,
                        float scale, ea_dtype dt, hipStream_t stream) {
    if (!q || !k || !v || !lse || !dout || !dk || !dv || !workspace) return EA_ERR_NULL;
    ea_status st = check_attn_sizes(B, T, Hq, Hkv, D, scale, dt);
    if (st != EA_OK) return st;
    for (const void* p : {q, k, v, static_cast<const void*>(lse), dout,
                          static_cast<const void*>(dk), static_cast<const void*>(dv)})
        if (!aligned16(p)) return EA_ERR_ALIGN;
    const BwdSizes z = bwd_sizes(B, T, Hq, Hkv, D, dt);
    if ((st = check_workspace(workspace, workspace_bytes, z.ws)) != EA_OK) return st;
    const Range ins[] = {range(q, z.qb), range(k, z.kb), range(v, z.kb), range(lse, z.lseb),
                         range(dout, z.qb), range(workspace, z.ws)};
    const Range outs[] = {range(dk, z.kb), range(dv, z.kb)};
    if ((st = check_alias(ins, outs)) != EA_OK) return st;
    return from_hip(ea::launch_bwd_dkdv(q, k, v, lse, dout, dk, dv, const_cast<void*>(workspace),
                                        B, T, Hq, Hkv, D, scale, static_cast<ea::IoType>(dt), stream));
}

ea_status attn_bwd_main(const void* q, const void* k, const void* v, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, const void* workspace,
                        size_t workspace_bytes, int B, int T, int Hq, int Hkv, int D,
                        float scale, ea_dtype dt, hipStream_t stream) {
    return main_impl(q, k, v, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, T, Hq, Hkv, D,
                     scale, dt, false, stream);
}

ea_status attn_bwd_rope_main(const void* q, const void* k, const void* v, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, const void* workspace,
                             size_t workspace_bytes, int B, int T, int Hq, int Hkv, int D,
                             float scale, ea_dtype dt, hipStream_t stream) {
    return main_impl(q, k, v, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, T, Hq, Hkv, D,
                     scale, dt, true, stream);
}

ea_status attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                      const void* dout, void* dq, const void* workspace, size_t workspace_bytes,
                      int B, int T, int Hq, int Hkv, int D, float scale, ea_dtype dt,
                      hipStream_t stream) {
    if (!q || !k || !v || !lse || !dout || !dq || !workspace) return EA_ERR_NULL;
    ea_status st = check_attn_sizes(B, T, Hq, Hkv, D, scale, dt);
    if (st != EA_OK) return st;
    for (const void* p : {q, k, v, static_cast<const void*>(lse), dout, static_cast<const void*>(dq)})
        if (!aligned16(p)) return EA_ERR_ALIGN;
    const BwdSizes z = bwd_sizes(B, T, Hq, Hkv, D, dt);
    if ((st = check_workspace(workspace, workspace_bytes, z.ws)) != EA_OK) return st;
    const Range ins[] = {range(q, z.qb), range(k, z.kb), range(v, z.kb), range(lse, z.lseb),
                         range(dout, z.qb), range(workspace, z.ws)};
    const Range outs[] = {range(dq, z.qb)};
    if ((st = check_alias(ins, outs)) != EA_OK) return st;
    return from_hip(ea::launch_bwd_dq(q, k, v, lse, dout, dq, const_cast<void*>(workspace), B, T,
                                      Hq, Hkv, D, scale, static_cast<ea::IoType>(dt), stream));
}

}  // extern "C"

namespace {

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept for the life of the process.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

ea_status scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return EA_ERR_HIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
                return EA_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return EA_OK;
}

}  // namespace

extern "C" {

ea_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int B, int T, int Hq, int Hkv, int D, float scale, ea_dtype dt,
                           hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return EA_ERR_NULL;
    ea_status st = check_attn_sizes(B, T, Hq, Hkv, D, scale, dt);
    if (st != EA_OK) return st;
    for (const void* p : {q, k, v, o, static_cast<const void*>(lse), dout,
                          static_cast<const void*>(dq), static_cast<const void*>(dk),
                          static_cast<const void*>(dv)})
        if (!aligned16(p)) return EA_ERR_ALIGN;
    const BwdSizes z = bwd_sizes(B, T, Hq, Hkv, D, dt);
    if (z.ws > (size_t)EA_NOALLOC_SCRATCH_BYTES) return EA_ERR_SCRATCH;
    const Range ins[] = {range(q, z.qb), range(k, z.kb), range(v, z.kb), range(o, z.qb),
                         range(lse, z.lseb), range(dout, z.qb)};
    const Range outs[] = {range(dq, z.qb), range(dk, z.kb), range(dv, z.kb)};
    if ((st = check_alias(ins, outs)) != EA_OK) return st;
    void* ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != EA_OK) return st;
    // The same two stages as attn_bwd; the pre-pass writes every D_t entry the main stage
    // reads, so nothing left in the scratch by an earlier call is ever read.
    return from_hip(ea::launch_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, B, T, Hq, Hkv, D,
                                        scale, static_cast<ea::IoType>(dt), nullptr, true, stream));
}

}  // extern "C"

namespace {

// Bytes spanned by `rows` rows of `cols` elements with leading dimension ld.
size_t span_bytes(long long rows, long long cols, long long ld, size_t es) {
    return (size_t)(((rows - 1) * ld + cols) * (long long)es);
}

// The QKV projection's three column segments (Q, K, V) of the [B*T, (Hq + 2 Hkv) D] product.
void qkv_segs(ea::GemmSeg* s, const void* q, const void* k, const void* v, int Hq, int Hkv, int D) {
    s[0] = ea::GemmSeg{q, (long long)Hq * D, 0};
    s[1] = ea::GemmSeg{k, (long long)Hkv * D, Hq * D};
    s[2] = ea::GemmSeg{v, (long long)Hkv * D, (Hq + Hkv) * D};
}

ea_status check_qkv_sizes(int B, int T, int C, int Hq, int Hkv, int D, ea_dtype dt) {
    if (B < 1 || T < 1 || C < 1 || Hq < 1 || Hkv < 1 || D < 2 || Hq % Hkv != 0) return EA_ERR_INVALID_ARG;
    if (!dtype_ok(dt)) return EA_ERR_UNSUPPORTED;
    const int epc = (int)(16 / elem_size(dt));
    if (C % epc != 0 || D % epc != 0 || D > 256) return EA_ERR_UNSUPPORTED;
    if ((long long)B * T > (1LL << 30) || (long long)(Hq + 2 * Hkv) * D > (1 << 24) || C > (1 << 24))
        return EA_ERR_UNSUPPORTED;
    return EA_OK;
}

// The split-K workspace of one product: 256-byte aligned, at least `need` bytes (may be NULL
// when need is 0), overlapping none of the operands.
ea_status check_splitk_ws(const void* ws, size_t bytes, size_t need, std::initializer_list<Range> others) {
    if (need == 0) return EA_OK;
    if (!ws) return EA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return EA_ERR_ALIGN;
    if (bytes < need) return EA_ERR_WORKSPACE;
    const Range rw = range(ws, need);
    for (Range r : others)
        if (overlap(rw, r)) return EA_ERR_ALIAS;
    return EA_OK;
}

// Shape checks of gemm; 0 when the product is supported.
ea_status check_gemm(int M, int N, int K, int lda, int ldb, int ldc, int trans_a, int trans_b, ea_dtype dt) {
    if (M < 1 || N < 1 || K < 1) return EA_ERR_INVALID_ARG;
    if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1)) return EA_ERR_INVALID_ARG;
    if (!dtype_ok(dt) || (trans_a == 1 && trans_b == 1)) return EA_ERR_UNSUPPORTED;
    const int epc = (int)(16 / elem_size(dt));
    // 16-byte chunks along every contiguous dimension that is loaded or stored.
    if (N % epc != 0 || ((trans_a == 0 || trans_b == 1) && K % epc != 0) || (trans_a == 1 && M % epc != 0))
        return EA_ERR_UNSUPPORTED;
    const long long a_cols = trans_a ? M : K, b_cols = trans_b ? K : N;
    if (lda < a_cols || ldb < b_cols || ldc < N) return EA_ERR_INVALID_ARG;
    if (lda % epc || ldb % epc || ldc % epc) return EA_ERR_ALIGN;
    return EA_OK;
}

ea_status gemm_impl(const void* a, const void* b, void* c, int M, int N, int K, int lda, int ldb,
                    int ldc, int trans_a, int trans_b, ea_dtype dt, void* ws, size_t ws_bytes,
                    bool use_ws, hipStream_t stream) {
    if (!a || !b || !c) return EA_ERR_NULL;
    ea_status st = check_gemm(M, N, K, lda, ldb, ldc, trans_a, trans_b, dt);
    if (st != EA_OK) return st;
    if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return EA_ERR_ALIGN;
    const long long a_rows = trans_a ? K : M, a_cols = trans_a ? M : K;
    const long long b_rows = trans_b ? N : K, b_cols = trans_b ? K : N;
    const size_t es = elem_size(dt);
    const Range ra = range(a, span_bytes(a_rows, a_cols, lda, es));
    const Range rb = range(b, span_bytes(b_rows, b_cols, ldb, es));
    const Range rc = range(c, span_bytes(M, N, ldc, es));
    if (overlap(rc, ra) || overlap(rc, rb)) return EA_ERR_ALIAS;
    const size_t need = use_ws ? ea::gemm_splitk_bytes(M, N, K, static_cast<ea::IoType>(dt)) : 0;
    if ((st = check_splitk_ws(ws, ws_bytes, need, {ra, rb, rc})) != EA_OK) return st;
    const ea::GemmSeg sa{a, lda, 0}, sb{b, ldb, 0}, sc{c, ldc, 0};
    return from_hip(ea::launch_gemm(&sa, 1, &sb, 1, &sc, 1, M, N, K, trans_a, trans_b,
                                    static_cast<ea::IoType>(dt), nullptr, stream, need ? ws : nullptr, need));
}

}  // namespace

extern "C" {

ea_status gemm(const void* a, const void* b, void* c, int M, int N, int K, int lda, int ldb,
               int ldc, int trans_a, int trans_b, ea_dtype dt, hipStream_t stream) {
    return gemm_impl(a, b, c, M, N, K, lda, ldb, ldc, trans_a, trans_b, dt, nullptr, 0, false, stream);
}

size_t gemm_workspace_size(int M, int N, int K, int trans_a, int trans_b, ea_dtype dt) {
    if (check_gemm(M, N, K, trans_a ? M : K, trans_b ? K : N, N, trans_a, trans_b, dt) != EA_OK) return 0;
    return ea::gemm_splitk_bytes(M, N, K, static_cast<ea::IoType>(dt));
}

ea_status gemm_ws(const void* a, const void* b, void* c, int M, int N, int K, int lda, int ldb,
                  int ldc, int trans_a, int trans_b, ea_dtype dt, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
    return gemm_impl(a, b, c, M, N, K, lda, ldb, ldc, trans_a, trans_b, dt, workspace, workspace_bytes,
                     true, stream);
}

ea_status qkv_proj(const void* x, const void* w_qkv, void* q, void* k, void* v, int B, int T,
                   int C, int Hq, int Hkv, int D, ea_dtype dt, int rope, double base, int pos0,
                   hipStream_t stream) {
    if (!x || !w_qkv || !q || !k || !v) return EA_ERR_NULL;
    ea_status st = check_qkv_sizes(B, T, C, Hq, Hkv, D, dt);
    if (st != EA_OK) return st;
    if (rope != 0 && rope != 1) return EA_ERR_INVALID_ARG;
    if (rope && (st = check_rope_args(base, pos0, T)) != EA_OK) return st;
    for (const void* p : {x, w_qkv, static_cast<const void*>(q), static_cast<const void*>(k),
                          static_cast<const void*>(v)})
        if (!aligned16(p)) return EA_ERR_ALIGN;
    const size_t es = elem_size(dt);
    const long long M = (long long)B * T, N = (long long)(Hq + 2 * Hkv) * D;
    const Range ins[] = {range(x, (size_t)(M * C) * es), range(w_qkv, (size_t)(C * N) * es)};
    const Range outs[] = {range(q, (size_t)(M * Hq * D) * es), range(k, (size_t)(M * Hkv * D) * es),
                          range(v, (size_t)(M * Hkv * D) * es)};
    if ((st = check_alias(ins, outs)) != EA_OK) return st;
    const ea::GemmSeg sa{x, C, 0}, sb{w_qkv, N, 0};
    ea::GemmSeg sc[3];
    qkv_segs(sc, q, k, v, Hq, Hkv, D);
    const ea::GemmRope r{0x3, T, D, pos0, base};
    return from_hip(ea::launch_gemm(&sa, 1, &sb, 1, sc, 3, (int)M, (int)N, C, 0, 0,
                                    static_cast<ea::IoType>(dt), rope ? &r : nullptr, stream));
}

}  // extern "C"

namespace {

ea_status qkv_proj_bwd_impl(const void* x, const void* w_qkv, const void* dq, const void* dk,
                            const void* dv, void* dx, void* dw_qkv, int B, int T, int C, int Hq,
                            int Hkv, int D, ea_dtype dt, void* ws, size_t ws_bytes, bool use_ws,
                            hipStream_t stream) {
    if (!x || !w_qkv || !dq || !dk || !dv || !dx || !dw_qkv) return EA_ERR_NULL;
    ea_status st = check_qkv_sizes(B, T, C, Hq, Hkv, D, dt);
    if (st != EA_OK) return st;
    for (const void* p : {x, w_qkv, dq, dk, dv, static_cast<const void*>(dx), static_cast<const void*>(dw_qkv)})
        if (!aligned16(p)) return EA_ERR_ALIGN;
    const size_t es = elem_size(dt);
    const long long M = (long long)B * T, N = (long long)(Hq + 2 * Hkv) * D;
    const Range ins[] = {range(x, (size_t)(M * C) * es), range(w_qkv, (size_t)(C * N) * es),
                         range(dq, (size_t)(M * Hq * D) * es), range(dk, (size_t)(M * Hkv * D) * es),
                         range(dv, (size_t)(M * Hkv * D) * es)};
    const Range outs[] = {range(dx, (size_t)(M * C) * es), range(dw_qkv, (size_t)(C * N) * es)};
    if ((st = check_alias(ins, outs)) != EA_OK) return st;
    const ea::IoType io = static_cast<ea::IoType>(dt);
    // The two products run one after the other on the stream and share the workspace.
    const size_t need_dx = use_ws ? ea::gemm_splitk_bytes((int)M, C, (int)N, io) : 0;
    const size_t need_dw = use_ws ? ea::gemm_splitk_bytes(C, (int)N, (int)M, io) : 0;
    if ((st = check_splitk_ws(ws, ws_bytes, std::max(need_dx, need_dw),
                              {ins[0], ins[1], ins[2], ins[3], ins[4], outs[0], outs[1]})) != EA_OK)
        return st;
    ea::GemmSeg g[3];
    qkv_segs(g, dq, dk, dv, Hq, Hkv, D);
    // dx = [dq | dk | dv] W^T: A split along K, B = W stored [C, N] = op(B)^T.
    const ea::GemmSeg wb{w_qkv, N, 0}, sdx{dx, C, 0};
    hipError_t e = ea::launch_gemm(g, 3, &wb, 1, &sdx, 1, (int)M, C, (int)N, 0, 1, io, nullptr, stream,
                                   need_dx ? ws : nullptr, need_dx);
    if (e != hipSuccess) return from_hip(e);
    // dW = x^T [dq | dk | dv]: A = x stored [M, C] = op(A)^T, B split along N.
    const ea::GemmSeg xa{x, C, 0}, sdw{dw_qkv, N, 0};
    return from_hip(ea::launch_gemm(&xa, 1, g, 3, &sdw, 1, C, (int)N, (int)M, 1, 0, io, nullptr, stream,
                                    need_dw ? ws : nullptr, need_dw));
}

}  // namespace

extern "C" {

ea_status qkv_proj_bwd(const void* x, const void* w_qkv, const void* dq, const void* dk,
                       const void* dv, void* dx, void* dw_qkv, int B, int T, int C, int Hq,
                       int Hkv, int D, ea_dtype dt, hipStream_t stream) {
    return qkv_proj_bwd_impl(x, w_qkv, dq, dk, dv, dx, dw_qkv, B, T, C, Hq, Hkv, D, dt, nullptr, 0, false,
                             stream);
}

size_t qkv_proj_bwd_workspace_size(int B, int T, int C, int Hq, int Hkv, int D, ea_dtype dt) {
    if (check_qkv_sizes(B, T, C, Hq, Hkv, D, dt) != EA_OK) return 0;
    const long long M = (long long)B * T, N = (long long)(Hq + 2 * Hkv) * D;
    if (M > 0x7fffffffLL || N > 0x7fffffffLL) return 0;
    const ea::IoType io = static_cast<ea::IoType>(dt);
    return std::max(ea::gemm_splitk_bytes((int)M, C, (int)N, io), ea::gemm_splitk_bytes(C, (int)N, (int)M, io));
}

ea_status qkv_proj_bwd_ws(const void* x, const void* w_qkv, const void* dq, const void* dk,
                          const void* dv, void* dx, void* dw_qkv, int B, int T, int C, int Hq,
                          int Hkv, int D, ea_dtype dt, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    return qkv_proj_bwd_impl(x, w_qkv, dq, dk, dv, dx, dw_qkv, B, T, C, Hq, Hkv, D, dt, workspace,
                             workspace_bytes, true, stream);
}

}  // extern "C"
