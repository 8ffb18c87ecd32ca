// ea_kernels.h -- internal launchers behind the C ABI (arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ea {

enum IoType { kF32 = 0, kBF16 = 1 };

// Inverse RoPE fused into the backward: gradients are returned for the pre-rotation Q and K.
struct RopeArgs {
    double base;
    int pos0;
};

// RoPE of x [B, T, H, D] into y; see rope_apply in euler_attn.h.
hipError_t launch_rope(const void* x, void* y, int B, int T, int H, int D, IoType dt,
                       double base, int pos0, int inverse, hipStream_t stream);

// RoPE of x into y (forward angles) that also writes the (cos, sin) table of every
// (position, pair), fp32 [T, D/2, 2], into tab.
hipError_t launch_rope_table(const void* x, void* y, int B, int T, int H, int D, IoType dt,
                             double base, int pos0, float* tab, hipStream_t stream);

// RoPE of two tensors sharing (B, T, D) in one launch: x0 [B,T,H0,D] -> y0, x1 [B,T,H1,D] -> y1.
hipError_t launch_rope_pair(const void* x0, void* y0, int H0, const void* x1, void* y1, int H1,
                            int B, int T, int D, IoType dt, double base, int pos0, int inverse,
                            hipStream_t stream);

// Whether attn_fwd splits each query block's keys over two waves at this shape (small
// problems); D in {32, 64, 128}.
bool fwd_splits_keys(int B, int T, int Hq, int Hkv, int D, IoType dt);
// Forward: o [B, T, Hq, D], lse [B, Hq, T] (natural log); causal = false lets every query
// see every key.
// With qtab set, q holds the pre-RoPE queries: each row is rotated by the (cos, sin) table
// (fp32 [T, D/2, 2]) as it loads, and the rotated rows are written to q_r.
hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int T, int Hq, int Hkv, int D, float scale, IoType dt,
                           bool causal, hipStream_t stream, const float* qtab = nullptr,
                           void* q_r = nullptr);

// Workspace of the backward: D_t = sum_d dO * O as fp32 [B, Hq, T], 256-byte aligned; with
// rope, then the (cos, sin) table of the inverse RoPE, fp32 [T, D/2, 2], 256-byte aligned.
size_t bwd_workspace_bytes(int B, int T, int Hq, int D, bool rope);

// Backward stages (their composition is launch_attn_bwd):
//   pre:  D_t (and, with rope, the RoPE table) into the workspace;
//   dkdv: dk, dv (group-summed) from q, k, v, lse, dout and D_t;
//   dq:   dq from q, k, v, lse, dout and D_t (independent of dkdv).
hipError_t launch_bwd_pre(const void* o, const void* dout, void* workspace, int B, int T, int Hq,
                          int D, IoType dt, const RopeArgs* rope, hipStream_t stream);
hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                           const void* dout, void* dk, void* dv, void* workspace, int B, int T,
                           int Hq, int Hkv, int D, float scale, IoType dt, hipStream_t stream);
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                         const void* dout, void* dq, void* workspace, int B, int T, int Hq,
                         int Hkv, int D, float scale, IoType dt, hipStream_t stream);
// dkdv and dq in one launch (the two roles' workgroups interleaved, heaviest first); with
// rope, dq and dk are rotated by -phi (table from pre) before they are stored.  dkdv and dq
// alone are causal; main and the full backward take the mask as an argument.
hipError_t launch_bwd_main(const void* q, const void* k, const void* v, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, void* workspace, int B,
                           int T, int Hq, int Hkv, int D, float scale, IoType dt, bool rope,
                           bool causal, hipStream_t stream);

// Backward: dq, dk, dv from q, k, v, o, lse, dout; workspace as above (rope may be null).
hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           void* workspace, int B, int T, int Hq, int Hkv, int D, float scale,
                           IoType dt, const RopeArgs* rope, bool causal, hipStream_t stream);

// Attention of Tq new query rows (q, o [B, Tq, Hq, D]; lse [B, Hq, Tq]) against a cache
// k, v [B, Tk, Hkv, D], Tq <= Tk: query row i sits at position Tk - Tq + i.  The workspace
// holds the per-chunk partials (decode_workspace_bytes, 256-byte aligned).
size_t decode_workspace_bytes(int B, int Tq, int Tk, int Hq, int Hkv, int D);
hipError_t launch_attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                              void* workspace, int B, int Tq, int Tk, int Hq, int Hkv, int D,
                              float scale, IoType dt, hipStream_t stream);

// Matrix product C = op(A) op(B) (gemm.hip).  A may be split along K, B and C along N, into up
// to kGemmMaxSeg segments (start = first index of the segment along the split dimension,
// ld = leading dimension in elements; the first segment starts at 0).  trans_a / trans_b:
// (0, 0), (0, 1) or (1, 0).  With rope, the column pairs of the C segments in rope->mask are
// rotated as heads of rope->D columns at position pos0 + (m mod T).
constexpr int kGemmMaxSeg = 3;
struct GemmSeg {
    const void* p;
    long long ld;
    int start;
};
struct GemmRope {
    int mask;
    int T, D, pos0;
    double base;
};
// splitk_ws (optional, splitk_bytes long): fp32 scratch that lets a product with few output tiles
// and a long K split its K range over more workgroups (two launches); gemm_splitk_bytes gives the
// size it uses (0: no split for this shape).
hipError_t launch_gemm(const GemmSeg* a, int na, const GemmSeg* b, int nb, const GemmSeg* c,
                       int nc, int M, int N, int K, int trans_a, int trans_b, IoType dt,
                       const GemmRope* rope, hipStream_t stream, void* splitk_ws = nullptr,
                       size_t splitk_bytes = 0);
size_t gemm_splitk_bytes(int M, int N, int K, IoType dt);

}  // namespace ea
