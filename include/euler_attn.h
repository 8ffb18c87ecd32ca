/*
 * euler_attn.h -- C ABI of libeuler_attn: causal grouped-query attention with rotary
 * position embeddings, forward and backward, as hand-written HIP kernels for gfx950.
 *
 * What is computed (sources: the web pages describing NanoEuler's training engine):
 *  - Rotary embeddings on queries and keys ("Show HN: NanoEuler", section 2 "模型组件";
 *    "Tiny Hackable CUDA Language Model Implementation", section 1 "架构设计").
 *  - Causal scaled dot-product attention: query t sees keys s <= t ("Tiny Hackable ...",
 *    section 1), with several query heads sharing one key/value head (GQA, "Show HN:
 *    NanoEuler", section 2).
 *  - Computed tile by tile with an online softmax so that the T x T score matrix is never
 *    stored ("Show HN: NanoEuler", section 4 "硬件与性能"; the blog's "Tiled
 *    FlashAttention" section), in forward and in backward (both hand-written and
 *    gradient-checked, "Show HN: NanoEuler", section 3).
 *
 * Conventions shared by every call:
 *  - Q, O, dO, dQ are [B, T, Hq, D]; K, V, dK, dV are [B, T, Hkv, D]; all contiguous,
 *    row-major, D fastest, element type `dt`.  LSE is [B, Hq, T] float32 (natural log).
 *  - Query head h uses key/value head floor(h / g), g = Hq / Hkv.
 *  - The causal mask keeps key s for query t iff s <= t (diagonal included).
 *  - All pointers are DEVICE pointers owned by the caller.  The library never allocates,
 *    frees or synchronises; work is enqueued on `stream` (NULL = the null stream) and the
 *    call returns after the enqueue.  Asynchronous device faults surface at the caller's
 *    next synchronisation.
 *  - Argument validation happens before anything is enqueued: on any error the call
 *    returns the status below and writes nothing.
 *  - Every tensor pointer must be 16-byte aligned.  All index arithmetic is 64-bit.
 */
#ifndef EULER_ATTN_H
#define EULER_ATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EA_OK = 0,
    EA_ERR_NULL = 1,          /* a required pointer is NULL                               */
    EA_ERR_INVALID_ARG = 2,   /* a size, count, scale, base or flag is out of range       */
    EA_ERR_UNSUPPORTED = 3,   /* valid but not built: head_dim or dtype                   */
    EA_ERR_ALIGN = 4,         /* a tensor pointer is not 16-byte aligned                  */
    EA_ERR_ALIAS = 5,         /* an output overlaps an input or another output            */
    EA_ERR_WORKSPACE = 6,     /* workspace smaller than attn_bwd_workspace_size()         */
    EA_ERR_HIP = 7,           /* the HIP runtime reported an error at launch              */
    EA_ERR_SCRATCH = 8        /* attn_bwd_noalloc: the problem exceeds its static scratch */
} ea_status;

typedef enum {
    EA_F32 = 0,   /* float32 I/O; contractions on fp32 MFMA, fp32 softmax               */
    EA_BF16 = 1   /* bfloat16 I/O; contractions on bf16 MFMA with fp32 accumulation,    */
                  /* every fp32 -> bf16 conversion rounds to nearest even                */
} ea_dtype;

/*
 * rope_apply -- rotary position embedding of x [B, T, H, D] into y (same shape and dtype).
 * For each row (b, t, h) and each adjacent pair (x[2i], x[2i+1]), i in [0, D/2), rotate by
 * phi = (pos0 + t) * base^(-2i/D):  y[2i] = x[2i] cos phi - x[2i+1] sin phi,
 * y[2i+1] = x[2i] sin phi + x[2i+1] cos phi.  inverse = 1 rotates by -phi, which is the
 * backward of the forward rotation (the rotation is orthogonal): apply it to dQ and dK to
 * obtain gradients with respect to the pre-RoPE tensors.  The angle is formed and reduced
 * modulo 2*pi in float64; sin/cos of the reduced angle and the rotation are float32.
 * Every even D from 2 to 256 is accepted: head dims that are a whole number of 16-byte
 * chunks (D a multiple of 8 for bf16, of 4 for fp32) are moved in 16-byte pieces, any other
 * even D pair by pair, with the same arithmetic.
 * y == x (exactly) is allowed (in place); any other overlap is EA_ERR_ALIAS.
 * Errors: NULL x or y; B, T, H < 1, D odd or < 2, pos0 < 0, base <= 1 or not finite,
 * inverse not 0/1 (EA_ERR_INVALID_ARG); D > 256 or unknown dt (EA_ERR_UNSUPPORTED).
 */
ea_status rope_apply(const void* x, void* y, int B, int T, int H, int D, ea_dtype dt,
                     double base, int pos0, int inverse, hipStream_t stream);

/*
 * rope_apply_qk -- rope_apply on two tensors that share (B, T, D) in one launch: q [B,T,Hq,D]
 * into q_out and k [B,T,Hkv,D] into k_out (the queries and keys before attn_fwd, or with
 * inverse = 1 the gradients dQ and dK after attn_bwd).  Same arithmetic, layouts and errors
 * as rope_apply; each output may equal its own input exactly, no other overlap is allowed.
 */
ea_status rope_apply_qk(const void* q, void* q_out, int Hq, const void* k, void* k_out, int Hkv,
                        int B, int T, int D, ea_dtype dt, double base, int pos0, int inverse,
                        hipStream_t stream);

/*
 * attn_fwd -- causal GQA attention forward.  For every batch b, query head h and query
 * position t:  S_ts = scale * <q_t, k_s> for s <= t;  O_t = sum_s softmax_s(S_t.) v_s;
 * LSE_t = log sum_{s<=t} exp(S_ts).  q and k are expected to carry RoPE already.
 * Outputs: o [B, T, Hq, D] in dt; lse [B, Hq, T] float32 (needed by attn_bwd).
 * Errors: NULL pointer; B, T, Hq, Hkv < 1, Hq % Hkv != 0, scale not finite or <= 0
 * (EA_ERR_INVALID_ARG); D not in {32, 64, 128} or unknown dt (EA_ERR_UNSUPPORTED);
 * misalignment (EA_ERR_ALIGN); o or lse overlapping q, k, v or each other (EA_ERR_ALIAS).
 */
ea_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int T, int Hq, int Hkv, int D, float scale, ea_dtype dt,
                   hipStream_t stream);

/*
 * attn_fwd_rope -- rope_apply on q and k fused with attn_fwd: the rotary embedding that
 * "Show HN: NanoEuler" (section 2) applies to queries and keys, then causal GQA attention on
 * the rotated tensors.  Inputs are the pre-RoPE q [B,T,Hq,D] and k [B,T,Hkv,D], and v.  Two
 * launches on stream: K is rotated once (into k_r), which also fills the (cos, sin) table of
 * every (position, pair) in the workspace; the forward then rotates each query row as it
 * loads it (queries stay in registers for the whole key loop, so each is rotated once) and
 * writes it to q_r.  Where that does not pay (attn_fwd_rope_fuses_q returns 0: sequences
 * shorter than 2048 positions, whose query tiles have too few key tiles to hide the rotation,
 * and problems whose forward splits each query block's keys over two waves) the first launch
 * rotates Q and K together instead and the forward reads q_r; the outputs are bitwise the
 * same either way.  Outputs: o, lse as attn_fwd; q_r, k_r the rotated q and k in dt, the inputs
 * attn_bwd / attn_bwd_rope need.  Angles and arithmetic are rope_apply's (base, pos0,
 * adjacent pairs; float64 angle reduction, float32 rotation); q_r and k_r equal rope_apply's
 * output bitwise.
 * workspace: at least attn_fwd_rope_workspace_size(T, D) bytes, 16-byte aligned, contents on
 * entry don't care (attn_fwd_rope_workspace_size returns 0 for T < 1 or D odd or < 2).
 * Errors: as attn_fwd, plus NULL q_r, k_r or workspace (EA_ERR_NULL); base <= 1 or not finite,
 * pos0 < 0 (EA_ERR_INVALID_ARG); workspace too small (EA_ERR_WORKSPACE); any of o, lse, q_r,
 * k_r, workspace overlapping q, k, v or each other (EA_ERR_ALIAS: no output may alias an
 * input here, in-place rotation included).
 */
size_t attn_fwd_rope_workspace_size(int T, int D);
/* attn_fwd_rope_fuses_q -- 1 if attn_fwd_rope rotates the queries inside the forward at this
 * shape, 0 if its first launch rotates them with K instead, -1 for sizes attn_fwd rejects.
 * Host-only: launches nothing. */
int attn_fwd_rope_fuses_q(int B, int T, int Hq, int Hkv, int D, ea_dtype dt);
ea_status attn_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse,
                        void* q_r, void* k_r, void* workspace, size_t workspace_bytes, int B,
                        int T, int Hq, int Hkv, int D, float scale, ea_dtype dt, double base,
                        int pos0, hipStream_t stream);

/*
 * attn_fwd_noncausal -- attn_fwd without the causal mask: every query row sees every key row,
 * S_ts = scale * <q_t, k_s> for all s in [0, T);  O_t = sum_s softmax_s(S_t.) v_s;
 * LSE_t = log sum_s exp(S_ts).  This is the form of the tiled FlashAttention forward that the
 * smartinfralog.com post on NanoEuler prints (section "Tiled FlashAttention": each query
 * tile walks over every K/V tile).  Same arguments, layouts, K/V-head map and errors as
 * attn_fwd; the lse it returns is the one attn_bwd_noncausal needs.
 */
ea_status attn_fwd_noncausal(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int T, int Hq, int Hkv, int D, float scale, ea_dtype dt,
                             hipStream_t stream);

/*
 * attn_decode -- attention of Tq new query rows against a KV cache, the step of generation
 * with a cache (one token at a time, or the K tokens of the multi-token prediction heads'
 * speculative decoding: "Show HN: NanoEuler", section 2).  q [B, Tq, Hq, D] holds the
 * queries of the last Tq positions of a Tk-long sequence; k, v [B, Tk, Hkv, D] hold the
 * whole cache, those positions included.  Query row i sits at position Tk - Tq + i and
 * attends causally to the keys s <= Tk - Tq + i:  O_i = softmax_s(scale * <q_i, k_s>) V,
 * LSE_i = log sum_s exp(scale * <q_i, k_s>), with the same K/V-head map as attn_fwd.  With
 * Tq = Tk the result is attn_fwd's (attn_fwd is the faster kernel for that case).
 * Outputs: o [B, Tq, Hq, D] in dt; lse [B, Hq, Tq] float32 (natural log).
 * The cache is split into chunks read by independent waves and their partial results are
 * merged exactly (in a fixed order: bitwise reproducible).  When a group's chunks fit one
 * workgroup (at most 4-16 chunks by head_dim and type) one launch merges them through LDS;
 * otherwise the partials go to the workspace (at least attn_decode_workspace_size(...)
 * bytes, 256-byte aligned, contents ignored) and a second launch merges them.
 * Errors: as attn_fwd (with T = Tk), plus Tq < 1 or Tq > Tk (EA_ERR_INVALID_ARG), workspace
 * too small (EA_ERR_WORKSPACE) or not 256-byte aligned (EA_ERR_ALIGN), and o, lse or the
 * workspace overlapping an input or each other (EA_ERR_ALIAS).
 */
size_t attn_decode_workspace_size(int B, int Tq, int Tk, int Hq, int Hkv, int D, ea_dtype dt);
ea_status attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                      void* workspace, size_t workspace_bytes, int B, int Tq, int Tk, int Hq,
                      int Hkv, int D, float scale, ea_dtype dt, hipStream_t stream);

/*
 * attn_bwd_workspace_size -- bytes of device scratch attn_bwd needs: the per-row
 * D_t = sum_d dO * O as float32 [B, Hq, T], rounded up to 256 bytes.  Linear in T (never
 * T^2).  Returns 0 for invalid sizes.
 */
size_t attn_bwd_workspace_size(int B, int T, int Hq, int Hkv, int D, ea_dtype dt);

/*
 * attn_bwd -- causal GQA attention backward (gradients of sum(dout * O)).  Inputs are the
 * forward's q, k, v, o, lse and the upstream gradient dout [B, T, Hq, D].  Outputs, all
 * overwritten (not accumulated):  dq [B, T, Hq, D];  dk, dv [B, T, Hkv, D], each summed
 * over the g query heads that share the K/V head.  The softmax is recomputed tile by tile
 * from lse; D_t = sum_d dout * o.  No atomics are used: dq, dk and dv are bitwise
 * reproducible from run to run.
 * workspace: device memory of at least attn_bwd_workspace_size(...) bytes, 256-byte
 * aligned, contents on entry ignored, clobbered on return.
 * Errors: as attn_fwd; dq/dk/dv/workspace overlapping any input or each other
 * (EA_ERR_ALIAS); workspace NULL or too small (EA_ERR_NULL / EA_ERR_WORKSPACE).
 */
ea_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes, int B, int T, int Hq, int Hkv,
                   int D, float scale, ea_dtype dt, hipStream_t stream);

/*
 * attn_bwd_noncausal -- the backward of attn_fwd_noncausal (no mask: every key contributes
 * to every query's gradient).  Inputs are that forward's q, k, v, o, lse and dout; outputs,
 * workspace (attn_bwd_workspace_size bytes), determinism and errors as attn_bwd.
 */
ea_status attn_bwd_noncausal(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, int B, int T, int Hq,
                             int Hkv, int D, float scale, ea_dtype dt, hipStream_t stream);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving or training loops, harnesses that forbid
 * hipMalloc.  Same arguments as attn_bwd minus the workspace, same kernels, same outputs
 * bitwise.  D_t goes to a static device array of EA_NOALLOC_SCRATCH_BYTES (16 MiB) that the
 * library holds on every device it runs on until the process ends; the call allocates and
 * frees nothing.  Limit: attn_bwd_workspace_size(B, T, Hq, Hkv, D, dt) must not exceed
 * EA_NOALLOC_SCRATCH_BYTES (B * Hq * T <= 4 Mi rows), else EA_ERR_SCRATCH before anything
 * is enqueued.  Every call on one device shares that device's array: calls that overlap in
 * time on one device (two streams, two host threads) race and must be serialised by the
 * caller.  The stream must belong to the current device.  Errors: as attn_bwd (no
 * workspace checks), EA_ERR_SCRATCH, and EA_ERR_HIP if the array's address cannot be found.
 */
#define EA_NOALLOC_SCRATCH_BYTES (16u << 20)
ea_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int B, int T, int Hq, int Hkv, int D, float scale, ea_dtype dt,
                           hipStream_t stream);

/*
 * The stages of attn_bwd, for callers that schedule them separately: attn_bwd is exactly
 * attn_bwd_preprocess followed by attn_bwd_main; attn_bwd_main computes what attn_bwd_dkdv
 * and attn_bwd_dq compute (in either order, or concurrently on two streams, once the
 * preprocess stage has completed) in a single launch.  All share attn_bwd's workspace and
 * sizes, and each validates its own arguments like attn_bwd.
 *  - attn_bwd_preprocess: D_t = sum_d dout * o for every (b, h, t) into the workspace
 *    (reads o and dout, writes only the workspace).
 *  - attn_bwd_main: dq, dk and dv (overwritten; dk, dv summed over each query-head group).
 *  - attn_bwd_dkdv: dk and dv only.
 *  - attn_bwd_dq: dq only.
 * The last three read the workspace written by the preprocess stage.
 */
ea_status attn_bwd_preprocess(const void* o, const void* dout, void* workspace,
                              size_t workspace_bytes, int B, int T, int Hq, int Hkv, int D,
                              ea_dtype dt, hipStream_t stream);
ea_status attn_bwd_main(const void* q, const void* k, const void* v, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, const void* workspace,
                        size_t workspace_bytes, int B, int T, int Hq, int Hkv, int D,
                        float scale, ea_dtype dt, hipStream_t stream);
ea_status attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                        const void* dout, void* dk, void* dv, const void* workspace,
                        size_t workspace_bytes, int B, int T, int Hq, int Hkv, int D,
                        float scale, ea_dtype dt, hipStream_t stream);
ea_status attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                      const void* dout, void* dq, const void* workspace, size_t workspace_bytes,
                      int B, int T, int Hq, int Hkv, int D, float scale, ea_dtype dt,
                      hipStream_t stream);

/*
 * The backward with the RoPE backward fused in.  The pages rotate queries and keys before the
 * attention ("Show HN: NanoEuler", section 2) and check RoPE's backward with the rest of the
 * model's gradients (section 4); the backward of the rotation is the rotation by -phi.
 * attn_bwd_rope takes the same inputs as attn_bwd (q and k are the rotated tensors that
 * attn_fwd received) and returns dq and dk with respect to the tensors BEFORE rope_apply,
 * i.e. what attn_bwd followed by rope_apply(inverse = 1) on dq and dk with the same base
 * and pos0 computes, but in one pass: the rotation is applied to the float32 gradients just
 * before they are rounded and stored (one rounding instead of two).  dv is unchanged.
 * The workspace (attn_bwd_rope_workspace_size bytes, 256-byte aligned) holds D_t as for
 * attn_bwd followed by a float32 (cos, sin) table [T, D/2, 2] of the rotation angles,
 * computed like rope_apply's.  Stages: attn_bwd_rope is attn_bwd_rope_preprocess (D_t and
 * the table) followed by attn_bwd_rope_main.  Errors: as attn_bwd, plus base <= 1 or not
 * finite, pos0 < 0 or pos0 + T > 2^31 (EA_ERR_INVALID_ARG).
 */
size_t attn_bwd_rope_workspace_size(int B, int T, int Hq, int Hkv, int D, ea_dtype dt);
ea_status attn_bwd_rope(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, int B, int T, int Hq, int Hkv,
                        int D, float scale, ea_dtype dt, double base, int pos0,
                        hipStream_t stream);
ea_status attn_bwd_rope_preprocess(const void* o, const void* dout, void* workspace,
                                   size_t workspace_bytes, int B, int T, int Hq, int Hkv, int D,
                                   ea_dtype dt, double base, int pos0, hipStream_t stream);
ea_status attn_bwd_rope_main(const void* q, const void* k, const void* v, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, const void* workspace,
                             size_t workspace_bytes, int B, int T, int Hq, int Hkv, int D,
                             float scale, ea_dtype dt, hipStream_t stream);

/*
 * The projections on either side of the attention: the query, key and value heads, RoPE on
 * queries and keys, no bias anywhere ("Show HN: NanoEuler", section 2); the attention result
 * projected back to the model dimension ("Tiny Hackable CUDA Language Model Implementation",
 * section 1); matrix products done by a matrix library beside the hand-written attention
 * ("Show HN: NanoEuler", section 4).  All products accumulate in float32 and round once
 * to dt.
 *
 * gemm -- C = op(A) op(B), row-major with leading dimensions (in elements).  op(A) is
 * [M, K]: A is stored [M, K] (trans_a = 0, lda >= K) or [K, M] (trans_a = 1, lda >= M).
 * op(B) is [K, N]: B is stored [K, N] (trans_b = 0, ldb >= N) or [N, K] (trans_b = 1,
 * ldb >= K).  C is [M, N], ldc >= N, overwritten.  The layer uses y = x W (0, 0),
 * dx = dy W^T (0, 1) and dW = x^T dy (1, 0) with W stored [in, out].
 * Errors: NULL pointer (EA_ERR_NULL); M, N, K < 1, a leading dimension too small, a flag
 * not 0/1 (EA_ERR_INVALID_ARG); unknown dt, trans_a = trans_b = 1, or a contiguous
 * dimension that is not a multiple of 16 bytes (N always; K when trans_a = 0 or
 * trans_b = 1; M when trans_a = 1) (EA_ERR_UNSUPPORTED); a pointer not 16-byte aligned or
 * a leading dimension not a multiple of 16 bytes (EA_ERR_ALIGN); C overlapping A or B
 * (EA_ERR_ALIAS).
 */
ea_status gemm(const void* a, const void* b, void* c, int M, int N, int K, int lda, int ldb,
               int ldc, int trans_a, int trans_b, ea_dtype dt, hipStream_t stream);

/*
 * gemm_ws -- gemm with a split of the K range.  A product with few output tiles and a long K
 * (a weight gradient dW = x^T dy: [C, C'] output, K = B T rows) leaves most of the chip idle
 * when each output tile is one workgroup; given a workspace, gemm_ws runs S slices of K per
 * tile (S from the shape: enough workgroups for two per compute unit, at least eight K
 * steps of the tile loop per slice, at most 8), each writing a float32 partial tile, and a
 * second launch sums
 * the S partials of every tile in slice order and rounds once to dt.  The result is
 * deterministic (the same bits on every call) but may differ from gemm's in the last place,
 * since the float32 sums are grouped differently.
 * gemm_workspace_size(M, N, K, trans_a, trans_b, dt) -- bytes of workspace for this shape
 * (0: no split for this shape, or an unsupported one; then gemm_ws is gemm and workspace may
 * be NULL).  workspace: 256-byte aligned, at least that many bytes, contents on entry don't
 * care, overwritten.  Errors: as gemm, plus workspace NULL (EA_ERR_NULL), misaligned
 * (EA_ERR_ALIGN), too small (EA_ERR_WORKSPACE) or overlapping A, B or C (EA_ERR_ALIAS), each
 * only when the size for the shape is not 0.
 */
size_t gemm_workspace_size(int M, int N, int K, int trans_a, int trans_b, ea_dtype dt);
ea_status gemm_ws(const void* a, const void* b, void* c, int M, int N, int K, int lda, int ldb,
                  int ldc, int trans_a, int trans_b, ea_dtype dt, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);

/*
 * qkv_proj -- the QKV projection of x [B, T, C] by w_qkv [C, (Hq + 2 Hkv) D] (row-major,
 * columns: the Hq query heads, then the Hkv key heads, then the Hkv value heads, D each):
 * q [B, T, Hq, D] = x Wq, k [B, T, Hkv, D] = x Wk, v [B, T, Hkv, D] = x Wv, in one launch.
 * With rope = 1, q and k are rotated in the epilogue exactly as rope_apply (base, pos0)
 * rotates them (angle in float64, reduced mod 2 pi, float32 sincos), from the float32 sums
 * before the single rounding: q and k are then what attn_fwd takes.
 * Errors: NULL pointer; B, T, C, Hq, Hkv < 1, Hq % Hkv != 0, D < 2, rope not 0/1, and with
 * rope base <= 1 or not finite, pos0 < 0 or pos0 + T > 2^31 (EA_ERR_INVALID_ARG); unknown
 * dt, C or D not a multiple of 16 bytes, D > 256 (EA_ERR_UNSUPPORTED); misalignment
 * (EA_ERR_ALIGN); an output overlapping an input or another output (EA_ERR_ALIAS).
 */
ea_status qkv_proj(const void* x, const void* w_qkv, void* q, void* k, void* v, int B, int T,
                   int C, int Hq, int Hkv, int D, ea_dtype dt, int rope, double base, int pos0,
                   hipStream_t stream);

/*
 * qkv_proj_bwd -- gradients of the QKV projection: with dq, dk, dv the gradients of the
 * projected q, k, v BEFORE RoPE (what attn_bwd_rope returns for q and k),
 * dx [B, T, C] = [dq | dk | dv] w_qkv^T and dw_qkv [C, (Hq + 2 Hkv) D] = x^T [dq | dk | dv],
 * both overwritten (two launches).  Sizes and errors as qkv_proj.
 */
ea_status qkv_proj_bwd(const void* x, const void* w_qkv, const void* dq, const void* dk,
                       const void* dv, void* dx, void* dw_qkv, int B, int T, int C, int Hq,
                       int Hkv, int D, ea_dtype dt, hipStream_t stream);

/*
 * qkv_proj_bwd_ws -- qkv_proj_bwd whose two products may split their K range as gemm_ws does
 * (in practice dw_qkv, whose K = B T is long and whose output has few tiles).  The workspace
 * (qkv_proj_bwd_workspace_size bytes, 256-byte aligned, may be NULL when that is 0) is shared
 * by the two launches, which run in order on the stream.  Results deterministic, and as
 * qkv_proj_bwd's up to float32 summation order; errors as qkv_proj_bwd plus gemm_ws's
 * workspace errors.
 */
size_t qkv_proj_bwd_workspace_size(int B, int T, int C, int Hq, int Hkv, int D, ea_dtype dt);
ea_status qkv_proj_bwd_ws(const void* x, const void* w_qkv, const void* dq, const void* dk,
                          const void* dv, void* dx, void* dw_qkv, int B, int T, int C, int Hq,
                          int Hkv, int D, ea_dtype dt, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* euler_attn_status_string(ea_status s);

/* Library version as major * 10000 + minor * 100 + patch. */
int euler_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EULER_ATTN_H */
