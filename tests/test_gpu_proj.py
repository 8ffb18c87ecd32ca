"""GPU parity of the projection kernels (gemm, qkv_proj, qkv_proj_bwd) against the oracle's
float64 products, and of the whole attention layer (QKV projection with RoPE, attention,
output projection; then the backward through all three) against the oracle chain.

Tolerances (normwise, max|x - r| / max|r|): every product accumulates in float32 from
operands that are exact in the I/O dtype, so the float32 sum's error (below 1e-5 relative for
K <= 4096 here) is far below the final rounding.  bf16 outputs round once to 8 significant
bits, unit roundoff 2^-8: |x - r| <= 2^-8 |r| per element, gate 2^-8 + 1e-4 for the sum.
fp32 outputs: the float32 accumulation alone, gate 1e-5.
"""
import numpy as np
import pytest
import torch

import causal_gqa_attention_fwd_amd as ea
from causal_gqa_attention_fwd_amd import workloads as W
from oracle import oracle

from _parity import TOL, check_fwd, check_grads, f64, normwise, say

pytestmark = pytest.mark.gpu

GEMM_TOL = {"bf16": 2.0 ** -8 + 1e-4, "f32": 1e-5}


def _check(dt, got, ref, what):
    e = normwise(f64(got), ref)
    say("  %s: normwise %.3g" % (what, e))
    assert np.all(np.isfinite(f64(got)))
    assert e <= GEMM_TOL[dt], (what, e)


# The last shape takes the 128 x 128 tiles (306 of them with a K of 2088) with ragged M, N and
# K tails; the others the 64 x 64 tiles.
SHAPES = [(1, 8, 8), (37, 40, 24), (130, 136, 72), (257, 264, 1000), (512, 768, 768),
          (4096, 1280, 768), (2056, 2184, 2088)]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0)])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "M%d_N%d_K%d" % s)
def test_gemm(dt, ta, tb, shape):
    M, N, K = shape
    if ta == 1:
        M = (M + 7) // 8 * 8
    seed = 4000 + M + N + K + 10 * ta + 20 * tb
    say("[parity] gemm %s ta=%d tb=%d M=%d N=%d K=%d seed %d" % (dt, ta, tb, M, N, K, seed))
    a = W.make_random((K, M) if ta else (M, K), seed, dt).cuda()
    b = W.make_random((N, K) if tb else (K, N), seed + 1, dt).cuda()
    c = ea.gemm(a, b, trans_a=bool(ta), trans_b=bool(tb))
    torch.cuda.synchronize()
    _check(dt, c, oracle.gemm(a, b, ta, tb), "gemm")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gemm_leading_dimensions_and_repeat(dt):
    # Operands and result inside wider row-major buffers (ld > row length); the columns
    # beyond N of the result buffer are left untouched.
    M, N, K, pad = 100, 72, 136, 24
    say("[parity] gemm with leading dimensions, %s" % dt)
    abuf = W.make_random((M, K + pad), 77, dt).cuda()
    bbuf = W.make_random((K, N + pad), 78, dt).cuda()
    cbuf = torch.full((M, N + pad), 3.0, device="cuda", dtype=abuf.dtype)
    code = ea.EA_F32 if dt == "f32" else ea.EA_BF16
    st = ea.lib().gemm(abuf.data_ptr(), bbuf.data_ptr(), cbuf.data_ptr(), M, N, K, K + pad, N + pad,
                       N + pad, 0, 0, code, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    _check(dt, cbuf[:, :N], oracle.gemm(abuf[:, :K], bbuf[:, :N]), "gemm ld")
    assert bool((cbuf[:, N:] == 3.0).all())
    again = ea.gemm(abuf[:, :K].contiguous(), bbuf[:, :N].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(again, cbuf[:, :N])


# Split-K shapes: few output tiles and a long K.  (768, 768, 4096) and (768, 1280, 4096) are the
# weight gradients of the output and QKV projections at B T = 4096; the others reach the largest
# split (8 slices of one tile), ragged M and N tiles, and a ragged last K tile (K % 64 != 0)
# that falls in the last slice only.
SPLIT_SHAPES = [(768, 768, 4096, 1, 0), (768, 1280, 4096, 1, 0), (64, 64, 8192, 0, 0),
                (200, 136, 3000, 0, 1), (104, 72, 2056, 1, 0), (40, 24, 1064, 0, 0)]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "M%d_N%d_K%d_ta%d_tb%d" % s)
def test_gemm_split_k(dt, shape):
    M, N, K, ta, tb = shape
    code = ea.EA_F32 if dt == "f32" else ea.EA_BF16
    need = ea.lib().gemm_workspace_size(M, N, K, ta, tb, code)
    assert need > 0  # the split path is the one under test
    seed = 4300 + M + N + K
    say("[parity] gemm_ws %s M=%d N=%d K=%d ta=%d tb=%d seed %d, workspace %d B" % (dt, M, N, K, ta, tb, seed, need))
    a = W.make_random((K, M) if ta else (M, K), seed, dt).cuda()
    b = W.make_random((N, K) if tb else (K, N), seed + 1, dt).cuda()
    ws = torch.full((need,), 0x7F, device="cuda", dtype=torch.uint8)  # stale contents don't matter
    c = ea.gemm(a, b, trans_a=bool(ta), trans_b=bool(tb), workspace=ws)
    c2 = ea.gemm(a, b, trans_a=bool(ta), trans_b=bool(tb), split_k=True)
    torch.cuda.synchronize()
    _check(dt, c, oracle.gemm(a, b, ta, tb), "gemm_ws")
    assert torch.equal(c, c2)  # deterministic: the same bits from any workspace


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gemm_split_k_leading_dimensions(dt):
    # gemm_ws on operands and result inside wider buffers: the split path's partial and reduce
    # launches read and write through the leading dimensions; the columns beyond N stay.
    M, N, K, pad = 96, 80, 2048, 24
    code = ea.EA_F32 if dt == "f32" else ea.EA_BF16
    need = ea.lib().gemm_workspace_size(M, N, K, 1, 0, code)
    assert need > 0
    say("[parity] gemm_ws with leading dimensions, %s, workspace %d B" % (dt, need))
    abuf = W.make_random((K, M + pad), 91, dt).cuda()
    bbuf = W.make_random((K, N + pad), 92, dt).cuda()
    cbuf = torch.full((M, N + pad), 3.0, device="cuda", dtype=abuf.dtype)
    ws = torch.empty(need, device="cuda", dtype=torch.uint8)
    st = ea.lib().gemm_ws(abuf.data_ptr(), bbuf.data_ptr(), cbuf.data_ptr(), M, N, K, M + pad, N + pad,
                          N + pad, 1, 0, code, ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    _check(dt, cbuf[:, :N], oracle.gemm(abuf[:, :M], bbuf[:, :N], 1, 0), "gemm_ws ld")
    assert bool((cbuf[:, N:] == 3.0).all())
    again = ea.gemm(abuf[:, :M].contiguous(), bbuf[:, :N].contiguous(), trans_a=True, split_k=True)
    torch.cuda.synchronize()
    assert torch.equal(again, cbuf[:, :N])


@pytest.mark.parametrize("name", ["gpu_model_bf16", "blog_t1024", "gpu_model_f32"])
def test_qkv_proj_bwd_split_k(name):
    w = W.WORKLOADS[name]
    say("[parity] qkv_proj_bwd_ws workload %s" % name)
    inp = W.make_proj_inputs(w)
    x, wq = inp["x"].cuda(), inp["w_qkv"].cuda()
    dq = W.make_random((w.B, w.T, w.Hq, w.D), w.seed + 611, w.dtype).cuda()
    dk = W.make_random((w.B, w.T, w.Hkv, w.D), w.seed + 612, w.dtype).cuda()
    dv = W.make_random((w.B, w.T, w.Hkv, w.D), w.seed + 613, w.dtype).cuda()
    code = ea.EA_F32 if w.dtype == "f32" else ea.EA_BF16
    assert ea.lib().qkv_proj_bwd_workspace_size(w.B, w.T, w.Hq * w.D, w.Hq, w.Hkv, w.D, code) > 0
    dx, dw = ea.qkv_proj_bwd(x, wq, dq, dk, dv, split_k=True)
    dx0, _ = ea.qkv_proj_bwd(x, wq, dq, dk, dv)
    dx2, dw2 = ea.qkv_proj_bwd(x, wq, dq, dk, dv, split_k=True)
    torch.cuda.synchronize()
    rdx, rdw = oracle.qkv_proj_bwd(x, wq, dq, dk, dv)
    _check(w.dtype, dx, rdx, "dx")
    _check(w.dtype, dw, rdw, "dw_qkv (split K)")
    assert torch.equal(dx, dx0)  # dx has enough tiles and is not split
    assert torch.equal(dx, dx2) and torch.equal(dw, dw2)


# Short sequences where dx splits too (few rows, K = (Hq + 2 Hkv) D): its A operand is the three
# gradient tensors side by side along K; with head_dim 32 and Hq + Hkv odd a K tile straddles
# the dk / dv boundary inside the second slice.
@pytest.mark.parametrize("case", [(1, 64, 12, 4, 64, "bf16"), (1, 50, 18, 9, 32, "bf16"), (2, 40, 16, 8, 64, "f32")],
                         ids=lambda c: "B%d_T%d_H%d-%d_D%d_%s" % c)
def test_qkv_proj_bwd_split_k_edges(case):
    B, T, Hq, Hkv, D, dt = case
    C, N = Hq * D, (Hq + 2 * Hkv) * D
    code = ea.EA_F32 if dt == "f32" else ea.EA_BF16
    assert ea.lib().gemm_workspace_size(B * T, C, N, 0, 1, code) > 0  # the dx product splits
    seed = 4900 + T + Hq + D
    say("[parity] qkv_proj_bwd_ws edge case %s seed %d" % (case, seed))
    x = W.make_random((B, T, C), seed, dt).cuda()
    wq = W.make_random((C, N), seed + 1, dt, scale=C ** -0.5).cuda()
    dq = W.make_random((B, T, Hq, D), seed + 2, dt).cuda()
    dk = W.make_random((B, T, Hkv, D), seed + 3, dt).cuda()
    dv = W.make_random((B, T, Hkv, D), seed + 4, dt).cuda()
    dx, dw = ea.qkv_proj_bwd(x, wq, dq, dk, dv, split_k=True)
    dx2, dw2 = ea.qkv_proj_bwd(x, wq, dq, dk, dv, split_k=True)
    torch.cuda.synchronize()
    rdx, rdw = oracle.qkv_proj_bwd(x, wq, dq, dk, dv)
    _check(dt, dx, rdx, "dx (split K)")
    _check(dt, dw, rdw, "dw_qkv")
    assert torch.equal(dx, dx2) and torch.equal(dw, dw2)


@pytest.mark.parametrize("name,pos0", [("tiny_cpu_model", 0), ("gpu_model_f32", 5), ("gpu_model_bf16", 0),
                                       ("blog_t1024", 0)])
def test_qkv_proj(name, pos0):
    w = W.WORKLOADS[name]
    say("[parity] qkv_proj workload %s pos0 %d" % (name, pos0))
    inp = W.make_proj_inputs(w)
    x, wq = inp["x"].cuda(), inp["w_qkv"].cuda()
    for rope in (True, False):
        q, k, v = ea.qkv_proj(x, wq, w.Hq, w.Hkv, w.D, rope=rope, base=w.base, pos0=pos0)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.qkv_proj(x, wq, w.Hq, w.Hkv, w.D, rope_on=rope, base=w.base, pos0=pos0)
        for got, ref, n in ((q, rq, "q"), (k, rk, "k"), (v, rv, "v")):
            _check(w.dtype, got, ref, "%s rope=%d" % (n, rope))
    # One rounding (fused) against two (projection, then rope_apply).
    q0, k0, _ = ea.qkv_proj(x, wq, w.Hq, w.Hkv, w.D, rope=False)
    q1, k1, _ = ea.qkv_proj(x, wq, w.Hq, w.Hkv, w.D, rope=True, base=w.base, pos0=pos0)
    q2, k2 = ea.rope_apply_qk(q0, k0, base=w.base, pos0=pos0)
    torch.cuda.synchronize()
    for a, b in ((q1, q2), (k1, k2)):
        assert normwise(f64(a), f64(b)) <= (2.0 ** -7 if w.dtype == "bf16" else 1e-6)


@pytest.mark.parametrize("name", ["tiny_cpu_model", "gpu_model_f32", "gpu_model_bf16", "blog_t1024"])
def test_qkv_proj_bwd(name):
    w = W.WORKLOADS[name]
    say("[parity] qkv_proj_bwd workload %s" % name)
    inp = W.make_proj_inputs(w)
    x, wq = inp["x"].cuda(), inp["w_qkv"].cuda()
    dq = W.make_random((w.B, w.T, w.Hq, w.D), w.seed + 601, w.dtype).cuda()
    dk = W.make_random((w.B, w.T, w.Hkv, w.D), w.seed + 602, w.dtype).cuda()
    dv = W.make_random((w.B, w.T, w.Hkv, w.D), w.seed + 603, w.dtype).cuda()
    dx, dw = ea.qkv_proj_bwd(x, wq, dq, dk, dv)
    torch.cuda.synchronize()
    rdx, rdw = oracle.qkv_proj_bwd(x, wq, dq, dk, dv)
    _check(w.dtype, dx, rdx, "dx")
    _check(w.dtype, dw, rdw, "dw_qkv")


@pytest.mark.parametrize("case", [(1, 17, 4, 2, 32, "f32"), (2, 33, 4, 1, 64, "bf16"), (1, 5, 8, 2, 128, "bf16"),
                                  (3, 100, 6, 3, 32, "bf16")], ids=lambda c: "B%d_T%d_H%d-%d_D%d_%s" % c)
def test_qkv_proj_edges(case):
    B, T, Hq, Hkv, D, dt = case
    C = Hq * D
    seed = 4700 + T + D
    say("[parity] qkv_proj edge case %s seed %d" % (case, seed))
    x = W.make_random((B, T, C), seed, dt).cuda()
    wq = W.make_random((C, (Hq + 2 * Hkv) * D), seed + 1, dt, scale=C ** -0.5).cuda()
    q, k, v = ea.qkv_proj(x, wq, Hq, Hkv, D, rope=True, base=1e4, pos0=7)
    rq, rk, rv = oracle.qkv_proj(x, wq, Hq, Hkv, D, rope_on=True, base=1e4, pos0=7)
    dq, dk, dv = (W.make_random(t.shape, seed + 2 + i, dt).cuda() for i, t in enumerate((q, k, v)))
    dx, dw = ea.qkv_proj_bwd(x, wq, dq, dk, dv)
    torch.cuda.synchronize()
    for got, ref, n in ((q, rq, "q"), (k, rk, "k"), (v, rv, "v")):
        _check(dt, got, ref, n)
    rdx, rdw = oracle.qkv_proj_bwd(x, wq, dq, dk, dv)
    _check(dt, dx, rdx, "dx")
    _check(dt, dw, rdw, "dw")


@pytest.mark.parametrize("name", ["tiny_cpu_model", "gpu_model_bf16"])
def test_attention_layer_chain(name):
    """x -> qkv_proj (RoPE) -> attn_fwd -> y = o W_o; dy -> do = dy W_o^T, dW_o = o^T dy ->
    attn_bwd_rope -> qkv_proj_bwd, against the oracle on the same GPU intermediates."""
    w = W.WORKLOADS[name]
    say("[parity] attention layer chain, workload %s" % name)
    inp = W.make_proj_inputs(w)
    x, wq, wo, dy = (inp[n].cuda() for n in ("x", "w_qkv", "w_o", "dy"))
    B, T, Hq, D = w.B, w.T, w.Hq, w.D
    q, k, v = ea.qkv_proj(x, wq, w.Hq, w.Hkv, D, rope=True, base=w.base)
    o, lse = ea.attn_fwd(q, k, v)
    y = ea.gemm(o.view(B * T, Hq * D), wo)
    do = ea.gemm(dy.view(B * T, -1), wo, trans_b=True)
    dwo = ea.gemm(o.view(B * T, Hq * D), dy.view(B * T, -1), trans_a=True)
    dq, dk, dv = ea.attn_bwd_rope(q, k, v, o, lse, do.view(B, T, Hq, D), base=w.base)
    dx, dwq = ea.qkv_proj_bwd(x, wq, dq, dk, dv)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_proj(x, wq, w.Hq, w.Hkv, D, rope_on=True, base=w.base)
    for got, ref, n in ((q, rq, "q"), (k, rk, "k"), (v, rv, "v")):
        _check(w.dtype, got, ref, n)
    ro, rlse = oracle.attn_fwd(q, k, v)
    check_fwd(w.dtype, o, lse, ro, rlse, "attn")
    _check(w.dtype, y, oracle.gemm(o.view(B * T, -1), wo), "y")
    _check(w.dtype, do, oracle.gemm(dy.view(B * T, -1), wo, trans_b=True), "do")
    _check(w.dtype, dwo, oracle.gemm(o.view(B * T, -1), dy.view(B * T, -1), trans_a=True), "dW_o")
    g = oracle.attn_bwd(q, k, v, do.view(B, T, Hq, D))
    ref = {"dq": oracle.rope(g[0], w.base, inverse=True), "dk": oracle.rope(g[1], w.base, inverse=True), "dv": g[2]}
    check_grads(w.dtype, {"dq": dq, "dk": dk, "dv": dv}, ref, "attn bwd")
    rdx, rdw = oracle.qkv_proj_bwd(x, wq, dq, dk, dv)
    _check(w.dtype, dx, rdx, "dx")
    _check(w.dtype, dwq, rdw, "dW_qkv")
    if w.dtype == "f32":
        # End to end from the raw inputs: the oracle's own chain.
        rdo = oracle.gemm(f64(dy).reshape(B * T, -1), f64(wo), trans_b=True).reshape(B, T, Hq, D)
        g2 = oracle.attn_bwd(rq, rk, rv, rdo)
        e2e_dx, e2e_dw = oracle.qkv_proj_bwd(x, wq, oracle.rope(g2[0], w.base, inverse=True),
                                             oracle.rope(g2[1], w.base, inverse=True), g2[2])
        e = max(normwise(f64(dx), e2e_dx), normwise(f64(dwq), e2e_dw))
        say("  end-to-end dx/dW_qkv normwise %.3g" % e)
        assert e <= TOL["f32"]["grad"]
