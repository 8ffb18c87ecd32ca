"""GPU parity: the HIP path (through the C ABI) against the double-precision oracle on the
same seeded inputs.

Per function: rope_apply against oracle.rope on the raw inputs; attn_fwd and attn_bwd
against oracle.attn_fwd / oracle.attn_bwd on exactly the post-RoPE tensors the kernels
received; the inverse rope_apply on the gradients against oracle.rope(inverse=True).
Workloads: the small and T=1024 shapes in full; the T=8192 and T=4096/head-dim-128 shapes at
full size on the GPU (the launch configuration the benchmark times), checked on whole
(batch, K/V head) slices that the oracle computes exactly.  Then an edge sweep of ragged
lengths, head dims, head groupings and both dtypes.
"""
import math

import numpy as np
import pytest
import torch

import causal_gqa_attention_fwd_amd as ea
from causal_gqa_attention_fwd_amd import workloads as W
from oracle import oracle

from _parity import check_fwd, check_grads, f64, gpu_forward_pipeline, maxabs, normwise, say

pytestmark = pytest.mark.gpu


def check_rope(dt, got, x_ref_input, base, what, pos0=0, inverse=False):
    ref = oracle.rope(x_ref_input, base, pos0=pos0, inverse=inverse)
    y = f64(got)
    err = np.abs(y - ref)
    if dt == "f32":
        bound = 4e-6 * np.max(np.abs(ref)) + 0 * ref
    else:
        bound = 2.0 ** -8 * np.abs(ref) + 4e-6 * np.max(np.abs(ref))
    worst = float(np.max(err - bound))
    say("  %s: rope maxabs %.3g (margin %.3g)" % (what, float(np.max(err)), -worst))
    assert worst <= 0, (what, worst)


@pytest.mark.parametrize("name", ["tiny_cpu_model", "gpu_model_f32", "gpu_model_bf16", "blog_t1024"])
def test_workload_full(name):
    w = W.WORKLOADS[name]
    say("[parity] workload %s %s" % (name, w.describe()))
    inp = W.make_inputs(w)
    q, k, v, qr, kr, o, lse = gpu_forward_pipeline(inp, w.base)
    torch.cuda.synchronize()
    check_rope(w.dtype, qr, inp["q_raw"], w.base, "q")
    check_rope(w.dtype, kr, inp["k_raw"], w.base, "k")
    o_ref, lse_ref = oracle.attn_fwd(qr, kr, v)
    check_fwd(w.dtype, o, lse, o_ref, lse_ref, "fwd")
    do = inp["dout"].cuda()
    dq, dk, dv = ea.attn_bwd(qr, kr, v, o, lse, do)
    torch.cuda.synchronize()
    dq_ref, dk_ref, dv_ref = oracle.attn_bwd(qr, kr, v, do)
    check_grads(w.dtype, {"dq": dq, "dk": dk, "dv": dv}, {"dq": dq_ref, "dk": dk_ref, "dv": dv_ref}, "bwd")
    dq_raw = ea.rope_apply(dq, w.base, inverse=True)
    dk_raw = ea.rope_apply(dk, w.base, inverse=True)
    torch.cuda.synchronize()
    check_rope(w.dtype, dq_raw, dq, w.base, "dq inverse", inverse=True)
    check_rope(w.dtype, dk_raw, dk, w.base, "dk inverse", inverse=True)
    # End to end from the raw inputs (reported; the fp32 path is also held to its gate).
    gq, gk, gv = oracle.grads_raw(inp["q_raw"], inp["k_raw"], inp["v"], inp["dout"], w.base)
    e2e = {"dq_raw": normwise(f64(dq_raw), gq), "dk_raw": normwise(f64(dk_raw), gk),
           "dv": normwise(f64(dv), gv)}
    say("  end-to-end normwise: %s" % e2e)
    if w.dtype == "f32":
        assert max(e2e.values()) <= 1e-3


# Slices: an interior one, the first (0, 0) and the last (B-1, Hkv-1) of the launch grid.
@pytest.mark.parametrize("name,slices", [("long_t8192", [(1, 2), (0, 0), (1, 3)]),
                                         ("gqa_t4096_d128", [(5, 3), (0, 0), (7, 7)])])
def test_workload_full_size_sampled(name, slices):
    w = W.WORKLOADS[name]
    g = w.g
    say("[parity] workload %s (full size on GPU, oracle on slices %s)" % (name, slices))
    inp = W.make_inputs(w)
    q, k, v, qr, kr, o, lse = gpu_forward_pipeline(inp, w.base)
    do = inp["dout"].cuda()
    dq, dk, dv = ea.attn_bwd(qr, kr, v, o, lse, do)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    for b, kv in slices:
        hs = slice(kv * g, (kv + 1) * g)
        say(" slice b=%d kv=%d" % (b, kv))
        check_rope(w.dtype, qr[b:b + 1], inp["q_raw"][b:b + 1], w.base, "q[b]")
        check_rope(w.dtype, kr[b:b + 1], inp["k_raw"][b:b + 1], w.base, "k[b]")
        sq, sk, sv, sdo = (qr[b:b + 1, :, hs], kr[b:b + 1, :, kv:kv + 1], v[b:b + 1, :, kv:kv + 1],
                           do[b:b + 1, :, hs])
        o_ref, lse_ref = oracle.attn_fwd(sq, sk, sv)
        check_fwd(w.dtype, o[b:b + 1, :, hs], lse[b:b + 1, hs], o_ref, lse_ref, "fwd slice")
        dq_ref, dk_ref, dv_ref = oracle.attn_bwd(sq, sk, sv, sdo)
        check_grads(w.dtype, {"dq": dq[b:b + 1, :, hs], "dk": dk[b:b + 1, :, kv:kv + 1],
                              "dv": dv[b:b + 1, :, kv:kv + 1]},
                    {"dq": dq_ref, "dk": dk_ref, "dv": dv_ref}, "bwd slice")


def _edge_cases():
    Ts = [1, 2, 3, 17, 63, 65, 127, 129, 1000]
    Ds = [32, 64, 128]
    heads = [(1, 1), (4, 1), (4, 2), (4, 4), (12, 4)]
    cases = []
    n = 0
    for T in Ts:
        for D in Ds:
            for dt in ("f32", "bf16"):
                hq, hkv = heads[n % len(heads)]
                B = 1 + (n % 2)
                if T == 1000 and (hq, hkv) != (12, 4):
                    hq, hkv = (4, 2)
                cases.append((B, T, hq, hkv, D, dt))
                n += 1
    return cases


EDGE = _edge_cases()


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "B%d_T%d_H%d-%d_D%d_%s" % c)
def test_edge_sweep(case):
    B, T, Hq, Hkv, D, dt = case
    seed = 7000 + T * 31 + D + Hq * 3 + Hkv
    say("[parity] edge case %s seed %d" % (case, seed))
    q = W.make_random((B, T, Hq, D), seed, dt).cuda()
    k = W.make_random((B, T, Hkv, D), seed + 1, dt).cuda()
    v = W.make_random((B, T, Hkv, D), seed + 2, dt).cuda()
    do = W.make_random((B, T, Hq, D), seed + 3, dt).cuda()
    o, lse = ea.attn_fwd(q, k, v)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(q, k, v)
    check_fwd(dt, o, lse, o_ref, lse_ref, "fwd")
    dq_ref, dk_ref, dv_ref = oracle.attn_bwd(q, k, v, do)
    check_grads(dt, {"dq": dq, "dk": dk, "dv": dv}, {"dq": dq_ref, "dk": dk_ref, "dv": dv_ref}, "bwd")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("D,H,T,base,pos0", [(32, 3, 33, 1e4, 0), (64, 12, 129, 1e4, 7),
                                             (128, 8, 70, 5e5, 4000), (8, 1, 5, 1e4, 0),
                                             (256, 2, 9, 1e4, 1),
                                             # head dims that are not whole 16-byte chunks
                                             # (pair by pair), and 12 (chunks for fp32 only)
                                             (2, 3, 9, 1e4, 0), (6, 5, 17, 1e4, 3),
                                             (10, 2, 40, 5e5, 100), (12, 4, 33, 1e4, 0),
                                             (254, 1, 6, 1e4, 2)])
def test_rope_variants(dt, D, H, T, base, pos0):
    say("[parity] rope dt=%s D=%d H=%d T=%d base=%g pos0=%d" % (dt, D, H, T, base, pos0))
    x = W.make_random((2, T, H, D), 99 + D + T, dt).cuda()
    y = ea.rope_apply(x, base, pos0)
    yi = ea.rope_apply(x, base, pos0, inverse=True)
    torch.cuda.synchronize()
    check_rope(dt, y, x, base, "fwd", pos0=pos0)
    check_rope(dt, yi, x, base, "inv", pos0=pos0, inverse=True)
    # in place
    z = x.clone()
    ea.rope_apply(z, base, pos0, out=z)
    torch.cuda.synchronize()
    assert torch.equal(z, y)


@pytest.mark.parametrize("D", [64, 6])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rope_qk_one_launch(dt, D):
    # The two-tensor launch equals two single-tensor launches bitwise, and the oracle; D = 6
    # takes the pair-by-pair kernel.
    say("[parity] rope_apply_qk dt=%s D=%d" % (dt, D))
    q = W.make_random((2, 77, 12, D), 501, dt).cuda()
    k = W.make_random((2, 77, 4, D), 502, dt).cuda()
    for inverse in (False, True):
        qo, ko = ea.rope_apply_qk(q, k, 10000.0, pos0=3, inverse=inverse)
        q1 = ea.rope_apply(q, 10000.0, pos0=3, inverse=inverse)
        k1 = ea.rope_apply(k, 10000.0, pos0=3, inverse=inverse)
        torch.cuda.synchronize()
        assert torch.equal(qo, q1) and torch.equal(ko, k1)
        check_rope(dt, qo, q, 10000.0, "q", pos0=3, inverse=inverse)
        check_rope(dt, ko, k, 10000.0, "k", pos0=3, inverse=inverse)
    # in place on both
    q2, k2 = q.clone(), k.clone()
    ea.rope_apply_qk(q2, k2, 10000.0, q_out=q2, k_out=k2)
    qo, ko = ea.rope_apply_qk(q, k, 10000.0)
    torch.cuda.synchronize()
    assert torch.equal(q2, qo) and torch.equal(k2, ko)


@pytest.mark.parametrize("case", [(16, 512, 12, 4, 32), (4, 1500, 18, 3, 64), (2, 2100, 12, 4, 64)],
                         ids=lambda c: "B%d_T%d_H%d-%d_D%d" % c)
def test_forward_three_head_workgroups(case):
    # bf16 problems with more than 2048 query blocks and three heads per K/V group take the
    # 12-wave forward workgroups (four 32-row waves per head); g = 6 also groups three heads.
    B, T, Hq, Hkv, D = case
    seed = 7700 + T + D + Hq
    say("[parity] forward, three heads per workgroup, %s seed %d" % (case, seed))
    q = W.make_random((B, T, Hq, D), seed, "bf16").cuda()
    k = W.make_random((B, T, Hkv, D), seed + 1, "bf16").cuda()
    v = W.make_random((B, T, Hkv, D), seed + 2, "bf16").cuda()
    o, lse = ea.attn_fwd(q, k, v)
    torch.cuda.synchronize()
    b, kv = B - 1, Hkv - 1
    g = Hq // Hkv
    hs = slice(kv * g, (kv + 1) * g)
    o_ref, lse_ref = oracle.attn_fwd(q[b:b + 1, :, hs], k[b:b + 1, :, kv:kv + 1], v[b:b + 1, :, kv:kv + 1])
    check_fwd("bf16", o[b:b + 1, :, hs], lse[b:b + 1, hs], o_ref, lse_ref, "fwd slice")


@pytest.mark.parametrize("case", [(16, 1100, 12, 4, 32), (8, 2100, 12, 4, 64), (6, 1500, 24, 4, 64)],
                         ids=lambda c: "B%d_T%d_H%d-%d_D%d" % c)
def test_backward_three_head_workgroups(case):
    # bf16 problems whose dQ launch runs alone with at least 512 workgroups of 128 query rows
    # and three heads per workgroup take the 12-wave dQ workgroups; g = 6 takes two of them
    # per K/V head.  Ragged query tails in every case.
    B, T, Hq, Hkv, D = case
    seed = 7800 + T + D + Hq
    say("[parity] backward, three heads per dQ workgroup, %s seed %d" % (case, seed))
    q = W.make_random((B, T, Hq, D), seed, "bf16").cuda()
    k = W.make_random((B, T, Hkv, D), seed + 1, "bf16").cuda()
    v = W.make_random((B, T, Hkv, D), seed + 2, "bf16").cuda()
    do = W.make_random((B, T, Hq, D), seed + 3, "bf16").cuda()
    o, lse = ea.attn_fwd(q, k, v)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do)
    again = ea.attn_bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    for t, t2 in zip((dq, dk, dv), again):
        assert bool(torch.isfinite(t).all())
        assert torch.equal(t, t2)  # two launches, no atomics: bitwise reproducible
    g = Hq // Hkv
    for b, kv in ((B - 1, Hkv - 1), (0, 1)):
        hs = slice(kv * g, (kv + 1) * g)
        sq, sk, sv, sdo = (q[b:b + 1, :, hs], k[b:b + 1, :, kv:kv + 1], v[b:b + 1, :, kv:kv + 1],
                           do[b:b + 1, :, hs])
        dq_ref, dk_ref, dv_ref = oracle.attn_bwd(sq, sk, sv, sdo)
        check_grads("bf16", {"dq": dq[b:b + 1, :, hs], "dk": dk[b:b + 1, :, kv:kv + 1],
                             "dv": dv[b:b + 1, :, kv:kv + 1]},
                    {"dq": dq_ref, "dk": dk_ref, "dv": dv_ref}, "bwd slice b=%d kv=%d" % (b, kv))


@pytest.mark.parametrize("case", [(4, 2100, 12, 4, 64), (2, 2100, 16, 8, 64), (4, 2100, 4, 4, 32),
                                  (72, 50, 24, 8, 64), (40, 100, 16, 16, 32), (2, 2100, 16, 8, 128)],
                         ids=lambda c: "B%d_T%d_H%d-%d_D%d" % c)
def test_backward_separate_launches(case):
    # bf16 problems with more than 512 (64-key) dK/dV workgroups run the two backward roles as
    # two launches: the separate dK/dV kernel, then the dQ-only kernel with six (three heads x
    # two), eight (two heads x four) and four (one head x four) 32-row waves.  Ragged tails in
    # every case; two are shorter than one 128-key tile (keys and query rows past the end
    # inside the only tile).  Head_dim 128 takes the four-wave 64-key dK/dV kernel.
    B, T, Hq, Hkv, D = case
    seed = 7900 + T + D + Hq
    say("[parity] backward as two launches, %s seed %d" % (case, seed))
    q = W.make_random((B, T, Hq, D), seed, "bf16").cuda()
    k = W.make_random((B, T, Hkv, D), seed + 1, "bf16").cuda()
    v = W.make_random((B, T, Hkv, D), seed + 2, "bf16").cuda()
    do = W.make_random((B, T, Hq, D), seed + 3, "bf16").cuda()
    o, lse = ea.attn_fwd(q, k, v)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    g = Hq // Hkv
    for b, kv in ((B - 1, Hkv - 1), (0, 0)):
        hs = slice(kv * g, (kv + 1) * g)
        sq, sk, sv, sdo = (q[b:b + 1, :, hs], k[b:b + 1, :, kv:kv + 1], v[b:b + 1, :, kv:kv + 1],
                           do[b:b + 1, :, hs])
        dq_ref, dk_ref, dv_ref = oracle.attn_bwd(sq, sk, sv, sdo)
        check_grads("bf16", {"dq": dq[b:b + 1, :, hs], "dk": dk[b:b + 1, :, kv:kv + 1],
                             "dv": dv[b:b + 1, :, kv:kv + 1]},
                    {"dq": dq_ref, "dk": dk_ref, "dv": dv_ref}, "bwd slice b=%d kv=%d" % (b, kv))
