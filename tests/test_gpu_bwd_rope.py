"""GPU parity of attn_bwd_rope, the backward with the RoPE backward fused in.

Per function: the oracle's backward on exactly the rotated tensors the kernel received,
followed by the oracle's inverse rotation (oracle.rope(..., inverse=True)), against the
fused kernel's dQ and dK; dV against the oracle's dV.  Also reported, and held to the fp32
gate: the end-to-end gradients from the raw inputs (oracle.grads_raw).  The fused result
must agree with the unfused composition (attn_bwd, then rope_apply(inverse)) to rounding,
with dV bitwise equal, and its two stages must compose to the one-call entry point bitwise.
"""
import numpy as np
import pytest
import torch

import causal_gqa_attention_fwd_amd as ea
from causal_gqa_attention_fwd_amd import workloads as W
from oracle import oracle

from _parity import TOL, check_grads, f64, gpu_forward_pipeline, normwise, say

pytestmark = pytest.mark.gpu


def oracle_fused(qr, kr, v, do, base, pos0=0):
    dq, dk, dv = oracle.attn_bwd(qr, kr, v, do)
    return {"dq": oracle.rope(dq, base, pos0=pos0, inverse=True),
            "dk": oracle.rope(dk, base, pos0=pos0, inverse=True), "dv": dv}


def check_against_unfused(dt, got, qr, kr, v, o, lse, do, base, pos0=0):
    dq2, dk2, dv2 = ea.attn_bwd(qr, kr, v, o, lse, do)
    dq2 = ea.rope_apply(dq2, base, pos0, inverse=True)
    dk2 = ea.rope_apply(dk2, base, pos0, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(got[2], dv2)
    # One rounding (fused) against two (unfused): within a bf16 half-ulp pair, or fp32 rounding.
    bound = 2.0 ** -7 if dt == "bf16" else 1e-6
    for a, b, n in ((got[0], dq2, "dq"), (got[1], dk2, "dk")):
        e = normwise(f64(a), f64(b))
        say("  fused vs unfused %s: normwise %.3g" % (n, e))
        assert e <= bound, (n, e)


@pytest.mark.parametrize("name", ["tiny_cpu_model", "gpu_model_f32", "gpu_model_bf16", "blog_t1024"])
def test_bwd_rope_workload(name):
    w = W.WORKLOADS[name]
    say("[parity] attn_bwd_rope workload %s %s" % (name, w.describe()))
    inp = W.make_inputs(w)
    q, k, v, qr, kr, o, lse = gpu_forward_pipeline(inp, w.base)
    do = inp["dout"].cuda()
    got = ea.attn_bwd_rope(qr, kr, v, o, lse, do, base=w.base)
    torch.cuda.synchronize()
    ref = oracle_fused(qr, kr, v, do, w.base)
    check_grads(w.dtype, dict(zip(("dq", "dk", "dv"), got)), ref, "bwd_rope")
    check_against_unfused(w.dtype, got, qr, kr, v, o, lse, do, w.base)
    gq, gk, gv = oracle.grads_raw(inp["q_raw"], inp["k_raw"], inp["v"], inp["dout"], w.base)
    e2e = {"dq_raw": normwise(f64(got[0]), gq), "dk_raw": normwise(f64(got[1]), gk),
           "dv": normwise(f64(got[2]), gv)}
    say("  end-to-end normwise: %s" % e2e)
    if w.dtype == "f32":
        assert max(e2e.values()) <= TOL["f32"]["grad"]


# Slices: an interior one, the first (0, 0) and the last (B-1, Hkv-1) of the launch grid.
@pytest.mark.parametrize("name,slices", [("long_t8192", [(1, 2), (0, 0), (1, 3)]),
                                         ("gqa_t4096_d128", [(5, 3), (0, 0), (7, 7)])])
def test_bwd_rope_full_size_sampled(name, slices):
    w = W.WORKLOADS[name]
    g = w.g
    say("[parity] attn_bwd_rope workload %s (full size on GPU, oracle on slices %s)" % (name, slices))
    inp = W.make_inputs(w)
    q, k, v, qr, kr, o, lse = gpu_forward_pipeline(inp, w.base)
    do = inp["dout"].cuda()
    dq, dk, dv = ea.attn_bwd_rope(qr, kr, v, o, lse, do, base=w.base)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    for b, kv in slices:
        say(" slice b=%d kv=%d" % (b, kv))
        hs = slice(kv * g, (kv + 1) * g)
        ref = oracle_fused(qr[b:b + 1, :, hs], kr[b:b + 1, :, kv:kv + 1], v[b:b + 1, :, kv:kv + 1],
                           do[b:b + 1, :, hs], w.base)
        check_grads(w.dtype, {"dq": dq[b:b + 1, :, hs], "dk": dk[b:b + 1, :, kv:kv + 1],
                              "dv": dv[b:b + 1, :, kv:kv + 1]}, ref, "bwd_rope slice b=%d kv=%d" % (b, kv))


EDGE = [(1, 1, 1, 1, 32, "f32", 0, 1e4), (2, 17, 4, 1, 64, "bf16", 3, 1e4),
        (1, 65, 4, 2, 128, "f32", 0, 5e5), (2, 129, 12, 4, 64, "bf16", 5000, 1e4),
        (1, 1000, 4, 4, 32, "bf16", 0, 1e4), (1, 127, 8, 2, 128, "bf16", 17, 5e5),
        (2, 63, 12, 4, 64, "f32", 1, 1e4), (1, 300, 4, 1, 32, "f32", 100000, 1e4)]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "B%d_T%d_H%d-%d_D%d_%s_p%d_b%g" % c)
def test_bwd_rope_edges(case):
    B, T, Hq, Hkv, D, dt, pos0, base = case
    seed = 9100 + T * 7 + D + Hq + pos0 % 97
    say("[parity] attn_bwd_rope edge case %s seed %d" % (case, seed))
    qr = W.make_random((B, T, Hq, D), seed, dt).cuda()
    kr = W.make_random((B, T, Hkv, D), seed + 1, dt).cuda()
    v = W.make_random((B, T, Hkv, D), seed + 2, dt).cuda()
    do = W.make_random((B, T, Hq, D), seed + 3, dt).cuda()
    o, lse = ea.attn_fwd(qr, kr, v)
    got = ea.attn_bwd_rope(qr, kr, v, o, lse, do, base=base, pos0=pos0)
    torch.cuda.synchronize()
    check_grads(dt, dict(zip(("dq", "dk", "dv"), got)), oracle_fused(qr, kr, v, do, base, pos0), "bwd_rope")
    check_against_unfused(dt, got, qr, kr, v, o, lse, do, base, pos0)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_bwd_rope_stages_compose_and_repeat(dt):
    B, T, Hq, Hkv, D = 2, 200, 12, 4, 64
    say("[parity] attn_bwd_rope stages dt=%s" % dt)
    qr = W.make_random((B, T, Hq, D), 61, dt).cuda()
    kr = W.make_random((B, T, Hkv, D), 62, dt).cuda()
    v = W.make_random((B, T, Hkv, D), 63, dt).cuda()
    do = W.make_random((B, T, Hq, D), 64, dt).cuda()
    o, lse = ea.attn_fwd(qr, kr, v)
    one = ea.attn_bwd_rope(qr, kr, v, o, lse, do, base=1e4, pos0=11)
    again = ea.attn_bwd_rope(qr, kr, v, o, lse, do, base=1e4, pos0=11)
    ws = torch.empty(ea.attn_bwd_rope_workspace_size(B, T, Hq, Hkv, D, qr.dtype), device="cuda",
                     dtype=torch.uint8)
    dq, dk, dv = torch.empty_like(qr), torch.empty_like(kr), torch.empty_like(v)
    ea.attn_bwd_rope_preprocess(o, do, ws, Hkv, base=1e4, pos0=11)
    ea.attn_bwd_rope_main(qr, kr, v, lse, do, ws, dq, dk, dv)
    torch.cuda.synchronize()
    for a, b, c in zip(one, again, (dq, dk, dv)):
        assert torch.equal(a, b) and torch.equal(a, c)
