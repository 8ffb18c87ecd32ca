"""GPU invariants of the HIP path that hold at any size: causality (bitwise), the first row,
constant V, GQA = MHA with repeated K/V, run-to-run determinism of O, LSE, dK and dV, and
the gradient-causality of dK/dV.  Also: the backward's stages called separately equal
attn_bwd.  Also the full-size T=8192 shape's mathematical
properties, which do not need the oracle."""
import math

import numpy as np
import pytest
import torch

import causal_gqa_attention_fwd_amd as ea
from causal_gqa_attention_fwd_amd import workloads as W

from _parity import say

pytestmark = pytest.mark.gpu


def rnd(shape, seed, dt):
    return W.make_random(shape, seed, dt).cuda()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_causality_bitwise(dt, D):
    B, T, Hq, Hkv = 2, 200, 6, 2
    say("[inv] causality dt=%s D=%d" % (dt, D))
    q, k, v = rnd((B, T, Hq, D), 1, dt), rnd((B, T, Hkv, D), 2, dt), rnd((B, T, Hkv, D), 3, dt)
    o, lse = ea.attn_fwd(q, k, v)
    for t in (0, 63, 64, 150):
        q2, k2, v2 = q.clone(), k.clone(), v.clone()
        q2[:, t + 1:] += 1.0
        k2[:, t + 1:] *= -2.0
        v2[:, t + 1:] += 3.0
        o2, lse2 = ea.attn_fwd(q2, k2, v2)
        torch.cuda.synchronize()
        assert torch.equal(o2[:, :t + 1], o[:, :t + 1]), t
        assert torch.equal(lse2[:, :, :t + 1], lse[:, :, :t + 1]), t


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_first_row_is_v0_and_constant_v(dt):
    B, T, Hq, Hkv, D = 2, 130, 4, 2, 64
    say("[inv] row0 / constant V dt=%s" % dt)
    q, k, v = rnd((B, T, Hq, D), 4, dt), rnd((B, T, Hkv, D), 5, dt), rnd((B, T, Hkv, D), 6, dt)
    o, lse = ea.attn_fwd(q, k, v)
    torch.cuda.synchronize()
    for h in range(Hq):
        assert torch.equal(o[:, 0, h], v[:, 0, h // 2])
    c = rnd((D,), 7, dt)
    vc = c.expand(B, T, Hkv, D).contiguous()
    oc, _ = ea.attn_fwd(q, k, vc)
    torch.cuda.synchronize()
    err = (oc.double() - c.double()).abs().max().item()
    tol = 1e-5 if dt == "f32" else 2.0 ** -7 * c.double().abs().max().item()
    assert err <= tol, err


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gqa_equals_mha_with_repeated_kv(dt):
    B, T, Hq, Hkv, D = 2, 300, 12, 4, 64
    g = Hq // Hkv
    say("[inv] gqa vs mha dt=%s" % dt)
    q, k, v = rnd((B, T, Hq, D), 8, dt), rnd((B, T, Hkv, D), 9, dt), rnd((B, T, Hkv, D), 10, dt)
    do = rnd((B, T, Hq, D), 11, dt)
    kr = k.repeat_interleave(g, dim=2).contiguous()
    vr = v.repeat_interleave(g, dim=2).contiguous()
    o, lse = ea.attn_fwd(q, k, v)
    o2, lse2 = ea.attn_fwd(q, kr, vr)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do)
    dq2, dk2, dv2 = ea.attn_bwd(q, kr, vr, o2, lse2, do)
    torch.cuda.synchronize()
    assert torch.allclose(o.float(), o2.float(), rtol=0, atol=1e-6 if dt == "f32" else 1e-2)
    assert torch.allclose(lse, lse2, rtol=0, atol=1e-5)
    dk_sum = dk2.float().reshape(B, T, Hkv, g, D).sum(3)
    dv_sum = dv2.float().reshape(B, T, Hkv, g, D).sum(3)
    rel = lambda a, b: ((a - b).abs().max() / b.abs().max()).item()  # noqa: E731
    tol = 1e-5 if dt == "f32" else 2e-2
    assert rel(dk.float(), dk_sum) <= tol
    assert rel(dv.float(), dv_sum) <= tol
    assert rel(dq.float(), dq2.float()) <= tol


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_determinism(dt):
    B, T, Hq, Hkv, D = 2, 513, 12, 4, 64
    say("[inv] determinism dt=%s" % dt)
    q, k, v = rnd((B, T, Hq, D), 12, dt), rnd((B, T, Hkv, D), 13, dt), rnd((B, T, Hkv, D), 14, dt)
    do = rnd((B, T, Hq, D), 15, dt)
    o1, l1 = ea.attn_fwd(q, k, v)
    o2, l2 = ea.attn_fwd(q, k, v)
    g1 = ea.attn_bwd(q, k, v, o1, l1, do)
    g2 = ea.attn_bwd(q, k, v, o1, l1, do)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # The backward uses no atomics: dq, dk and dv are bitwise reproducible.
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gradient_causality(dt):
    B, T, Hq, Hkv, D = 1, 260, 4, 2, 64
    say("[inv] gradient causality dt=%s" % dt)
    q, k, v = rnd((B, T, Hq, D), 16, dt), rnd((B, T, Hkv, D), 17, dt), rnd((B, T, Hkv, D), 18, dt)
    do = rnd((B, T, Hq, D), 19, dt)
    o, lse = ea.attn_fwd(q, k, v)
    _, dk, dv = ea.attn_bwd(q, k, v, o, lse, do)
    s = 100
    q2, do2 = q.clone(), do.clone()
    q2[:, :s] += 0.5
    do2[:, :s] -= 1.0
    o2, lse2 = ea.attn_fwd(q2, k, v)
    _, dk2, dv2 = ea.attn_bwd(q2, k, v, o2, lse2, do2)
    torch.cuda.synchronize()
    assert torch.equal(dk2[:, s:], dk[:, s:])
    assert torch.equal(dv2[:, s:], dv[:, s:])


def test_long_context_properties():
    # T = 8192 with peaky keys: finite outputs and LSE_t >= max_s S_ts.
    w = W.WORKLOADS["long_t8192"]
    say("[inv] long-context properties %s" % w.describe())
    inp = W.make_inputs(w)
    q, k, v = inp["q_raw"].cuda(), inp["k_raw"].cuda(), inp["v"].cuda()
    do = inp["dout"].cuda()
    o, lse = ea.attn_fwd(q, k, v)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    # the last row's LSE is at least its max score (checked for one head in fp32 on the GPU)
    b, h, kvh = 1, 5, 5 // w.g
    s_last = (k[b, :, kvh].float() @ q[b, -1, h].float()) / math.sqrt(w.D)
    assert lse[b, h, -1].item() >= s_last.max().item() - 1e-3


@pytest.mark.parametrize("dt,shape", [("f32", (2, 190, 8, 2, 64)), ("bf16", (2, 190, 8, 2, 64)),
                                      ("bf16", (4, 2100, 12, 4, 64)), ("bf16", (4, 2100, 4, 4, 32)),
                                      ("bf16", (2, 2100, 16, 8, 128))],
                         ids=["f32-small", "bf16-small", "bf16-T2100-D64", "bf16-T2100-D32", "bf16-T2100-D128"])
def test_backward_stages_compose(dt, shape):
    # Small problems run both roles in one launch, the T=2100 ones (more than 512 64-key dK/dV
    # workgroups) as two launches with the separate dK/dV kernel: either way the stage entry
    # points must reproduce the one-call backward bitwise.
    B, T, Hq, Hkv, D = shape
    say("[inv] backward stages dt=%s shape=%s" % (dt, shape))
    q, k, v = rnd((B, T, Hq, D), 20, dt), rnd((B, T, Hkv, D), 21, dt), rnd((B, T, Hkv, D), 22, dt)
    do = rnd((B, T, Hq, D), 23, dt)
    o, lse = ea.attn_fwd(q, k, v)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do)
    ws = torch.empty(ea.attn_bwd_workspace_size(B, T, Hq, Hkv, D, q.dtype), device=q.device,
                     dtype=torch.uint8)
    dq2, dk2, dv2 = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    ea.attn_bwd_preprocess(o, do, ws, Hkv)
    ea.attn_bwd_dq(q, k, v, lse, do, ws, dq2)      # dq before dkdv: the order is free
    ea.attn_bwd_dkdv(q, k, v, lse, do, ws, dk2, dv2)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    dq3, dk3, dv3 = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    ea.attn_bwd_main(q, k, v, lse, do, ws, dq3, dk3, dv3)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq3) and torch.equal(dk, dk3) and torch.equal(dv, dv3)
