"""GPU parity of attn_fwd_rope, the forward with RoPE on Q and K fused in.

Per function: the oracle's forward on the oracle's rotation of the raw inputs
(oracle.forward_raw) against O and LSE, and oracle.rope of the raw q and k against the rotated
q_r and k_r the call returns.  Against the unfused path: k_r and q_r are rope_apply's output
bitwise (every kernel rotates a pair with the same fixed-order arithmetic, from the same
(cos, sin) values), and O / LSE equal attn_fwd on the returned q_r and k_r bitwise (the
kernel computes on exactly the rows it writes out).
"""
import numpy as np
import pytest
import torch

import causal_gqa_attention_fwd_amd as ea
from causal_gqa_attention_fwd_amd import workloads as W
from oracle import oracle

from _parity import check_fwd, f64, normwise, say

pytestmark = pytest.mark.gpu

CASES = [
    # dt, B, T, Hq, Hkv, D, base, pos0
    ("f32", 2, 65, 4, 2, 32, 1e4, 0),
    ("bf16", 2, 190, 12, 4, 64, 1e4, 0),     # three heads per group, ragged tail
    ("bf16", 1, 129, 8, 2, 128, 5e5, 7),     # head_dim 128, positions offset by 7
    ("bf16", 2, 300, 4, 4, 64, 1e4, 0),      # one head per group
    ("f32", 1, 100, 6, 3, 64, 1e4, 3),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_B%d_T%d_H%d-%d_D%d_p%d" % (c[:6] + (c[7],)))
def test_fwd_rope_parity(case):
    dt, B, T, Hq, Hkv, D, base, pos0 = case
    seed = 9100 + T + D + Hq
    say("[parity] attn_fwd_rope %s seed %d" % (case, seed))
    q = W.make_random((B, T, Hq, D), seed, dt).cuda()
    k = W.make_random((B, T, Hkv, D), seed + 1, dt).cuda()
    v = W.make_random((B, T, Hkv, D), seed + 2, dt).cuda()
    o, lse, qr, kr = ea.attn_fwd_rope(q, k, v, base=base, pos0=pos0)
    qr2, kr2 = ea.rope_apply_qk(q, k, base=base, pos0=pos0)
    o2, lse2 = ea.attn_fwd(qr, kr, v)
    torch.cuda.synchronize()
    assert torch.equal(kr, kr2)
    say("  q_r against rope_apply: normwise %.3g" % normwise(f64(qr), f64(qr2)))
    assert torch.equal(qr, qr2)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    # Oracle: rotation of the raw inputs, and attention on exactly the rotated rows the kernel used.
    qr_ref = oracle.rope(q.cpu(), base, pos0=pos0)
    kr_ref = oracle.rope(k.cpu(), base, pos0=pos0)
    tol = 2.0 ** -7 if dt == "bf16" else 1e-6
    for got, ref, n in ((qr, qr_ref, "q_r"), (kr, kr_ref, "k_r")):
        e = normwise(f64(got), ref)
        say("  %s against the oracle rotation: normwise %.3g" % (n, e))
        assert e <= tol, (n, e)
    o_ref, lse_ref = oracle.attn_fwd(qr.cpu(), kr.cpu(), v.cpu())
    check_fwd(dt, o, lse, o_ref, lse_ref, "attn_fwd_rope")
    assert np.all(np.isfinite(f64(o)))


def test_fwd_rope_feeds_the_fused_backward():
    # The step as bench.py runs it: attn_fwd_rope, then attn_bwd_rope on its q_r and k_r; the
    # gradients match the unfused chain (rope_apply_qk, attn_fwd, attn_bwd_rope) bitwise.
    w = W.WORKLOADS["blog_t1024"]
    say("[parity] attn_fwd_rope -> attn_bwd_rope, %s" % w.name)
    inp = W.make_inputs(w)
    q, k, v, do = (inp[n].cuda() for n in ("q_raw", "k_raw", "v", "dout"))
    o, lse, qr, kr = ea.attn_fwd_rope(q, k, v, base=w.base)
    g1 = ea.attn_bwd_rope(qr, kr, v, o, lse, do, base=w.base)
    qr2, kr2 = ea.rope_apply_qk(q, k, base=w.base)
    o2, lse2 = ea.attn_fwd(qr2, kr2, v)
    g2 = ea.attn_bwd_rope(qr2, kr2, v, o2, lse2, do, base=w.base)
    torch.cuda.synchronize()
    assert torch.equal(kr, kr2) and torch.equal(qr, qr2)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    for t in g1:
        assert bool(torch.isfinite(t).all())


# Forward shapes of large problems (more than 2048 32-row query blocks, so no key split):
# three heads per group as twelve 32-row waves (B=1, T=6144, 12/4 heads); one head per group
# with 64-row waves (QB = 2) in four-wave workgroups (544 of them); two heads per group with
# 64-row waves in eight-wave workgroups (576 of them).  Ragged tails in the last two.
BIG = [(1, 6144, 12, 4, 64), (2, 4160, 16, 16, 64), (4, 2112, 32, 16, 64)]


@pytest.mark.parametrize("case", BIG, ids=lambda c: "B%d_T%d_H%d-%d_D%d" % c)
def test_fwd_rope_large_problem_shapes(case):
    B, T, Hq, Hkv, D = case
    seed = 9300 + T + Hq
    say("[parity] attn_fwd_rope, large-problem forward shape %s seed %d" % (case, seed))
    q = W.make_random((B, T, Hq, D), seed, "bf16").cuda()
    k = W.make_random((B, T, Hkv, D), seed + 1, "bf16").cuda()
    v = W.make_random((B, T, Hkv, D), seed + 2, "bf16").cuda()
    o, lse, qr, kr = ea.attn_fwd_rope(q, k, v, base=1e4)
    qr2, kr2 = ea.rope_apply_qk(q, k, base=1e4)
    o2, lse2 = ea.attn_fwd(qr, kr, v)
    torch.cuda.synchronize()
    assert torch.equal(qr, qr2) and torch.equal(kr, kr2)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    # The oracle on the last (batch, K/V head) slice: rotation and attention.
    g = Hq // Hkv
    b, kv = B - 1, Hkv - 1
    hs = slice(kv * g, (kv + 1) * g)
    e = normwise(f64(qr[b:b + 1, :, hs]), oracle.rope(q[b:b + 1, :, hs].cpu(), 1e4))
    assert e <= 2.0 ** -7, e
    o_ref, lse_ref = oracle.attn_fwd(qr[b:b + 1, :, hs].cpu(), kr[b:b + 1, :, kv:kv + 1].cpu(),
                                     v[b:b + 1, :, kv:kv + 1].cpu())
    check_fwd("bf16", o[b:b + 1, :, hs], lse[b:b + 1, hs], o_ref, lse_ref, "fwd slice")
