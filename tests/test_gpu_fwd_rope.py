"""GPU parity of attn_fwd_rope, the forward with RoPE on Q and K fused in.

Per function: the oracle's forward on the oracle's rotation of the raw inputs
(oracle.forward_raw) against O and LSE, and oracle.rope of the raw q and k against the rotated
q_r and k_r the call returns.  Against the unfused path: k_r is rope_apply's output bitwise
(the same rotation launch), q_r agrees with it to one bf16 rounding, and O / LSE equal
attn_fwd on the returned q_r and k_r bitwise (the kernel computes on exactly the rows it
writes out).
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
    eq = normwise(f64(qr), f64(qr2))
    say("  q_r against rope_apply: normwise %.3g (bitwise %s)" % (eq, bool(torch.equal(qr, qr2))))
    assert eq <= (2.0 ** -7 if dt == "bf16" else 1e-6)  # at most one rounding apart
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
    torch.cuda.synchronize()
    assert torch.equal(kr, kr2)
    if torch.equal(qr, qr2):
        g2 = ea.attn_bwd_rope(qr2, kr2, v, o2, lse2, do, base=w.base)
        torch.cuda.synchronize()
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)
    for t in g1:
        assert bool(torch.isfinite(t).all())
