"""GPU parity of attn_fwd_noncausal / attn_bwd_noncausal against the oracle's non-causal
attention (oracle.attn_fwd_nc / attn_bwd_nc): every query row sees every key row, the form of
the tiled forward the NanoEuler blog post prints ("Tiled FlashAttention").

Covered: the model workloads in full; the 8192-token workload at full size on the GPU with
the oracle on one (batch, K/V head) slice (this shape takes the 64-row-per-wave forward and
the two-launch backward); an edge sweep over ragged lengths, head dims, head groupings and
both dtypes (key-split forward, fused one-launch backward); agreement with the causal kernels
on the last row; run-to-run bitwise determinism of the backward.
"""
import pytest
import torch

import causal_gqa_attention_fwd_amd as ea
from causal_gqa_attention_fwd_amd import workloads as W
from oracle import oracle

from _parity import check_fwd, check_grads, f64, maxabs, say

pytestmark = pytest.mark.gpu


def _run(q, k, v, do):
    o, lse = ea.attn_fwd_noncausal(q, k, v)
    dq, dk, dv = ea.attn_bwd_noncausal(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def _check(dt, got, q, k, v, do, what):
    o, lse, dq, dk, dv = got
    o_ref, lse_ref = oracle.attn_fwd_nc(q, k, v)
    check_fwd(dt, o, lse, o_ref, lse_ref, what + " fwd")
    dq_ref, dk_ref, dv_ref = oracle.attn_bwd_nc(q, k, v, do)
    check_grads(dt, {"dq": dq, "dk": dk, "dv": dv}, {"dq": dq_ref, "dk": dk_ref, "dv": dv_ref}, what + " bwd")


@pytest.mark.parametrize("name", ["tiny_cpu_model", "gpu_model_f32", "gpu_model_bf16", "blog_t1024"])
def test_noncausal_workload(name):
    w = W.WORKLOADS[name]
    say("[parity] non-causal workload %s %s" % (name, w.describe()))
    inp = W.make_inputs(w)
    q, k, v, do = (inp[n].cuda() for n in ("q_raw", "k_raw", "v", "dout"))
    _check(w.dtype, _run(q, k, v, do), q, k, v, do, "noncausal")


def test_noncausal_full_size_sampled():
    w = W.WORKLOADS["long_t8192"]
    g = w.g
    b, kv = 1, 2
    say("[parity] non-causal workload long_t8192 (full size on GPU, oracle on slice b=%d kv=%d)" % (b, kv))
    inp = W.make_inputs(w)
    q, k, v, do = (inp[n].cuda() for n in ("q_raw", "k_raw", "v", "dout"))
    got = _run(q, k, v, do)
    for t in got:
        assert bool(torch.isfinite(t).all())
    hs = slice(kv * g, (kv + 1) * g)
    o, lse, dq, dk, dv = got
    sl = (o[b:b + 1, :, hs], lse[b:b + 1, hs], dq[b:b + 1, :, hs], dk[b:b + 1, :, kv:kv + 1],
          dv[b:b + 1, :, kv:kv + 1])
    _check(w.dtype, sl, q[b:b + 1, :, hs], k[b:b + 1, :, kv:kv + 1], v[b:b + 1, :, kv:kv + 1],
           do[b:b + 1, :, hs], "noncausal slice")


EDGE = [(1, 1, 1, 1, 32, "f32"), (2, 2, 4, 2, 64, "bf16"), (1, 17, 4, 1, 128, "bf16"),
        (2, 63, 12, 4, 64, "f32"), (1, 64, 4, 4, 32, "bf16"), (2, 65, 4, 2, 64, "bf16"),
        (1, 127, 8, 2, 128, "f32"), (1, 129, 12, 4, 64, "bf16"), (1, 1000, 4, 2, 64, "bf16"),
        (2, 300, 6, 3, 32, "f32"), (1, 257, 32, 8, 128, "bf16"), (3, 191, 12, 4, 32, "bf16")]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "B%d_T%d_H%d-%d_D%d_%s" % c)
def test_noncausal_edges(case):
    B, T, Hq, Hkv, D, dt = case
    seed = 8300 + T * 13 + D + Hq
    say("[parity] non-causal edge case %s seed %d" % (case, seed))
    q = W.make_random((B, T, Hq, D), seed, dt).cuda()
    k = W.make_random((B, T, Hkv, D), seed + 1, dt).cuda()
    v = W.make_random((B, T, Hkv, D), seed + 2, dt).cuda()
    do = W.make_random((B, T, Hq, D), seed + 3, dt).cuda()
    _check(dt, _run(q, k, v, do), q, k, v, do, "noncausal")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_last_row_matches_causal_and_deterministic(dt):
    B, T, Hq, Hkv, D = 2, 333, 12, 4, 64
    say("[parity] non-causal vs causal last row, dt=%s" % dt)
    q = W.make_random((B, T, Hq, D), 71, dt).cuda()
    k = W.make_random((B, T, Hkv, D), 72, dt).cuda()
    v = W.make_random((B, T, Hkv, D), 73, dt).cuda()
    do = W.make_random((B, T, Hq, D), 74, dt).cuda()
    o, lse, dq, dk, dv = _run(q, k, v, do)
    oc, lsec = ea.attn_fwd(q, k, v)
    torch.cuda.synchronize()
    eo = maxabs(f64(o[:, -1]), f64(oc[:, -1]))
    el = maxabs(f64(lse[:, :, -1]), f64(lsec[:, :, -1]))
    say("  last row: O maxabs %.3g, LSE maxabs %.3g" % (eo, el))
    assert eo <= (1e-6 if dt == "f32" else 2 ** -8) and el <= 1e-5
    assert maxabs(f64(o[:, 0]), f64(oc[:, 0])) > 1e-3   # the first row differs
    again = _run(q, k, v, do)
    for a, b in zip((o, lse, dq, dk, dv), again):
        assert torch.equal(a, b)
