"""attn_bwd_noalloc on the GPU, through the C ABI: the backward with its D_t scratch in the
library's static per-device array instead of a caller workspace.  Its outputs must equal
attn_bwd's (same kernels, same arithmetic) bitwise, on two calls in a row where the second is
smaller than the first (the scratch keeps the first call's contents), and agree with the
oracle on the same inputs within the parity tolerances.  The call must not allocate device
memory: torch's allocator statistics and the device's free memory are unchanged by it (after
a first call on the device, which loads the code object holding the static array)."""
import pytest
import torch

import causal_gqa_attention_fwd_amd as ea
from causal_gqa_attention_fwd_amd import workloads as W
from oracle import oracle

from _parity import check_grads, say

pytestmark = pytest.mark.gpu


def _inputs(B, T, Hq, Hkv, D, dt, seed):
    q = W.make_random((B, T, Hq, D), seed, dt).cuda()
    k = W.make_random((B, T, Hkv, D), seed + 1, dt).cuda()
    v = W.make_random((B, T, Hkv, D), seed + 2, dt).cuda()
    do = W.make_random((B, T, Hq, D), seed + 3, dt).cuda()
    o, lse = ea.attn_fwd(q, k, v)
    torch.cuda.synchronize()
    return q, k, v, o, lse, do


# The first call is the larger one; the second (smaller, other dtype and head_dim) reads a
# scratch that still holds the first call's D_t past its own rows.
CALLS = [(4, 1024, 12, 4, 64, "bf16", 8101), (1, 77, 4, 2, 32, "f32", 8102)]


def test_noalloc_matches_attn_bwd_twice():
    # First use on this device: the library looks up (and the runtime loads) the static array.
    q, k, v, o, lse, do = _inputs(1, 16, 2, 1, 32, "bf16", 8100)
    ea.attn_bwd_noalloc(q, k, v, o, lse, do, torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    torch.cuda.synchronize()
    outs = []
    for (B, T, Hq, Hkv, D, dt, seed) in CALLS:
        say("[noalloc] B=%d T=%d Hq=%d Hkv=%d D=%d %s seed %d" % (B, T, Hq, Hkv, D, dt, seed))
        q, k, v, o, lse, do = _inputs(B, T, Hq, Hkv, D, dt, seed)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        torch.cuda.synchronize()
        stats0 = torch.cuda.memory_stats()
        free0, _ = torch.cuda.mem_get_info()
        ea.attn_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv)
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        stats1 = torch.cuda.memory_stats()
        assert stats1.get("allocation.all.allocated", 0) == stats0.get("allocation.all.allocated", 0)
        assert free1 == free0, (free0, free1)
        ref = ea.attn_bwd(q, k, v, o, lse, do)
        torch.cuda.synchronize()
        for a, b, n in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
            assert torch.equal(a, b), n
        # The oracle on the last (batch, K/V head) slice.
        g = Hq // Hkv
        b, kv = B - 1, Hkv - 1
        hs = slice(kv * g, (kv + 1) * g)
        dq_r, dk_r, dv_r = oracle.attn_bwd(q[b:b + 1, :, hs], k[b:b + 1, :, kv:kv + 1],
                                           v[b:b + 1, :, kv:kv + 1], do[b:b + 1, :, hs])
        check_grads(dt, {"dq": dq[b:b + 1, :, hs], "dk": dk[b:b + 1, :, kv:kv + 1],
                         "dv": dv[b:b + 1, :, kv:kv + 1]}, {"dq": dq_r, "dk": dk_r, "dv": dv_r},
                    "noalloc slice")
        outs.append((dq, dk, dv))
    for t in outs[0] + outs[1]:
        assert bool(torch.isfinite(t).all())


def test_noalloc_rejects_a_problem_beyond_the_scratch():
    # D_t of B * Hq * T rows must fit 16 MiB; one position more than 4 Mi rows is refused
    # before anything is enqueued, with real (small) tensors whose sizes are not read.
    q, k, v, o, lse, do = _inputs(1, 8, 2, 1, 32, "bf16", 8103)
    L = ea.lib()
    st = L.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            do.data_ptr(), 1 << 40, 2 << 40, 3 << 40, 64, 1025, 64, 64, 32, 0.125,
                            ea.EA_BF16, None)
    assert ea.STATUS[st] == "EA_ERR_SCRATCH"
