"""GPU parity of attn_decode (new query rows against a KV cache) with the oracle's
attn_fwd_kv on the same seeded inputs, through the C ABI.

Cases cover one and several new tokens, caches that fit one chunk (no merge), caches split
over a few chunks (one launch, merged in LDS: B2_Tq2_Tk100, B1_Tq4_Tk129, B1_Tq16_Tk777,
B2_Tq5_Tk2049, B1_Tq11_Tk300) and over many (merge launch: B3_Tq1_Tk1000, B4_Tq1_Tk4097),
row blocks of more than 16 rows for the bf16 16-row products (B1_Tq6_Tk300, B2_Tq8_Tk2000,
B1_Tq12_Tk700),
ragged cache lengths, every head_dim, both dtypes and several head groupings; the cache shape of a 32/8-head, head_dim-128 model at
8192 cached positions is run at full size.  With Tq = Tk the result must match attn_fwd.
"""
import numpy as np
import pytest
import torch

import causal_gqa_attention_fwd_amd as ea
from causal_gqa_attention_fwd_amd import workloads as W
from oracle import oracle

from _parity import check_fwd, f64, maxabs, normwise, say

pytestmark = pytest.mark.gpu

CASES = [  # B, Tq, Tk, Hq, Hkv, D, dtype
    (1, 1, 1, 4, 2, 64, "f32"), (2, 1, 5, 12, 4, 64, "bf16"), (1, 3, 31, 8, 1, 32, "f32"),
    (2, 2, 100, 12, 4, 64, "bf16"), (1, 4, 129, 4, 4, 128, "bf16"), (3, 1, 1000, 32, 8, 128, "bf16"),
    (1, 16, 777, 12, 4, 64, "f32"), (2, 5, 2049, 6, 2, 32, "bf16"), (1, 11, 300, 4, 1, 128, "f32"),
    (4, 1, 4097, 12, 4, 64, "bf16"),
    # bf16 head_dim 64 / 128 run 16-row products: more than 16 rows per block (18: a partly
    # filled second half; 32: both halves full, split launch; 36: a second row block).
    (1, 6, 300, 12, 4, 64, "bf16"), (2, 8, 2000, 16, 4, 128, "bf16"), (1, 12, 700, 12, 4, 64, "bf16"),
    # Chunks of an odd number of 32-key tiles (96 keys) in the single launch (the split launch
    # meets them at 4 x 4097 above).
    (1, 2, 330, 12, 4, 64, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_Tq%d_Tk%d_H%d-%d_D%d_%s" % c)
def test_decode_parity(case):
    B, Tq, Tk, Hq, Hkv, D, dt = case
    seed = 4400 + Tq * 13 + Tk + D
    say("[parity] attn_decode %s seed %d" % (case, seed))
    q = W.make_random((B, Tq, Hq, D), seed, dt).cuda()
    k = W.make_random((B, Tk, Hkv, D), seed + 1, dt).cuda()
    v = W.make_random((B, Tk, Hkv, D), seed + 2, dt).cuda()
    o, lse = ea.attn_decode(q, k, v)
    o2, lse2 = ea.attn_decode(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)  # chunks merged in a fixed order
    o_ref, lse_ref = oracle.attn_fwd_kv(q, k, v)
    check_fwd(dt, o, lse, o_ref, lse_ref, "decode")


def test_decode_cache_of_a_32_8_head_model_full_size():
    # One new token per sequence, 8 sequences, 8192 cached positions, 32/8 heads, head_dim 128.
    B, Tq, Tk, Hq, Hkv, D = 8, 1, 8192, 32, 8, 128
    say("[parity] attn_decode full size B=%d Tk=%d heads %d/%d D=%d" % (B, Tk, Hq, Hkv, D))
    q = W.make_random((B, Tq, Hq, D), 4501, "bf16").cuda()
    k = W.make_random((B, Tk, Hkv, D), 4502, "bf16").cuda()
    v = W.make_random((B, Tk, Hkv, D), 4503, "bf16").cuda()
    o, lse = ea.attn_decode(q, k, v)
    o2, lse2 = ea.attn_decode(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)  # deterministic
    o_ref, lse_ref = oracle.attn_fwd_kv(q, k, v)
    check_fwd("bf16", o, lse, o_ref, lse_ref, "decode full size")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_decode_with_whole_sequence_matches_attn_fwd(dt):
    B, T, Hq, Hkv, D = 2, 70, 12, 4, 64
    q = W.make_random((B, T, Hq, D), 4601, dt).cuda()
    k = W.make_random((B, T, Hkv, D), 4602, dt).cuda()
    v = W.make_random((B, T, Hkv, D), 4603, dt).cuda()
    o, lse = ea.attn_decode(q, k, v)
    o_f, lse_f = ea.attn_fwd(q, k, v)
    torch.cuda.synchronize()
    e_o = maxabs(f64(o), f64(o_f)) if dt == "bf16" else normwise(f64(o), f64(o_f))
    e_l = normwise(f64(lse), f64(lse_f))
    say("  decode vs attn_fwd (Tq = Tk): O %.3g, LSE %.3g" % (e_o, e_l))
    assert e_o <= (2e-2 if dt == "bf16" else 1e-5) and e_l <= 1e-5


def test_decode_sees_only_its_prefix():
    # Changing cache rows after a query's position leaves that query's output bitwise equal.
    B, Tq, Tk, Hq, Hkv, D = 1, 4, 300, 8, 2, 64
    q = W.make_random((B, Tq, Hq, D), 4701, "bf16").cuda()
    k = W.make_random((B, Tk, Hkv, D), 4702, "bf16").cuda()
    v = W.make_random((B, Tk, Hkv, D), 4703, "bf16").cuda()
    o, lse = ea.attn_decode(q, k, v)
    k2, v2 = k.clone(), v.clone()
    k2[:, Tk - 3:] = 3.0
    v2[:, Tk - 3:] = -2.0   # visible only to the last query row
    o2, lse2 = ea.attn_decode(q, k2, v2)
    torch.cuda.synchronize()
    assert torch.equal(o[:, 0], o2[:, 0]) and torch.equal(lse[:, :, 0], lse2[:, :, 0])
    assert not torch.equal(o[:, 3], o2[:, 3])
