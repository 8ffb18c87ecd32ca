"""The FLOP and byte counts behind bench.py's figures, pinned without the GPU.

The throughput the bench reports is (algorithmic FLOPs) / (time), with FLOPs counted on the
unmasked (query, key) pairs of causal attention: key s is visible to query t iff s <= t
("Tiny Hackable CUDA Language Model Implementation", section 1: a causal mask on the scaled
dot product).  Forward: two contractions over head_dim per visible pair (Q K^T and P V);
backward: five (S recomputed, dP, dV, dK, dQ).  These tests count the pairs and the
multiply-adds of those contractions by brute force on tiny shapes and compare them with the
closed forms the bench uses, then pin the closed forms at the benchmark shapes.
"""
from __future__ import annotations

import importlib.util
import os

import pytest

from causal_gqa_attention_fwd_amd.workloads import WORKLOADS, Workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def brute_pairs(B, T, Hq):
    n = 0
    for _b in range(B):
        for _h in range(Hq):
            for t in range(T):
                for s in range(T):
                    if s <= t:
                        n += 1
    return n


def brute_macs(B, T, Hq, D, products):
    """Multiply-adds of `products` contractions over head_dim, one per visible pair each."""
    macs = 0
    for _b in range(B):
        for _h in range(Hq):
            for t in range(T):
                for s in range(t + 1):
                    for _p in range(products):
                        for _d in range(D):
                            macs += 1
    return macs


@pytest.mark.parametrize("B,T,Hq,Hkv,D", [(1, 1, 1, 1, 2), (2, 5, 4, 2, 4), (1, 9, 3, 1, 8), (3, 7, 6, 3, 2)])
def test_pairs_and_flops_match_brute_force(B, T, Hq, Hkv, D):
    w = Workload("tiny", B, T, Hq, Hkv, D, "f32", 0)
    assert w.pairs == brute_pairs(B, T, Hq)
    assert w.flops_fwd() == 2 * brute_macs(B, T, Hq, D, 2)    # Q K^T, P V
    assert w.flops_bwd() == 2 * brute_macs(B, T, Hq, D, 5)    # S, dP, dV, dK, dQ
    assert w.flops_total() == w.flops_fwd() + w.flops_bwd()


def test_pairs_count_grows_with_the_mask_not_the_square():
    # Doubling T roughly quadruples the pairs, exactly (2T)(2T+1)/2 / (T(T+1)/2).
    w1 = Workload("a", 1, 100, 1, 1, 2, "f32", 0)
    w2 = Workload("b", 1, 200, 1, 1, 2, "f32", 0)
    assert w1.pairs == 5050 and w2.pairs == 20100


def test_benchmark_shapes_closed_forms():
    # pairs = B * Hq * T (T + 1) / 2; total FLOPs = 14 * D * pairs.
    expect = {
        "blog_t1024": (25_190_400, 22_570_598_400),
        "long_t8192": (805_404_672, 721_642_586_112),
        "gqa_t4096_d128": (2_148_007_936, 3_849_230_221_312),
        "gpu_model_bf16": (25_214_976, 22_592_618_496),
        "tiny_cpu_model": (132_096, 59_179_008),
    }
    for name, (pairs, total) in expect.items():
        w = WORKLOADS[name]
        assert w.pairs == pairs, name
        assert w.flops_total() == total, name


def test_bench_algorithmic_bytes_and_flops():
    bench = _bench()
    w = Workload("tiny", 2, 5, 4, 2, 8, "bf16", 0)
    a = bench.algorithmic(w)
    es = 2
    q = 2 * 5 * 4 * 8 * es       # Q, O, dO, dQ each
    k = 2 * 5 * 2 * 8 * es       # K, V, dK, dV each
    lse = 2 * 4 * 5 * 4          # fp32 [B, Hq, T]
    assert a["rope_qk"]["bytes"] == 2 * (q + k)                     # read and write Q and K
    assert a["attn_fwd"]["bytes"] == q + 2 * k + q + lse           # Q, K, V in; O, LSE out
    assert a["attn_fwd"]["flops"] == 4 * 8 * w.pairs
    assert a["attn_bwd_main"]["flops"] == 10 * 8 * w.pairs
    assert a["attn_bwd_main"]["executed_flops"] == 14 * 8 * w.pairs
    # Q, K, V, dO, LSE, D_t in; dQ, dK, dV out.
    assert a["attn_bwd_main"]["bytes"] == (q + 2 * k + q + 2 * lse) + (q + 2 * k)
