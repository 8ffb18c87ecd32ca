"""Pins for the oracle's causal GQA attention forward (CPU only).

Definition (causal scaled dot-product attention with a causal mask, "Tiny Hackable CUDA
Language Model Implementation", section 1; query heads sharing K/V heads, "Show HN:
NanoEuler", section 2): S = scale * Q K^T for s <= t, P = softmax over s, O = P V,
LSE = log-sum-exp of the row.  Pins: an independent brute-force formulation, invariants,
closed forms and the PyTorch float64 library routine on the same inputs.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def brute_force(q, k, v, scale):
    """Second formulation: K/V copied per query head, the whole T x T matrix with -inf above
    the diagonal, normalisation without max subtraction (fine for tiny N(0,1) inputs)."""
    B, T, Hq, D = q.shape
    g = Hq // k.shape[2]
    kk = np.repeat(k, g, axis=2)
    vv = np.repeat(v, g, axis=2)
    o = np.zeros_like(q)
    lse = np.zeros((B, Hq, T))
    mask = np.triu(np.ones((T, T), bool), 1)
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, :, h, :] @ kk[b, :, h, :].T)
            s[mask] = -np.inf
            e = np.exp(s)
            z = e.sum(axis=1, keepdims=True)
            o[b, :, h, :] = (e / z) @ vv[b, :, h, :]
            lse[b, h, :] = np.log(z[:, 0])
    return o, lse


@pytest.mark.parametrize("B,T,Hq,Hkv,D", [(1, 1, 2, 1, 2), (2, 6, 2, 1, 4), (2, 5, 4, 2, 2),
                                          (1, 6, 4, 2, 4), (2, 3, 4, 4, 4)])
def test_brute_force_tiny(B, T, Hq, Hkv, D):
    q, k, v = _rand((B, T, Hq, D), 1), _rand((B, T, Hkv, D), 2), _rand((B, T, Hkv, D), 3)
    scale = 1 / math.sqrt(D)
    o, lse = oracle.attn_fwd(q, k, v, scale)
    o2, lse2 = brute_force(q, k, v, scale)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-13)


def test_probabilities_rows_sum_to_one_and_are_causal():
    # With V = identity (D >= T), O_t is the probability row P_t: it sums to 1, is zero
    # strictly above the diagonal and positive on and below it (diagonal included).
    T, D = 9, 12
    q, k = _rand((1, T, 2, D), 4), _rand((1, T, 1, D), 5)
    v = np.zeros((1, T, 1, D))
    for s in range(T):
        v[0, s, 0, s] = 1.0
    o, _ = oracle.attn_fwd(q, k, v)
    for h in range(2):
        P = o[0, :, h, :T]
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        assert np.all(P[np.triu_indices(T, 1)] == 0.0)
        assert np.all(P[np.tril_indices(T)] > 0.0)


def test_constant_v_returns_v():
    q, k = _rand((2, 17, 4, 8), 6), _rand((2, 17, 2, 8), 7)
    c = _rand((8,), 8)
    v = np.broadcast_to(c, (2, 17, 2, 8)).copy()
    o, _ = oracle.attn_fwd(q, k, v)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-14)


def test_causality_bitwise():
    B, T, Hq, Hkv, D = 1, 12, 4, 2, 8
    q, k, v = _rand((B, T, Hq, D), 9), _rand((B, T, Hkv, D), 10), _rand((B, T, Hkv, D), 11)
    o, lse = oracle.attn_fwd(q, k, v)
    for t in (0, 5, 10):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        q2[:, t + 1:] += 3.0
        k2[:, t + 1:] -= 2.0
        v2[:, t + 1:] *= -5.0
        o2, lse2 = oracle.attn_fwd(q2, k2, v2)
        np.testing.assert_array_equal(o2[:, :t + 1], o[:, :t + 1])
        np.testing.assert_array_equal(lse2[:, :, :t + 1], lse[:, :, :t + 1])
        assert not np.array_equal(o2[:, t + 1:], o[:, t + 1:])


def test_single_position():
    q, k, v = _rand((3, 1, 4, 16), 12), _rand((3, 1, 2, 16), 13), _rand((3, 1, 2, 16), 14)
    scale = 0.3
    o, lse = oracle.attn_fwd(q, k, v, scale)
    for h in range(4):
        np.testing.assert_allclose(o[:, 0, h], v[:, 0, h // 2], rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[:, h, 0], scale * np.sum(q[:, 0, h] * k[:, 0, h // 2], -1),
                                   rtol=0, atol=1e-14)


def test_constant_key_gives_running_mean():
    B, T, Hq, Hkv, D = 2, 20, 4, 2, 8
    q, v = _rand((B, T, Hq, D), 15), _rand((B, T, Hkv, D), 16)
    kvec = _rand((D,), 17)
    k = np.broadcast_to(kvec, (B, T, Hkv, D)).copy()
    scale = 1 / math.sqrt(D)
    o, lse = oracle.attn_fwd(q, k, v, scale)
    counts = np.arange(1, T + 1)[None, :, None, None]
    mean_v = np.cumsum(v, axis=1) / counts
    for h in range(Hq):
        np.testing.assert_allclose(o[:, :, h], mean_v[:, :, h // 2], rtol=0, atol=1e-13)
        expect = scale * (q[:, :, h] @ kvec) + np.log(np.arange(1, T + 1))[None]
        np.testing.assert_allclose(lse[:, h], expect, rtol=0, atol=1e-13)


def test_zero_query_lse_is_log_count():
    T = 31
    q = np.zeros((1, T, 2, 4))
    k, v = _rand((1, T, 1, 4), 18), _rand((1, T, 1, 4), 19)
    _, lse = oracle.attn_fwd(q, k, v)
    np.testing.assert_allclose(lse[0], np.log(np.arange(1, T + 1))[None].repeat(2, 0), rtol=0,
                               atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    B, T, Hq, Hkv, D = 2, 15, 6, 2, 8
    q, k, v = _rand((B, T, Hq, D), 20), _rand((B, T, Hkv, D), 21), _rand((B, T, Hkv, D), 22)
    o, lse = oracle.attn_fwd(q, k, v)
    o2, lse2 = oracle.attn_fwd(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2))
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-15)


def test_scale_argument_scales_scores():
    B, T, Hq, Hkv, D = 1, 10, 2, 1, 8
    q, k, v = _rand((B, T, Hq, D), 23), _rand((B, T, Hkv, D), 24), _rand((B, T, Hkv, D), 25)
    o1, l1 = oracle.attn_fwd(q, k, v, scale=0.7)
    o2, l2 = oracle.attn_fwd(2.0 * q, k, v, scale=0.35)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-14)


@pytest.mark.parametrize("B,T,Hq,Hkv,D", [(2, 37, 4, 2, 16), (1, 64, 12, 4, 8), (1, 33, 3, 1, 32)])
def test_torch_sdpa_float64(B, T, Hq, Hkv, D):
    q, k, v = _rand((B, T, Hq, D), 26), _rand((B, T, Hkv, D), 27), _rand((B, T, Hkv, D), 28)
    o, lse = oracle.attn_fwd(q, k, v)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                           enable_gqa=True)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-13)
    g = Hq // Hkv
    s = (tq @ tk.repeat_interleave(g, dim=1).transpose(-1, -2)) / math.sqrt(D)
    s = s.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-13)


def test_bad_head_counts_rejected():
    with pytest.raises(ValueError):
        oracle.attn_fwd(np.zeros((1, 2, 3, 4)), np.zeros((1, 2, 2, 4)), np.zeros((1, 2, 2, 4)))
