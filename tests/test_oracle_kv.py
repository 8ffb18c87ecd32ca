"""Pins for the oracle's attention of Tq new query rows against a KV cache (CPU only).

Definition: the causal GQA attention of the pages ("Tiny Hackable CUDA Language Model
Implementation", section 1; "Show HN: NanoEuler", section 2 for shared K/V heads) evaluated
for the last Tq positions of a Tk-long sequence, as generation with a cache does ("Show HN:
NanoEuler", section 2, speculative decoding with the MTP heads; the chat REPL of its key
points): query row i sits at position Tk - Tq + i and sees the keys s <= Tk - Tq + i.
Pins: an independent brute-force formulation, the PyTorch float64 library routine with an
explicit mask, closed forms, causality, and the reduction to the last rows of the full
causal attention.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def brute_force(q, k, v, scale):
    """Second formulation: K/V copied per head, the full Tq x Tk matrix with -inf where
    s > Tk - Tq + i, normalisation without max subtraction (tiny N(0,1) inputs)."""
    B, Tq, Hq, D = q.shape
    Tk = k.shape[1]
    g = Hq // k.shape[2]
    kk = np.repeat(k, g, axis=2)
    vv = np.repeat(v, g, axis=2)
    o = np.zeros_like(q)
    lse = np.zeros((B, Hq, Tq))
    i = np.arange(Tq)[:, None]
    s_idx = np.arange(Tk)[None, :]
    masked = s_idx > (Tk - Tq) + i
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, :, h, :] @ kk[b, :, h, :].T)
            s[masked] = -np.inf
            e = np.exp(s)
            z = e.sum(axis=1, keepdims=True)
            o[b, :, h, :] = (e / z) @ vv[b, :, h, :]
            lse[b, h, :] = np.log(z[:, 0])
    return o, lse


@pytest.mark.parametrize("B,Tq,Tk,Hq,Hkv,D", [(1, 1, 1, 2, 1, 2), (2, 1, 6, 4, 2, 4), (1, 3, 5, 2, 1, 4),
                                              (2, 4, 4, 4, 2, 2), (1, 2, 7, 6, 3, 4)])
def test_brute_force(B, Tq, Tk, Hq, Hkv, D):
    q, k, v = _rand((B, Tq, Hq, D), 1), _rand((B, Tk, Hkv, D), 2), _rand((B, Tk, Hkv, D), 3)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attn_fwd_kv(q, k, v, scale)
    o2, lse2 = brute_force(q, k, v, scale)
    assert np.max(np.abs(o - o2)) < 1e-13 and np.max(np.abs(lse - lse2)) < 1e-13


@pytest.mark.parametrize("B,Tq,Tk,Hq,Hkv,D", [(2, 1, 37, 8, 2, 16), (1, 5, 40, 6, 2, 32), (2, 16, 16, 4, 4, 8)])
def test_torch_sdpa_with_mask(B, Tq, Tk, Hq, Hkv, D):
    q, k, v = _rand((B, Tq, Hq, D), 11), _rand((B, Tk, Hkv, D), 12), _rand((B, Tk, Hkv, D), 13)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attn_fwd_kv(q, k, v, scale)
    g = Hq // Hkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    allowed = torch.arange(Tk)[None, :] <= (Tk - Tq) + torch.arange(Tq)[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed, scale=scale)
    scores = (tq @ tk.transpose(-1, -2)) * scale
    ref_lse = torch.logsumexp(scores.masked_fill(~allowed, float("-inf")), dim=-1)
    assert np.max(np.abs(o - ref.permute(0, 2, 1, 3).numpy())) < 1e-12
    assert np.max(np.abs(lse - ref_lse.numpy())) < 1e-12


def test_single_query_sees_every_key_and_closed_forms():
    # Tq = 1: the query sits at the last position and sees all Tk keys.  Constant K = k:
    # O = mean of all V, LSE = scale q.k + ln Tk.  Q = 0: LSE_i = ln(Tk - Tq + i + 1) and O_i
    # = mean of the visible V rows.
    B, Tk, Hq, Hkv, D = 2, 23, 4, 2, 8
    scale = 0.3
    q = _rand((B, 1, Hq, D), 21)
    krow = _rand((D,), 22)
    k = np.broadcast_to(krow, (B, Tk, Hkv, D)).copy()
    v = _rand((B, Tk, Hkv, D), 23)
    o, lse = oracle.attn_fwd_kv(q, k, v, scale)
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        assert np.allclose(o[:, 0, h], v[:, :, kv].mean(axis=1), atol=1e-13)
        assert np.allclose(lse[:, h, 0], scale * (q[:, 0, h] @ krow) + math.log(Tk), atol=1e-12)
    Tq = 5
    q0 = np.zeros((B, Tq, Hq, D))
    k2 = _rand((B, Tk, Hkv, D), 24)
    o, lse = oracle.attn_fwd_kv(q0, k2, v, scale)
    for i in range(Tq):
        last = Tk - Tq + i
        assert np.allclose(lse[:, :, i], math.log(last + 1), atol=1e-13)
        for h in range(Hq):
            kv = h // (Hq // Hkv)
            assert np.allclose(o[:, i, h], v[:, :last + 1, kv].mean(axis=1), atol=1e-13)


def test_causality_bitwise():
    B, Tq, Tk, Hq, Hkv, D = 1, 4, 12, 4, 2, 8
    q, k, v = _rand((B, Tq, Hq, D), 31), _rand((B, Tk, Hkv, D), 32), _rand((B, Tk, Hkv, D), 33)
    o, lse = oracle.attn_fwd_kv(q, k, v)
    for i in range(Tq):
        last = Tk - Tq + i
        k2, v2 = k.copy(), v.copy()
        k2[:, last + 1:] += 5.0
        v2[:, last + 1:] -= 3.0
        o2, lse2 = oracle.attn_fwd_kv(q, k2, v2)
        assert np.array_equal(o2[:, i], o[:, i]) and np.array_equal(lse2[:, :, i], lse[:, :, i])
        if last + 1 < Tk:
            assert not np.array_equal(o2[:, -1], o[:, -1])


def test_last_rows_of_full_causal_attention():
    # The cache form is the full causal attention restricted to its last Tq query rows.
    B, T, Tq, Hq, Hkv, D = 2, 30, 7, 6, 2, 16
    qf, k, v = _rand((B, T, Hq, D), 41), _rand((B, T, Hkv, D), 42), _rand((B, T, Hkv, D), 43)
    o_full, lse_full = oracle.attn_fwd(qf, k, v)
    o, lse = oracle.attn_fwd_kv(qf[:, T - Tq:].copy(), k, v)
    assert np.max(np.abs(o - o_full[:, T - Tq:])) < 1e-14
    assert np.max(np.abs(lse - lse_full[:, :, T - Tq:])) < 1e-14


def test_rejects_more_queries_than_keys():
    with pytest.raises(ValueError):
        oracle.attn_fwd_kv(_rand((1, 5, 2, 4), 1), _rand((1, 4, 1, 4), 2), _rand((1, 4, 1, 4), 3))
