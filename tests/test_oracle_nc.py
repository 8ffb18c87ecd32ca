"""Pins for the oracle's non-causal attention, forward and backward (CPU only).

Definition: the per-head attention the blog prints beside its tiled FlashAttention
("NanoEuler" blog, "Tiled FlashAttention": every query row of a head is scored against every
key row, softmax over all of them, then the weighted sum of V), with the grouped K/V heads of
"Show HN: NanoEuler", section 2.  Pins: an independent brute-force formulation, the PyTorch
float64 library routine (forward, and its autograd for the gradients), closed forms,
invariants that hold only without a mask (key-permutation invariance; the sum of dK over the
key rows vanishes; the sum of dV is the sum of dO), agreement with the causal oracle on the
last row, and central finite differences.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _qkv(B, T, Hq, Hkv, D, seed):
    return _rand((B, T, Hq, D), seed), _rand((B, T, Hkv, D), seed + 1), _rand((B, T, Hkv, D), seed + 2)


def brute_force(q, k, v, scale):
    """Second formulation: K/V copied per head, the full T x T matrix, normalisation without
    max subtraction (tiny N(0,1) inputs)."""
    B, T, Hq, D = q.shape
    g = Hq // k.shape[2]
    kk = np.repeat(k, g, axis=2)
    vv = np.repeat(v, g, axis=2)
    o = np.zeros_like(q)
    lse = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            e = np.exp(scale * (q[b, :, h, :] @ kk[b, :, h, :].T))
            z = e.sum(axis=1, keepdims=True)
            o[b, :, h, :] = (e / z) @ vv[b, :, h, :]
            lse[b, h, :] = np.log(z[:, 0])
    return o, lse


def _torch_ref(q, k, v, scale):
    """(O, LSE) from torch's float64 SDPA without a mask, GQA by repeating K/V heads."""
    g = q.shape[2] // k.shape[2]
    tq = q.permute(0, 2, 1, 3)
    tk = k.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    tv = v.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=False, scale=scale)
    lse = torch.logsumexp((tq @ tk.transpose(-1, -2)) * scale, dim=-1)
    return o.permute(0, 2, 1, 3), lse


@pytest.mark.parametrize("B,T,Hq,Hkv,D", [(1, 1, 1, 1, 2), (2, 5, 4, 2, 4), (1, 7, 6, 3, 4), (2, 3, 2, 2, 8)])
def test_brute_force(B, T, Hq, Hkv, D):
    q, k, v = _qkv(B, T, Hq, Hkv, D, 100 + T)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attn_fwd_nc(q, k, v, scale)
    o2, lse2 = brute_force(q, k, v, scale)
    assert np.max(np.abs(o - o2)) < 1e-13 and np.max(np.abs(lse - lse2)) < 1e-13


@pytest.mark.parametrize("B,T,Hq,Hkv,D", [(2, 37, 8, 2, 16), (1, 40, 6, 2, 32), (2, 16, 4, 4, 8)])
def test_torch_sdpa(B, T, Hq, Hkv, D):
    q, k, v = _qkv(B, T, Hq, Hkv, D, 200 + T)
    scale = 0.7 / math.sqrt(D)
    o, lse = oracle.attn_fwd_nc(q, k, v, scale)
    ro, rlse = _torch_ref(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale)
    assert np.max(np.abs(o - ro.numpy())) < 1e-12
    assert np.max(np.abs(lse - rlse.numpy())) < 1e-12


def test_closed_forms():
    # Constant K = k: every row is the plain mean of all T value rows, LSE = scale q.k + ln T.
    # Q = 0: LSE = ln T for every row.
    B, T, Hq, Hkv, D = 2, 23, 4, 2, 8
    scale = 0.3
    q = _rand((B, T, Hq, D), 21)
    krow = _rand((D,), 22)
    k = np.broadcast_to(krow, (B, T, Hkv, D)).copy()
    v = _rand((B, T, Hkv, D), 23)
    o, lse = oracle.attn_fwd_nc(q, k, v, scale)
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        for t in range(T):
            assert np.allclose(o[:, t, h], v[:, :, kv].mean(axis=1), atol=1e-13)
        assert np.allclose(lse[:, h, :], scale * (q[:, :, h] @ krow) + math.log(T), atol=1e-12)
    _, lse0 = oracle.attn_fwd_nc(np.zeros_like(q), _rand((B, T, Hkv, D), 24), v, scale)
    assert np.allclose(lse0, math.log(T), atol=1e-13)


def test_every_row_sees_the_last_key_and_key_order_is_irrelevant():
    B, T, Hq, Hkv, D = 1, 12, 4, 2, 8
    q, k, v = _qkv(B, T, Hq, Hkv, D, 31)
    o, lse = oracle.attn_fwd_nc(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[:, -1] += 5.0
    v2[:, -1] -= 3.0
    o2, _ = oracle.attn_fwd_nc(q, k2, v2)
    assert np.all(np.abs(o2[:, 0] - o[:, 0]) > 0)     # the first row sees the last key
    perm = np.random.default_rng(5).permutation(T)
    o3, lse3 = oracle.attn_fwd_nc(q, k[:, perm], v[:, perm])
    assert np.max(np.abs(o3 - o)) < 1e-13 and np.max(np.abs(lse3 - lse)) < 1e-13


def test_last_row_and_single_row_match_causal():
    # The last query row sees every key under either mask; with T = 1 the forms coincide.
    B, T, Hq, Hkv, D = 2, 19, 6, 2, 16
    q, k, v = _qkv(B, T, Hq, Hkv, D, 41)
    o, lse = oracle.attn_fwd_nc(q, k, v)
    oc, lsec = oracle.attn_fwd(q, k, v)
    assert np.max(np.abs(o[:, -1] - oc[:, -1])) < 1e-14
    assert np.max(np.abs(lse[:, :, -1] - lsec[:, :, -1])) < 1e-14
    assert np.max(np.abs(o[:, 0] - oc[:, 0])) > 1e-3
    q1, k1, v1 = q[:, :1].copy(), k[:, :1].copy(), v[:, :1].copy()
    g_nc = oracle.attn_bwd_nc(q1, k1, v1, q1)
    g_c = oracle.attn_bwd(q1, k1, v1, q1)
    for a, b in zip(g_nc, g_c):
        assert np.max(np.abs(a - b)) < 1e-15


@pytest.mark.parametrize("B,T,Hq,Hkv,D", [(2, 9, 4, 2, 8), (1, 33, 6, 3, 16), (1, 20, 2, 2, 4)])
def test_grads_vs_torch_autograd(B, T, Hq, Hkv, D):
    q, k, v = _qkv(B, T, Hq, Hkv, D, 300 + T)
    do = _rand((B, T, Hq, D), 399)
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv = oracle.attn_bwd_nc(q, k, v, do, scale)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    ro, _ = _torch_ref(tq, tk, tv, scale)
    (ro * torch.from_numpy(do)).sum().backward()
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(a - t.grad.numpy())) < 1e-12


def test_grad_invariants():
    # Softmax rows sum to one, so sum_s dS_ts = 0: the dK rows of each head sum to zero, and
    # the dV rows sum to the group's sum of dO rows.
    B, T, Hq, Hkv, D = 2, 21, 6, 2, 8
    q, k, v = _qkv(B, T, Hq, Hkv, D, 51)
    do = _rand((B, T, Hq, D), 54)
    dq, dk, dv = oracle.attn_bwd_nc(q, k, v, do, 0.4)
    g = Hq // Hkv
    for kv in range(Hkv):
        assert np.max(np.abs(dk[:, :, kv].sum(axis=1))) < 1e-12
        assert np.max(np.abs(dv[:, :, kv].sum(axis=1) - do[:, :, kv * g:(kv + 1) * g].sum(axis=(1, 2)))) < 1e-12
    assert np.max(np.abs(dq)) > 1e-3


def test_grads_finite_differences():
    B, T, Hq, Hkv, D = 1, 6, 4, 2, 4
    q, k, v = _qkv(B, T, Hq, Hkv, D, 61)
    do = _rand((B, T, Hq, D), 64)
    scale = 0.5
    grads = oracle.attn_bwd_nc(q, k, v, do, scale)
    eps = 1e-5

    def loss(qq, kk, vv):
        return float(np.sum(oracle.attn_fwd_nc(qq, kk, vv, scale)[0] * do))

    for which, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.max(np.abs(num - grads[which])) < 1e-8, which


def test_rejects_bad_heads():
    with pytest.raises(ValueError):
        oracle.attn_fwd_nc(_rand((1, 4, 3, 4), 1), _rand((1, 4, 2, 4), 2), _rand((1, 4, 2, 4), 3))
