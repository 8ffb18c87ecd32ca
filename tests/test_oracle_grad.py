"""Pins for the oracle's analytic backward (CPU only).

The pages' own check for hand-written gradients is central finite differences in double
precision on every analytic gradient ("Show HN: NanoEuler", section 3, and its "make check";
the blog's FAQ gives eps = 1e-5).  That is done here on every element at small shapes (RoPE
included, so its backward is checked too) and on seeded coordinates at the 4-batch,
128-token, 4/2-head, head-dim-32 shape, plus gradient identities and PyTorch float64
autograd through its attention routine.

FD gate: normwise max|g_fd - g| / max|g| <= 1e-6 (central differences have truncation error
O(eps^2) ~ 1e-10 and round-off ~ 1e-11 |L| / |g| here; the pages' 1e-4 is met a fortiori).
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle

EPS = 1e-5
BASE = 10000.0


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def loss(q_raw, k_raw, v, dout, scale):
    o, _ = oracle.forward_raw(q_raw, k_raw, v, BASE, scale)
    return float(np.sum(o * dout))


def normwise(a, ref):
    return float(np.max(np.abs(a - ref)) / max(np.max(np.abs(ref)), 1e-300))


def fd_grad(fn, x, coords):
    g = np.zeros(len(coords))
    for n, c in enumerate(coords):
        old = x[c]
        x[c] = old + EPS
        lp = fn()
        x[c] = old - EPS
        lm = fn()
        x[c] = old
        g[n] = (lp - lm) / (2 * EPS)
    return g


@pytest.mark.parametrize("B,T,Hq,Hkv,D", [(1, 1, 2, 1, 4), (1, 5, 2, 1, 4), (2, 17, 4, 2, 8),
                                          (1, 33, 3, 1, 4)])
def test_fd_every_element(B, T, Hq, Hkv, D):
    q, k = _rand((B, T, Hq, D), 100 + T), _rand((B, T, Hkv, D), 200 + T)
    v, do = _rand((B, T, Hkv, D), 300 + T), _rand((B, T, Hq, D), 400 + T)
    scale = 1 / math.sqrt(D)
    dq, dk, dv = oracle.grads_raw(q, k, v, do, BASE, scale)
    fn = lambda: loss(q, k, v, do, scale)  # noqa: E731
    for x, g in ((q, dq), (k, dk), (v, dv)):
        coords = list(np.ndindex(x.shape))
        gfd = fd_grad(fn, x, coords).reshape(x.shape)
        assert normwise(g, gfd) <= 1e-6, normwise(g, gfd)


def test_fd_sampled_coordinates_tiny_cpu_model_shape():
    # 4 x 128 tokens, 4 Q / 2 KV heads, head_dim 32; 256 seeded coordinates per tensor.
    # A coordinate in (b, kv group) only affects that group's heads, so each perturbation
    # recomputes the loss on that (b, kv) slice alone (exact: other groups are constant).
    B, T, Hq, Hkv, D = 4, 128, 4, 2, 32
    g = Hq // Hkv
    q, k = _rand((B, T, Hq, D), 1), _rand((B, T, Hkv, D), 2)
    v, do = _rand((B, T, Hkv, D), 3), _rand((B, T, Hq, D), 4)
    scale = 1 / math.sqrt(D)
    dq, dk, dv = oracle.grads_raw(q, k, v, do, BASE, scale)
    rng = np.random.default_rng(7)
    for name, x, gx, H in (("q", q, dq, Hq), ("k", k, dk, Hkv), ("v", v, dv, Hkv)):
        coords = [tuple(int(rng.integers(0, n)) for n in x.shape) for _ in range(256)]
        got, want = [], []
        for c in coords:
            b = c[0]
            kv = c[2] // g if name == "q" else c[2]
            hs = slice(kv * g, (kv + 1) * g)

            def fn():
                return loss(q[b:b + 1, :, hs], k[b:b + 1, :, kv:kv + 1],
                            v[b:b + 1, :, kv:kv + 1], do[b:b + 1, :, hs], scale)
            got.append(gx[c])
            want.append(fd_grad(fn, x, [c])[0])
        got, want = np.array(got), np.array(want)
        assert normwise(got, want) <= 1e-6, (name, normwise(got, want))


def test_gradient_identities():
    B, T, Hq, Hkv, D = 2, 23, 6, 2, 8
    q, k = _rand((B, T, Hq, D), 31), _rand((B, T, Hkv, D), 32)
    v, do = _rand((B, T, Hkv, D), 33), _rand((B, T, Hq, D), 34)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do)
    # Softmax is shift-invariant along s, so the post-RoPE dK sums to zero over positions.
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, rtol=0, atol=1e-12)
    # Each probability row sums to one, so sum_s dV_s = sum over the group and t of dO_t.
    g = Hq // Hkv
    want = do.reshape(B, T, Hkv, g, D).sum(axis=(1, 3))
    np.testing.assert_allclose(dv.sum(axis=1), want, rtol=0, atol=1e-12)


def test_constant_v_has_no_q_or_k_gradient():
    B, T, Hq, Hkv, D = 1, 19, 4, 2, 8
    q, k, do = _rand((B, T, Hq, D), 41), _rand((B, T, Hkv, D), 42), _rand((B, T, Hq, D), 43)
    v = np.broadcast_to(_rand((D,), 44), (B, T, Hkv, D)).copy()
    dq, dk, _ = oracle.attn_bwd(q, k, v, do)
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13


def test_gradient_causality():
    # dK_s and dV_s only see queries t >= s: perturbing Q_t and dO_t for t < s leaves them
    # unchanged (bitwise).  dQ_t only depends on dO_t (other rows of dO do not enter).
    B, T, Hq, Hkv, D = 1, 14, 2, 1, 8
    q, k = _rand((B, T, Hq, D), 51), _rand((B, T, Hkv, D), 52)
    v, do = _rand((B, T, Hkv, D), 53), _rand((B, T, Hq, D), 54)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do)
    s = 6
    q2, do2 = q.copy(), do.copy()
    q2[:, :s] += 1.5
    do2[:, :s] -= 2.0
    _, dk2, dv2 = oracle.attn_bwd(q2, k, v, do2)
    np.testing.assert_array_equal(dk2[:, s:], dk[:, s:])
    np.testing.assert_array_equal(dv2[:, s:], dv[:, s:])
    do3 = do.copy()
    do3[:, 9] += 1.0
    dq3, _, _ = oracle.attn_bwd(q, k, v, do3)
    rows = [t for t in range(T) if t != 9]
    np.testing.assert_array_equal(dq3[:, rows], dq[:, rows])


def test_gqa_gradient_is_group_sum_of_mha():
    B, T, Hq, Hkv, D = 2, 11, 6, 2, 8
    g = Hq // Hkv
    q, k = _rand((B, T, Hq, D), 61), _rand((B, T, Hkv, D), 62)
    v, do = _rand((B, T, Hkv, D), 63), _rand((B, T, Hq, D), 64)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do)
    dq_m, dk_m, dv_m = oracle.attn_bwd(q, np.repeat(k, g, axis=2), np.repeat(v, g, axis=2), do)
    np.testing.assert_allclose(dq, dq_m, rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk, dk_m.reshape(B, T, Hkv, g, D).sum(axis=3), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, dv_m.reshape(B, T, Hkv, g, D).sum(axis=3), rtol=0, atol=1e-13)


@pytest.mark.parametrize("B,T,Hq,Hkv,D", [(2, 29, 4, 2, 16), (1, 48, 12, 4, 8)])
def test_torch_autograd_float64(B, T, Hq, Hkv, D):
    q, k = _rand((B, T, Hq, D), 71), _rand((B, T, Hkv, D), 72)
    v, do = _rand((B, T, Hkv, D), 73), _rand((B, T, Hq, D), 74)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do)
    tq, tk, tv = (torch.from_numpy(a).permute(0, 2, 1, 3).clone().requires_grad_(True)
                  for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)
    o.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, t.grad.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)
