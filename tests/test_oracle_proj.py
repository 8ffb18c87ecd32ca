"""Pins for the oracle's projections (CPU only): gemm, qkv_proj, qkv_proj_bwd.

Definitions: the matrix products on either side of the attention ("Show HN: NanoEuler",
sections 2 and 4; "Tiny Hackable CUDA Language Model Implementation", section 1: the
attention result is projected back to the model dimension) and the RoPE of the pages on the
projected queries and keys.  Pins: explicit triple-loop sums (a formulation that shares
nothing with numpy's matmul), closed forms with identity and selector weights, the
norm-preserving rotation, and central finite differences of a scalar loss through the whole
projection (RoPE included) for the backward.
"""
import numpy as np
import pytest

from oracle import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def loops(a, b, trans_a, trans_b):
    """C[i][j] = sum_k op(A)[i][k] op(B)[k][j], element by element."""
    M = a.shape[1] if trans_a else a.shape[0]
    K = a.shape[0] if trans_a else a.shape[1]
    N = b.shape[0] if trans_b else b.shape[1]
    c = np.zeros((M, N))
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                av = a[k, i] if trans_a else a[i, k]
                bv = b[j, k] if trans_b else b[k, j]
                s += av * bv
            c[i, j] = s
    return c


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (6, 4, 9)])
def test_gemm_loops(ta, tb, M, N, K):
    a = _rand((K, M) if ta else (M, K), 10 + M)
    b = _rand((N, K) if tb else (K, N), 20 + N)
    assert np.max(np.abs(oracle.gemm(a, b, ta, tb) - loops(a, b, ta, tb))) < 1e-12


def test_gemm_identity_and_selector():
    a = _rand((5, 6), 1)
    assert np.array_equal(oracle.gemm(a, np.eye(6)), a)
    assert np.array_equal(oracle.gemm(np.eye(6), a, trans_b=True), a.T)
    sel = np.zeros((6, 2))
    sel[4, 0] = 1.0
    sel[1, 1] = -2.0
    c = oracle.gemm(a, sel)
    assert np.array_equal(c[:, 0], a[:, 4]) and np.array_equal(c[:, 1], -2.0 * a[:, 1])


def _qkv_loops(x, w, Hq, Hkv, D):
    """Per-head projections written as explicit sums."""
    B, T, C = x.shape
    q = np.zeros((B, T, Hq, D))
    k = np.zeros((B, T, Hkv, D))
    v = np.zeros((B, T, Hkv, D))
    for b in range(B):
        for t in range(T):
            for h in range(Hq):
                for d in range(D):
                    q[b, t, h, d] = sum(x[b, t, c] * w[c, h * D + d] for c in range(C))
            for h in range(Hkv):
                for d in range(D):
                    k[b, t, h, d] = sum(x[b, t, c] * w[c, (Hq + h) * D + d] for c in range(C))
                    v[b, t, h, d] = sum(x[b, t, c] * w[c, (Hq + Hkv + h) * D + d] for c in range(C))
    return q, k, v


def test_qkv_proj_loops_without_rope():
    B, T, C, Hq, Hkv, D = 2, 3, 5, 4, 2, 2
    x = _rand((B, T, C), 31)
    w = _rand((C, (Hq + 2 * Hkv) * D), 32)
    got = oracle.qkv_proj(x, w, Hq, Hkv, D, rope_on=False)
    for a, b in zip(got, _qkv_loops(x, w, Hq, Hkv, D)):
        assert np.max(np.abs(a - b)) < 1e-12


def test_qkv_proj_identity_weights_reduce_to_rope():
    # C = Hq D, Wq = I, Wk = the first Hkv D columns of I, Wv = 2 I (first Hkv D columns):
    # q = rope(x as heads), k = rope(x's first Hkv heads), v = 2 x's first Hkv heads.
    B, T, Hq, Hkv, D = 2, 7, 4, 2, 8
    C = Hq * D
    x = _rand((B, T, C), 41)
    w = np.concatenate([np.eye(C), np.eye(C)[:, :Hkv * D], 2.0 * np.eye(C)[:, :Hkv * D]], axis=1)
    q, k, v = oracle.qkv_proj(x, w, Hq, Hkv, D, rope_on=True, base=500.0, pos0=3)
    xh = x.reshape(B, T, Hq, D)
    assert np.array_equal(q, oracle.rope(xh, 500.0, pos0=3))
    assert np.array_equal(k, oracle.rope(np.ascontiguousarray(xh[:, :, :Hkv]), 500.0, pos0=3))
    assert np.array_equal(v, 2.0 * xh[:, :, :Hkv])
    # The rotation keeps each pair's norm.
    qn = oracle.qkv_proj(x, w, Hq, Hkv, D, rope_on=False)[0]
    r = lambda z: z[..., 0::2] ** 2 + z[..., 1::2] ** 2  # noqa: E731
    assert np.max(np.abs(r(q) - r(qn))) < 1e-12
    assert np.max(np.abs(q[:, 1:] - qn[:, 1:])) > 1e-3   # and does rotate


@pytest.mark.parametrize("rope_on", [False, True])
def test_qkv_proj_bwd_finite_differences(rope_on):
    # L(x, W) = sum(gq * q) + sum(gk * k) + sum(gv * v) with q, k rotated when rope_on; the
    # gradients of the pre-RoPE projections are then R^-1 gq and R^-1 gk.
    B, T, C, Hq, Hkv, D = 1, 3, 4, 2, 1, 4
    base, pos0 = 100.0, 2
    x = _rand((B, T, C), 51)
    w = _rand((C, (Hq + 2 * Hkv) * D), 52)
    gq, gk, gv = _rand((B, T, Hq, D), 53), _rand((B, T, Hkv, D), 54), _rand((B, T, Hkv, D), 55)
    if rope_on:
        dq, dk = oracle.rope(gq, base, pos0, inverse=True), oracle.rope(gk, base, pos0, inverse=True)
    else:
        dq, dk = gq, gk
    dx, dw = oracle.qkv_proj_bwd(x, w, dq, dk, gv)

    def loss(xx, ww):
        q, k, v = oracle.qkv_proj(xx, ww, Hq, Hkv, D, rope_on=rope_on, base=base, pos0=pos0)
        return float(np.sum(gq * q) + np.sum(gk * k) + np.sum(gv * v))

    eps = 1e-5
    for arr, grad, which in ((x, dx, 0), (w, dw, 1)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(*arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += eps
            m[idx] -= eps
            args_p = (p, w) if which == 0 else (x, p)
            args_m = (m, w) if which == 0 else (x, m)
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.max(np.abs(num - grad)) < 1e-8, which


def test_shape_errors():
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros((2, 3)), np.zeros((4, 2)))
    with pytest.raises(ValueError):
        oracle.qkv_proj(np.zeros((1, 2, 4)), np.zeros((4, 5)), 1, 1, 2)
