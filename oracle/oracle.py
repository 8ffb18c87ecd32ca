"""Plain double-precision CPU oracle for causal GQA attention with RoPE.

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this module; the product path (the HIP library and its Python
binding) never does.  The arithmetic lives in ``oracle.cpp`` (C++, float64, OpenMP), built
here with g++; this module only marshals numpy arrays (the projections are numpy float64
matrix products, written here).  It shares no code with the HIP path.

What each function computes, and the passage it follows, is stated at the C definition:
 * ``rope``      -- rotary embedding on queries and keys ("Show HN: NanoEuler", section 2;
                    "Tiny Hackable CUDA Language Model Implementation", section 1).
 * ``attn_fwd``  -- causal scaled dot-product attention with grouped K/V heads, O and the
                    per-row log-sum-exp ("Tiny Hackable ...", section 1; "Show HN: NanoEuler",
                    section 2 for GQA).
 * ``attn_bwd``  -- the analytic gradients of L = sum(dO * O) with respect to the post-RoPE
                    Q, K and V, dK/dV summed over each query-head group.
 * ``grads_raw`` -- the end-to-end gradients with respect to the pre-RoPE Q and K.
 * ``attn_fwd_nc``, ``attn_bwd_nc`` -- the non-causal form (every query row sees every key
                    row), the per-head attention the blog prints ("Tiled FlashAttention").
 * ``gemm``, ``qkv_proj``, ``qkv_proj_bwd`` -- the projections on either side of the
                    attention: matrix products in float64 (numpy's matmul as the library
                    step), the QKV split into heads, RoPE (``rope`` above) on queries and keys
                    ("Show HN: NanoEuler", sections 2 and 4; "Tiny Hackable ...", section 1:
                    the attention result is projected back to the model dimension).
 * ``attn_fwd_kv`` -- the same causal attention for Tq new query rows against a cache of
                    Tk >= Tq keys (generation with a KV cache: "Show HN: NanoEuler", section 2,
                    speculative decoding with the MTP heads, and the chat REPL of its key
                    points): query row i sits at position Tk - Tq + i.

Every function here is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants, brute force, a library special case and central finite differences.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.cpp`` into ``liboracle.so`` with g++ (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c++17", "-fno-fast-math",
               _SRC, "-o", tmp]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        L = ctypes.c_long
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        lib.oracle_rope.argtypes = [dp, dp, L, L, L, L, ctypes.c_double, L, ctypes.c_int]
        lib.oracle_rope.restype = ctypes.c_int
        lib.oracle_attn_fwd.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, L, ctypes.c_double]
        lib.oracle_attn_fwd.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, L, L, L, L, L, ctypes.c_double]
        lib.oracle_attn_fwd_kv.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, L, L, ctypes.c_double]
        lib.oracle_attn_fwd_kv.restype = ctypes.c_int
        lib.oracle_attn_fwd_nc.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, L, ctypes.c_double]
        lib.oracle_attn_fwd_nc.restype = ctypes.c_int
        lib.oracle_attn_bwd_nc.argtypes = [dp, dp, dp, dp, dp, dp, dp, L, L, L, L, L, ctypes.c_double]
        lib.oracle_attn_bwd_nc.restype = ctypes.c_int
        lib.oracle_attn_bwd.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    """Exact upcast of a numpy array or CPU torch tensor (fp32 / bf16 / fp64) to float64."""
    if hasattr(a, "detach"):  # torch tensor: go through float64 on the CPU (exact)
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    """OpenMP threads the oracle's parallel regions use (OMP_NUM_THREADS)."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Set the OpenMP threads of the following calls (timing only; results do not change)."""
    _load().oracle_set_num_threads(int(n))


def rope(x, base: float = 10000.0, pos0: int = 0, inverse: bool = False) -> np.ndarray:
    """Rotary embedding of x [B, T, H, D] (adjacent pairs; angle (pos0+t)*base^(-2i/D))."""
    x = _f64(x)
    if x.ndim != 4:
        raise ValueError("rope expects [B, T, H, D]")
    B, T, H, D = x.shape
    y = np.empty_like(x)
    rc = _load().oracle_rope(_ptr(x), _ptr(y), B, T, H, D, float(base), int(pos0), int(bool(inverse)))
    if rc != 0:
        raise ValueError("rope: head_dim must be even")
    return y


def _check_qkv(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("expected [B, T, H, D] tensors")
    B, T, Hq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != T or k.shape[3] != D:
        raise ValueError("k/v shape mismatch")
    Hkv = k.shape[2]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, T, Hq, Hkv, D


def attn_fwd(q, k, v, scale: float | None = None):
    """Causal GQA attention forward -> (O [B,T,Hq,D], LSE [B,Hq,T]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, Hq, Hkv, D = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.empty_like(q)
    lse = np.empty((B, Hq, T), dtype=np.float64)
    rc = _load().oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T, Hq, Hkv, D,
                                 float(scale))
    if rc != 0:
        raise ValueError("attn_fwd: bad head counts")
    return o, lse


def attn_fwd_kv(q, k, v, scale: float | None = None):
    """Causal GQA attention of q [B,Tq,Hq,D] against a cache k, v [B,Tk,Hkv,D], Tk >= Tq; query
    row i sits at position Tk - Tq + i -> (O [B,Tq,Hq,D], LSE [B,Hq,Tq]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4 or k.shape != v.shape:
        raise ValueError("expected q [B,Tq,Hq,D] and k, v [B,Tk,Hkv,D]")
    B, Tq, Hq, D = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D or Hkv < 1 or Hq % Hkv != 0 or Tq > Tk:
        raise ValueError("attn_fwd_kv: bad shapes")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.empty_like(q)
    lse = np.empty((B, Hq, Tq), dtype=np.float64)
    rc = _load().oracle_attn_fwd_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Tq, Tk, Hq, Hkv, D,
                                    float(scale))
    if rc != 0:
        raise ValueError("attn_fwd_kv: bad shapes")
    return o, lse


def attn_fwd_nc(q, k, v, scale: float | None = None):
    """Non-causal GQA attention forward -> (O [B,T,Hq,D], LSE [B,Hq,T]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, Hq, Hkv, D = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.empty_like(q)
    lse = np.empty((B, Hq, T), dtype=np.float64)
    rc = _load().oracle_attn_fwd_nc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T, Hq, Hkv, D,
                                    float(scale))
    if rc != 0:
        raise ValueError("attn_fwd_nc: bad head counts")
    return o, lse


def attn_bwd_nc(q, k, v, dout, scale: float | None = None):
    """Gradients (dQ, dK, dV) of sum(dO * O) for the non-causal attention, float64."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, T, Hq, Hkv, D = _check_qkv(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must match q")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    rc = _load().oracle_attn_bwd_nc(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                    B, T, Hq, Hkv, D, float(scale))
    if rc != 0:
        raise ValueError("attn_bwd_nc: bad head counts")
    return dq, dk, dv


def attn_bwd(q, k, v, dout, scale: float | None = None):
    """Analytic gradients of sum(dO * O) w.r.t. the post-RoPE q, k and v (float64)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, T, Hq, Hkv, D = _check_qkv(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must match q")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    rc = _load().oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                 B, T, Hq, Hkv, D, float(scale))
    if rc != 0:
        raise ValueError("attn_bwd: bad head counts")
    return dq, dk, dv


def forward_raw(q_raw, k_raw, v, base: float = 10000.0, scale: float | None = None):
    """O and LSE of attention applied to RoPE(q_raw), RoPE(k_raw), v."""
    return attn_fwd(rope(q_raw, base), rope(k_raw, base), v, scale)


def grads_raw(q_raw, k_raw, v, dout, base: float = 10000.0, scale: float | None = None):
    """End-to-end gradients of sum(dO * O(RoPE(q_raw), RoPE(k_raw), v)) w.r.t. q_raw, k_raw, v.

    The RoPE rotation is orthogonal, so its backward is the inverse rotation.
    """
    qr, kr = rope(q_raw, base), rope(k_raw, base)
    dq, dk, dv = attn_bwd(qr, kr, v, dout, scale)
    return rope(dq, base, inverse=True), rope(dk, base, inverse=True), dv


def gemm(a, b, trans_a: bool = False, trans_b: bool = False) -> np.ndarray:
    """op(A) op(B) in float64; op transposes a stored operand when its flag is set."""
    a, b = _f64(a), _f64(b)
    if a.ndim != 2 or b.ndim != 2:
        raise ValueError("gemm expects 2-D operands")
    opa = a.T if trans_a else a
    opb = b.T if trans_b else b
    if opa.shape[1] != opb.shape[0]:
        raise ValueError("inner dimensions differ")
    return opa @ opb


def _split_qkv(y, B, T, Hq, Hkv, D):
    q = y[:, :Hq * D].reshape(B, T, Hq, D)
    k = y[:, Hq * D:(Hq + Hkv) * D].reshape(B, T, Hkv, D)
    v = y[:, (Hq + Hkv) * D:].reshape(B, T, Hkv, D)
    return np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v)


def qkv_proj(x, w_qkv, Hq: int, Hkv: int, D: int, rope_on: bool = True, base: float = 10000.0,
             pos0: int = 0):
    """QKV projection of x [B, T, C] by w_qkv [C, (Hq + 2 Hkv) D] (columns: query heads, key
    heads, value heads): q, k, v as [B, T, H, D]; with rope_on, q and k rotated by rope()."""
    x, w = _f64(x), _f64(w_qkv)
    B, T, C = x.shape
    if w.shape != (C, (Hq + 2 * Hkv) * D):
        raise ValueError("w_qkv must be [C, (Hq + 2 Hkv) D]")
    q, k, v = _split_qkv(x.reshape(B * T, C) @ w, B, T, Hq, Hkv, D)
    if rope_on:
        q = rope(q, base, pos0)
        k = rope(k, base, pos0)
    return q, k, v


def qkv_proj_bwd(x, w_qkv, dq, dk, dv):
    """Gradients of the QKV projection from dq, dk, dv (w.r.t. the projections before RoPE):
    dx [B, T, C] = [dq | dk | dv] w_qkv^T and dw_qkv = x^T [dq | dk | dv]."""
    x, w = _f64(x), _f64(w_qkv)
    dq, dk, dv = _f64(dq), _f64(dk), _f64(dv)
    B, T, C = x.shape
    g = np.concatenate([dq.reshape(B * T, -1), dk.reshape(B * T, -1), dv.reshape(B * T, -1)], axis=1)
    if g.shape[1] != w.shape[1]:
        raise ValueError("gradient widths do not match w_qkv")
    dx = (g @ w.T).reshape(B, T, C)
    dw = x.reshape(B * T, C).T @ g
    return dx, dw
