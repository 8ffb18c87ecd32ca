"""causal_gqa_attention_fwd_amd -- Python binding of libeuler_attn (gfx950 / MI355X).

Causal grouped-query attention with rotary embeddings, forward and backward, as
hand-written HIP kernels behind a C ABI (``include/euler_attn.h``).  This module only
marshals arguments: torch supplies device memory and the current stream, every step of the
computation runs in the library's kernels.  There is no fallback: if the library is not
built, or the tensors are not on a ROCm device, the calls raise.

    rope_apply(x, base=1e4, pos0=0, inverse=False, out=None) -> y
    attn_fwd(q, k, v, scale=None, out=None, lse=None)        -> (o, lse)
    attn_bwd(q, k, v, o, lse, dout, scale=None, ...)         -> (dq, dk, dv)
    attn_bwd_rope(q, k, v, o, lse, dout, base=1e4, pos0=0, ...)
                         -> (dq, dk, dv) with dq, dk for the tensors before RoPE
    attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv)        -> attn_bwd, no allocation
    attn_decode(q, k_cache, v_cache, scale=None, ...)         -> (o, lse) for the last Tq rows
    attn_fwd_noncausal / attn_bwd_noncausal                   -> as attn_fwd / attn_bwd, no mask
    gemm(a, b, trans_a=False, trans_b=False, out=None, split_k=False) -> op(a) @ op(b)
    qkv_proj(x, w_qkv, Hq, Hkv, D, rope=True, base=1e4, ...)  -> (q, k, v) [B, T, H, D]
    qkv_proj_bwd(x, w_qkv, dq, dk, dv, split_k=False)          -> (dx, dw_qkv)

Layouts: q, o, dout, dq [B, T, Hq, D]; k, v, dk, dv [B, T, Hkv, D]; lse [B, Hq, T] fp32.
dtype float32 or bfloat16.  head_dim 32, 64 or 128 for attention.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["rope_apply", "rope_apply_qk", "attn_fwd", "attn_fwd_noncausal", "attn_fwd_rope",
           "attn_fwd_rope_workspace_size", "attn_fwd_rope_fuses_q", "attn_bwd", "attn_bwd_noncausal", "attn_bwd_workspace_size", "attn_bwd_preprocess",
           "attn_bwd_main", "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_rope", "attn_bwd_rope_workspace_size",
           "attn_bwd_rope_preprocess", "attn_bwd_rope_main", "attn_decode", "attn_decode_workspace_size", "gemm",
           "qkv_proj", "qkv_proj_bwd", "gemm_workspace_size", "attn_bwd_noalloc", "NOALLOC_SCRATCH_BYTES", "lib", "LIB_PATH", "EA_F32",
           "EA_BF16", "STATUS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libeuler_attn.so")
EA_F32, EA_BF16 = 0, 1
STATUS = {0: "EA_OK", 1: "EA_ERR_NULL", 2: "EA_ERR_INVALID_ARG", 3: "EA_ERR_UNSUPPORTED",
          4: "EA_ERR_ALIGN", 5: "EA_ERR_ALIAS", 6: "EA_ERR_WORKSPACE", 7: "EA_ERR_HIP",
          8: "EA_ERR_SCRATCH"}
# Bytes of the static device scratch behind attn_bwd_noalloc (EA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 16 << 20

_lib = None


def lib() -> ctypes.CDLL:
    """Load libeuler_attn.so (built in-tree by ``python -m causal_gqa_attention_fwd_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libeuler_attn.so is not built (%s); run "
                           "`python -m causal_gqa_attention_fwd_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, ci, cd, cf, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_float, ctypes.c_size_t
    L.rope_apply.argtypes = [vp, vp, ci, ci, ci, ci, ci, cd, ci, ci, vp]
    L.rope_apply.restype = ci
    L.rope_apply_qk.argtypes = [vp, vp, ci, vp, vp, ci, ci, ci, ci, ci, cd, ci, ci, vp]
    L.rope_apply_qk.restype = ci
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp]
    L.attn_fwd.restype = ci
    L.attn_fwd_noncausal.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp]
    L.attn_fwd_noncausal.restype = ci
    L.attn_fwd_rope_workspace_size.argtypes = [ci, ci]
    L.attn_fwd_rope_workspace_size.restype = sz
    L.attn_fwd_rope_fuses_q.argtypes = [ci, ci, ci, ci, ci, ci]
    L.attn_fwd_rope_fuses_q.restype = ci
    L.attn_fwd_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, cf, ci, cd, ci, vp]
    L.attn_fwd_rope.restype = ci
    L.attn_bwd_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci]
    L.attn_bwd_workspace_size.restype = sz
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, cf, ci, vp]
    L.attn_bwd.restype = ci
    L.attn_bwd_noncausal.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, cf, ci, vp]
    L.attn_bwd_noncausal.restype = ci
    L.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp]
    L.attn_bwd_noalloc.restype = ci
    L.attn_bwd_preprocess.argtypes = [vp, vp, vp, sz, ci, ci, ci, ci, ci, ci, vp]
    L.attn_bwd_preprocess.restype = ci
    L.attn_bwd_main.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, cf, ci, vp]
    L.attn_bwd_main.restype = ci
    L.attn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, cf, ci, vp]
    L.attn_bwd_dkdv.restype = ci
    L.attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, cf, ci, vp]
    L.attn_bwd_dq.restype = ci
    L.attn_bwd_rope_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci]
    L.attn_bwd_rope_workspace_size.restype = sz
    L.attn_bwd_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, cf, ci, cd, ci, vp]
    L.attn_bwd_rope.restype = ci
    L.attn_bwd_rope_preprocess.argtypes = [vp, vp, vp, sz, ci, ci, ci, ci, ci, ci, cd, ci, vp]
    L.attn_bwd_rope_preprocess.restype = ci
    L.attn_bwd_rope_main.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, cf, ci, vp]
    L.attn_bwd_rope_main.restype = ci
    L.attn_decode_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci, ci]
    L.attn_decode_workspace_size.restype = sz
    L.attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, ci, cf, ci, vp]
    L.attn_decode.restype = ci
    L.gemm.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, ci, vp]
    L.gemm.restype = ci
    L.gemm_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci]
    L.gemm_workspace_size.restype = sz
    L.gemm_ws.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, ci, vp, sz, vp]
    L.gemm_ws.restype = ci
    L.qkv_proj.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, cd, ci, vp]
    L.qkv_proj.restype = ci
    L.qkv_proj_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp]
    L.qkv_proj_bwd.restype = ci
    L.qkv_proj_bwd_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci, ci]
    L.qkv_proj_bwd_workspace_size.restype = sz
    L.qkv_proj_bwd_ws.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp, sz, vp]
    L.qkv_proj_bwd_ws.restype = ci
    L.euler_attn_status_string.argtypes = [ci]
    L.euler_attn_status_string.restype = ctypes.c_char_p
    L.euler_attn_version.argtypes = []
    L.euler_attn_version.restype = ci
    _lib = L
    return L


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return EA_F32
    if t.dtype == torch.bfloat16:
        return EA_BF16
    raise TypeError("euler_attn supports float32 and bfloat16 tensors, got %s" % t.dtype)


def _check(name: str, t: torch.Tensor, ndim: int, device=None, dtype=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise RuntimeError("%s must be on a ROCm GPU device (got %s); there is no CPU path"
                           % (name, t.device))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dimensions, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))


def _raise(status: int, what: str) -> None:
    if status != 0:
        msg = lib().euler_attn_status_string(status).decode()
        raise RuntimeError("%s failed: %s" % (what, msg))


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def rope_apply(x: torch.Tensor, base: float = 10000.0, pos0: int = 0, inverse: bool = False,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """Rotary embedding of x [B, T, H, D] (adjacent pairs, angle (pos0+t)*base^(-2i/D))."""
    _check("x", x, 4)
    y = torch.empty_like(x) if out is None else out
    _check("out", y, 4, x.device, x.dtype)
    if y.shape != x.shape:
        raise ValueError("out must have the shape of x")
    B, T, H, D = x.shape
    with torch.cuda.device(x.device):
        st = lib().rope_apply(x.data_ptr(), y.data_ptr(), B, T, H, D, _dtype_code(x), float(base),
                              int(pos0), int(bool(inverse)), _stream(x.device))
    _raise(st, "rope_apply")
    return y


def rope_apply_qk(q: torch.Tensor, k: torch.Tensor, base: float = 10000.0, pos0: int = 0,
                  inverse: bool = False, q_out: torch.Tensor | None = None,
                  k_out: torch.Tensor | None = None):
    """rope_apply on q [B,T,Hq,D] and k [B,T,Hkv,D] in one launch; returns (q_out, k_out)."""
    _check("q", q, 4)
    _check("k", k, 4, q.device, q.dtype)
    if k.shape[0] != q.shape[0] or k.shape[1] != q.shape[1] or k.shape[3] != q.shape[3]:
        raise ValueError("q and k must share B, T and D")
    qo = torch.empty_like(q) if q_out is None else q_out
    ko = torch.empty_like(k) if k_out is None else k_out
    _check("q_out", qo, 4, q.device, q.dtype)
    _check("k_out", ko, 4, q.device, q.dtype)
    if qo.shape != q.shape or ko.shape != k.shape:
        raise ValueError("outputs must match their inputs' shapes")
    B, T, Hq, D = q.shape
    with torch.cuda.device(q.device):
        st = lib().rope_apply_qk(q.data_ptr(), qo.data_ptr(), Hq, k.data_ptr(), ko.data_ptr(), k.shape[2],
                                 B, T, D, _dtype_code(q), float(base), int(pos0), int(bool(inverse)),
                                 _stream(q.device))
    _raise(st, "rope_apply_qk")
    return qo, ko


def _shapes(q, k, v):
    _check("q", q, 4)
    _check("k", k, 4, q.device, q.dtype)
    _check("v", v, 4, q.device, q.dtype)
    B, T, Hq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != T or k.shape[3] != D:
        raise ValueError("k and v must be [B, T, Hkv, D] matching q [B, T, Hq, D]")
    return B, T, Hq, k.shape[2], D


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
             out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Causal GQA attention forward; returns (o [B,T,Hq,D], lse [B,Hq,T] float32)."""
    return _fwd("attn_fwd", q, k, v, scale, out, lse)


def attn_fwd_noncausal(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
                       out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """GQA attention forward without the causal mask (every query sees every key)."""
    return _fwd("attn_fwd_noncausal", q, k, v, scale, out, lse)


def attn_fwd_rope_workspace_size(T: int, D: int) -> int:
    """Bytes of the workspace attn_fwd_rope needs (the RoPE (cos, sin) table)."""
    return int(lib().attn_fwd_rope_workspace_size(T, D))


def attn_fwd_rope_fuses_q(B: int, T: int, Hq: int, Hkv: int, D: int, dtype=torch.bfloat16) -> int:
    """1 if attn_fwd_rope rotates the queries inside the forward at this shape, 0 if its first
    launch rotates them with K, -1 for sizes attn_fwd rejects (host-only query)."""
    code = EA_F32 if dtype == torch.float32 else EA_BF16
    return int(lib().attn_fwd_rope_fuses_q(B, T, Hq, Hkv, D, code))


def attn_fwd_rope(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, base: float = 10000.0,
                  pos0: int = 0, scale: float | None = None, workspace: torch.Tensor | None = None):
    """RoPE on pre-rotation q and k fused with the causal GQA forward.

    Returns (o, lse, q_r, k_r): the attention output and log-sum-exp as attn_fwd, and the
    rotated q and k, which attn_bwd / attn_bwd_rope take as their q and k."""
    B, T, Hq, Hkv, D = _shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q)
    l = torch.empty((B, Hq, T), device=q.device, dtype=torch.float32)
    qr = torch.empty_like(q)
    kr = torch.empty_like(k)
    need = attn_fwd_rope_workspace_size(T, D)
    ws = torch.empty(need, device=q.device, dtype=torch.uint8) if workspace is None else workspace
    wp, wb = _ws_args(ws, q.device)
    with torch.cuda.device(q.device):
        st = lib().attn_fwd_rope(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                                 qr.data_ptr(), kr.data_ptr(), wp, wb, B, T, Hq, Hkv, D, float(scale),
                                 _dtype_code(q), float(base), int(pos0), _stream(q.device))
    _raise(st, "attn_fwd_rope")
    return o, l, qr, kr


def _fwd(name, q, k, v, scale, out, lse):
    B, T, Hq, Hkv, D = _shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    _check("out", o, 4, q.device, q.dtype)
    if o.shape != q.shape:
        raise ValueError("out must have the shape of q")
    l = torch.empty((B, Hq, T), device=q.device, dtype=torch.float32) if lse is None else lse
    _check("lse", l, 3, q.device, torch.float32)
    if tuple(l.shape) != (B, Hq, T):
        raise ValueError("lse must be [B, Hq, T]")
    with torch.cuda.device(q.device):
        st = getattr(lib(), name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                                  B, T, Hq, Hkv, D, float(scale), _dtype_code(q), _stream(q.device))
    _raise(st, name)
    return o, l


def attn_bwd_workspace_size(B: int, T: int, Hq: int, Hkv: int, D: int, dtype=torch.bfloat16) -> int:
    code = EA_F32 if dtype == torch.float32 else EA_BF16
    return int(lib().attn_bwd_workspace_size(B, T, Hq, Hkv, D, code))


def attn_bwd_rope_workspace_size(B: int, T: int, Hq: int, Hkv: int, D: int, dtype=torch.bfloat16) -> int:
    code = EA_F32 if dtype == torch.float32 else EA_BF16
    return int(lib().attn_bwd_rope_workspace_size(B, T, Hq, Hkv, D, code))


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
             lse: torch.Tensor, dout: torch.Tensor, scale: float | None = None,
             workspace: torch.Tensor | None = None, dq: torch.Tensor | None = None,
             dk: torch.Tensor | None = None, dv: torch.Tensor | None = None):
    """Causal GQA attention backward; returns (dq, dk, dv), dk/dv summed over each group."""
    return _bwd(q, k, v, o, lse, dout, scale, workspace, dq, dk, dv, None)


def attn_bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                     lse: torch.Tensor, dout: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor,
                     dv: torch.Tensor, scale: float | None = None):
    """attn_bwd without a workspace: D_t goes to the library's static per-device scratch, so
    nothing is allocated (the caller passes the outputs).  Calls that overlap in time on one
    device race on that scratch.  Returns (dq, dk, dv)."""
    B, T, Hq, Hkv, D = _shapes(q, k, v)
    _check("o", o, 4, q.device, q.dtype)
    _check("dout", dout, 4, q.device, q.dtype)
    _check("lse", lse, 3, q.device, torch.float32)
    if o.shape != q.shape or dout.shape != q.shape or tuple(lse.shape) != (B, Hq, T):
        raise ValueError("o/dout must match q and lse must be [B, Hq, T]")
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check(name, t, 4, q.device, q.dtype)
        if t.shape != ref.shape:
            raise ValueError("%s has the wrong shape" % name)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    with torch.cuda.device(q.device):
        st = lib().attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, T, Hq,
                                    Hkv, D, float(scale), _dtype_code(q), _stream(q.device))
    _raise(st, "attn_bwd_noalloc")
    return dq, dk, dv


def attn_bwd_noncausal(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                       lse: torch.Tensor, dout: torch.Tensor, scale: float | None = None,
                       workspace: torch.Tensor | None = None, dq: torch.Tensor | None = None,
                       dk: torch.Tensor | None = None, dv: torch.Tensor | None = None):
    """Backward of attn_fwd_noncausal; returns (dq, dk, dv), dk/dv summed over each group."""
    return _bwd(q, k, v, o, lse, dout, scale, workspace, dq, dk, dv, "noncausal")


def attn_bwd_rope(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                  lse: torch.Tensor, dout: torch.Tensor, base: float = 10000.0, pos0: int = 0,
                  scale: float | None = None, workspace: torch.Tensor | None = None,
                  dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                  dv: torch.Tensor | None = None):
    """attn_bwd with the RoPE backward fused in: q, k are the rotated tensors attn_fwd saw;
    dq, dk are returned for the tensors before rope_apply(base, pos0).  Returns (dq, dk, dv)."""
    return _bwd(q, k, v, o, lse, dout, scale, workspace, dq, dk, dv, (float(base), int(pos0)))


def _bwd(q, k, v, o, lse, dout, scale, workspace, dq, dk, dv, rope):
    # rope: None (causal), "noncausal", or (base, pos0) for the fused RoPE backward.
    B, T, Hq, Hkv, D = _shapes(q, k, v)
    _check("o", o, 4, q.device, q.dtype)
    _check("dout", dout, 4, q.device, q.dtype)
    _check("lse", lse, 3, q.device, torch.float32)
    if o.shape != q.shape or dout.shape != q.shape or tuple(lse.shape) != (B, Hq, T):
        raise ValueError("o/dout must match q and lse must be [B, Hq, T]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check(name, t, 4, q.device, q.dtype)
        if t.shape != ref.shape:
            raise ValueError("%s has the wrong shape" % name)
    with_rope = isinstance(rope, tuple)
    wsfn = lib().attn_bwd_rope_workspace_size if with_rope else lib().attn_bwd_workspace_size
    need = int(wsfn(B, T, Hq, Hkv, D, _dtype_code(q)))
    if workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the device of q")
    nbytes = workspace.numel() * workspace.element_size()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), nbytes, B, T, Hq, Hkv, D,
            float(scale), _dtype_code(q))
    name = "attn_bwd_rope" if with_rope else ("attn_bwd" if rope is None else "attn_bwd_noncausal")
    with torch.cuda.device(q.device):
        if with_rope:
            st = lib().attn_bwd_rope(*args, rope[0], rope[1], _stream(q.device))
        else:
            st = getattr(lib(), name)(*args, _stream(q.device))
    _raise(st, name)
    return dq, dk, dv


def _ws_args(workspace: torch.Tensor, device) -> tuple:
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the device of the inputs")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def attn_bwd_preprocess(o: torch.Tensor, dout: torch.Tensor, workspace: torch.Tensor, Hkv: int) -> None:
    """Backward stage 1: D_t = sum_d dout * o into the workspace."""
    _check("o", o, 4)
    _check("dout", dout, 4, o.device, o.dtype)
    B, T, Hq, D = o.shape
    wp, wb = _ws_args(workspace, o.device)
    with torch.cuda.device(o.device):
        st = lib().attn_bwd_preprocess(o.data_ptr(), dout.data_ptr(), wp, wb, B, T, Hq, Hkv, D,
                                       _dtype_code(o), _stream(o.device))
    _raise(st, "attn_bwd_preprocess")


def attn_bwd_main(q, k, v, lse, dout, workspace, dq, dk, dv, scale: float | None = None) -> None:
    """Backward stage 2 in one launch: dq, dk, dv; needs the preprocess workspace."""
    B, T, Hq, Hkv, D = _shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    wp, wb = _ws_args(workspace, q.device)
    with torch.cuda.device(q.device):
        st = lib().attn_bwd_main(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(),
                                 dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), wp, wb,
                                 B, T, Hq, Hkv, D, float(scale), _dtype_code(q), _stream(q.device))
    _raise(st, "attn_bwd_main")


def attn_bwd_dkdv(q, k, v, lse, dout, workspace, dk, dv, scale: float | None = None) -> None:
    """Backward stage 2: dk, dv (group-summed, overwritten); needs the preprocess workspace."""
    B, T, Hq, Hkv, D = _shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    wp, wb = _ws_args(workspace, q.device)
    with torch.cuda.device(q.device):
        st = lib().attn_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(),
                                 dout.data_ptr(), dk.data_ptr(), dv.data_ptr(), wp, wb, B, T, Hq,
                                 Hkv, D, float(scale), _dtype_code(q), _stream(q.device))
    _raise(st, "attn_bwd_dkdv")


def attn_bwd_dq(q, k, v, lse, dout, workspace, dq, scale: float | None = None) -> None:
    """Backward stage 3: dq (overwritten); needs the preprocess workspace."""
    B, T, Hq, Hkv, D = _shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    wp, wb = _ws_args(workspace, q.device)
    with torch.cuda.device(q.device):
        st = lib().attn_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(),
                               dout.data_ptr(), dq.data_ptr(), wp, wb, B, T, Hq, Hkv, D,
                               float(scale), _dtype_code(q), _stream(q.device))
    _raise(st, "attn_bwd_dq")


def attn_bwd_rope_preprocess(o: torch.Tensor, dout: torch.Tensor, workspace: torch.Tensor, Hkv: int,
                             base: float = 10000.0, pos0: int = 0) -> None:
    """Stage 1 of attn_bwd_rope: D_t and the RoPE (cos, sin) table into the workspace."""
    _check("o", o, 4)
    _check("dout", dout, 4, o.device, o.dtype)
    B, T, Hq, D = o.shape
    wp, wb = _ws_args(workspace, o.device)
    with torch.cuda.device(o.device):
        st = lib().attn_bwd_rope_preprocess(o.data_ptr(), dout.data_ptr(), wp, wb, B, T, Hq, Hkv, D,
                                            _dtype_code(o), float(base), int(pos0), _stream(o.device))
    _raise(st, "attn_bwd_rope_preprocess")


def attn_bwd_rope_main(q, k, v, lse, dout, workspace, dq, dk, dv, scale: float | None = None) -> None:
    """Stage 2 of attn_bwd_rope in one launch: dv, and dq, dk rotated back by -phi."""
    B, T, Hq, Hkv, D = _shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    wp, wb = _ws_args(workspace, q.device)
    with torch.cuda.device(q.device):
        st = lib().attn_bwd_rope_main(q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(),
                                      dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), wp, wb,
                                      B, T, Hq, Hkv, D, float(scale), _dtype_code(q), _stream(q.device))
    _raise(st, "attn_bwd_rope_main")


def attn_decode_workspace_size(B: int, Tq: int, Tk: int, Hq: int, Hkv: int, D: int, dtype=torch.bfloat16) -> int:
    code = EA_F32 if dtype == torch.float32 else EA_BF16
    return int(lib().attn_decode_workspace_size(B, Tq, Tk, Hq, Hkv, D, code))


def attn_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
                out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None):
    """Attention of q [B,Tq,Hq,D] (the last Tq positions) against the cache k, v [B,Tk,Hkv,D];
    returns (o [B,Tq,Hq,D], lse [B,Hq,Tq] float32)."""
    _check("q", q, 4)
    _check("k", k, 4, q.device, q.dtype)
    _check("v", v, 4, q.device, q.dtype)
    B, Tq, Hq, D = q.shape
    Tk, Hkv = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k and v must be [B, Tk, Hkv, D] matching q [B, Tq, Hq, D]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    _check("out", o, 4, q.device, q.dtype)
    l = torch.empty((B, Hq, Tq), device=q.device, dtype=torch.float32) if lse is None else lse
    _check("lse", l, 3, q.device, torch.float32)
    need = int(lib().attn_decode_workspace_size(B, Tq, Tk, Hq, Hkv, D, _dtype_code(q)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), device=q.device, dtype=torch.uint8)
    wp, wb = _ws_args(workspace, q.device)
    with torch.cuda.device(q.device):
        st = lib().attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), wp, wb,
                               B, Tq, Tk, Hq, Hkv, D, float(scale), _dtype_code(q), _stream(q.device))
    _raise(st, "attn_decode")
    return o, l


def gemm_workspace_size(M: int, N: int, K: int, trans_a: bool = False, trans_b: bool = False,
                        dtype=torch.bfloat16) -> int:
    """Bytes of the workspace that lets gemm(..., split_k=True) split K for this shape (0: none)."""
    code = EA_F32 if dtype == torch.float32 else EA_BF16
    return int(lib().gemm_workspace_size(M, N, K, int(bool(trans_a)), int(bool(trans_b)), code))


def gemm(a: torch.Tensor, b: torch.Tensor, trans_a: bool = False, trans_b: bool = False,
         out: torch.Tensor | None = None, split_k: bool = False,
         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """op(a) @ op(b) for contiguous 2-D tensors (op transposes when its flag is set).  With
    split_k (gemm_ws), a product with few output tiles and a long K splits K over more
    workgroups, through a workspace (allocated here when not given)."""
    _check("a", a, 2)
    _check("b", b, 2, a.device, a.dtype)
    M, K = (a.shape[1], a.shape[0]) if trans_a else (a.shape[0], a.shape[1])
    Kb, N = (b.shape[1], b.shape[0]) if trans_b else (b.shape[0], b.shape[1])
    if K != Kb:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, Kb))
    c = torch.empty((M, N), device=a.device, dtype=a.dtype) if out is None else out
    _check("out", c, 2, a.device, a.dtype)
    if tuple(c.shape) != (M, N):
        raise ValueError("out must be [%d, %d]" % (M, N))
    ta, tb = int(bool(trans_a)), int(bool(trans_b))
    if split_k or workspace is not None:
        if workspace is None:
            need = int(lib().gemm_workspace_size(M, N, K, ta, tb, _dtype_code(a)))
            workspace = torch.empty(max(need, 256), device=a.device, dtype=torch.uint8)
        wp, wb = _ws_args(workspace, a.device)
        with torch.cuda.device(a.device):
            st = lib().gemm_ws(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, a.shape[1], b.shape[1], N,
                               ta, tb, _dtype_code(a), wp, wb, _stream(a.device))
        _raise(st, "gemm_ws")
        return c
    with torch.cuda.device(a.device):
        st = lib().gemm(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, a.shape[1], b.shape[1], N,
                        ta, tb, _dtype_code(a), _stream(a.device))
    _raise(st, "gemm")
    return c


def qkv_proj(x: torch.Tensor, w_qkv: torch.Tensor, Hq: int, Hkv: int, D: int, rope: bool = True,
             base: float = 10000.0, pos0: int = 0, q: torch.Tensor | None = None,
             k: torch.Tensor | None = None, v: torch.Tensor | None = None):
    """q, k, v = x Wq, x Wk, x Wv from x [B, T, C] and w_qkv [C, (Hq + 2 Hkv) D], as
    [B, T, H, D]; with rope, q and k are rotated (as rope_apply) before they are stored."""
    _check("x", x, 3)
    _check("w_qkv", w_qkv, 2, x.device, x.dtype)
    B, T, C = x.shape
    outs = []
    for name, t, H in (("q", q, Hq), ("k", k, Hkv), ("v", v, Hkv)):
        t = torch.empty((B, T, H, D), device=x.device, dtype=x.dtype) if t is None else t
        _check(name, t, 4, x.device, x.dtype)
        if tuple(t.shape) != (B, T, H, D):
            raise ValueError("%s must be [B, T, %d, D]" % (name, H))
        outs.append(t)
    with torch.cuda.device(x.device):
        st = lib().qkv_proj(x.data_ptr(), w_qkv.data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(),
                            outs[2].data_ptr(), B, T, C, Hq, Hkv, D, _dtype_code(x), int(bool(rope)),
                            float(base), int(pos0), _stream(x.device))
    _raise(st, "qkv_proj")
    return tuple(outs)


def qkv_proj_bwd(x: torch.Tensor, w_qkv: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor,
                 dv: torch.Tensor, dx: torch.Tensor | None = None, dw_qkv: torch.Tensor | None = None,
                 split_k: bool = False, workspace: torch.Tensor | None = None):
    """dx = [dq | dk | dv] w_qkv^T and dw_qkv = x^T [dq | dk | dv] (dq, dk: gradients of the
    projections before RoPE).  With split_k (qkv_proj_bwd_ws) the products may split K, as
    gemm(..., split_k=True).  Returns (dx, dw_qkv)."""
    _check("x", x, 3)
    _check("w_qkv", w_qkv, 2, x.device, x.dtype)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, 4, x.device, x.dtype)
    B, T, C = x.shape
    Hq, D = dq.shape[2], dq.shape[3]
    Hkv = dk.shape[2]
    dx = torch.empty_like(x) if dx is None else dx
    dw = torch.empty_like(w_qkv) if dw_qkv is None else dw_qkv
    _check("dx", dx, 3, x.device, x.dtype)
    _check("dw_qkv", dw, 2, x.device, x.dtype)
    if dx.shape != x.shape or dw.shape != w_qkv.shape:
        raise ValueError("dx / dw_qkv must match x / w_qkv")
    if split_k or workspace is not None:
        if workspace is None:
            need = int(lib().qkv_proj_bwd_workspace_size(B, T, C, Hq, Hkv, D, _dtype_code(x)))
            workspace = torch.empty(max(need, 256), device=x.device, dtype=torch.uint8)
        wp, wb = _ws_args(workspace, x.device)
        with torch.cuda.device(x.device):
            st = lib().qkv_proj_bwd_ws(x.data_ptr(), w_qkv.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                       dv.data_ptr(), dx.data_ptr(), dw.data_ptr(), B, T, C, Hq, Hkv, D,
                                       _dtype_code(x), wp, wb, _stream(x.device))
        _raise(st, "qkv_proj_bwd_ws")
        return dx, dw
    with torch.cuda.device(x.device):
        st = lib().qkv_proj_bwd(x.data_ptr(), w_qkv.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                dx.data_ptr(), dw.data_ptr(), B, T, C, Hq, Hkv, D, _dtype_code(x),
                                _stream(x.device))
    _raise(st, "qkv_proj_bwd")
    return dx, dw
