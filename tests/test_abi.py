"""The C ABI of libeuler_attn, on the CPU: the library loads, exports every symbol the
header declares, and rejects invalid calls with the documented status before touching the
device (validation never dereferences a pointer, so fake addresses are used here).
No call in this file reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import causal_gqa_attention_fwd_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "euler_attn.h")

OK, NULL, INVALID, UNSUP, ALIGN, ALIAS, WS, HIP, SCRATCH = range(9)
F32, BF16 = 0, 1
A = 1 << 32  # fake, 256-byte aligned "device" addresses, far apart


def fake(n):
    return A * (n + 1)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ea.LIB_PATH):
        pytest.skip("libeuler_attn.so not built")
    return ea.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("rope_apply", "attn_fwd", "attn_fwd_rope", "attn_fwd_rope_workspace_size", "attn_bwd",
              "attn_bwd_workspace_size", "attn_bwd_rope",
              "attn_fwd_noncausal", "attn_bwd_noncausal", "attn_decode",
              "attn_bwd_rope_workspace_size", "euler_attn_status_string", "euler_attn_version"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    for code in range(9):
        s = L.euler_attn_status_string(code).decode()
        assert s.startswith(ea.STATUS[code])
    assert L.euler_attn_version() >= 100


def rope(L, x=fake(0), y=fake(1), B=1, T=4, H=2, D=64, dt=BF16, base=1e4, pos0=0, inv=0):
    return L.rope_apply(x, y, B, T, H, D, dt, base, pos0, inv, None)


def test_rope_validation(L):
    assert rope(L, x=None) == NULL
    assert rope(L, y=None) == NULL
    for kw in (dict(B=0), dict(T=0), dict(H=0), dict(D=7), dict(D=0), dict(pos0=-1),
               dict(base=1.0), dict(base=float("nan")), dict(base=float("inf")), dict(inv=2)):
        assert rope(L, **kw) == INVALID, kw
    assert rope(L, D=258) == UNSUP
    assert rope(L, dt=5) == UNSUP
    assert rope(L, x=fake(0) + 4) == ALIGN
    assert rope(L, y=fake(0) + 16) == ALIAS  # partial overlap
    # y == x is allowed: it passes validation (and would launch), so not called here.


def test_rope_qk_validation(L):
    def r(q=fake(0), qo=fake(1), Hq=4, k=fake(2), ko=fake(3), Hkv=2, D=64, inv=0):
        return L.rope_apply_qk(q, qo, Hq, k, ko, Hkv, 2, 16, D, BF16, 1e4, 0, inv, None)
    assert r(k=None) == NULL
    assert r(Hkv=0) == INVALID
    assert r(inv=3) == INVALID
    assert r(D=258) == UNSUP
    assert r(ko=fake(3) + 8) == ALIGN
    assert r(ko=fake(2) + 64) == ALIAS          # k_out partially over k
    assert r(qo=fake(2)) == ALIAS               # q_out over k
    assert r(k=fake(0) + 1024) == ALIAS         # k inside q


def fwd(L, q=fake(0), k=fake(1), v=fake(2), o=fake(3), lse=fake(4), B=2, T=16, Hq=4, Hkv=2,
        D=64, scale=0.125, dt=BF16, fn="attn_fwd"):
    return getattr(L, fn)(q, k, v, o, lse, B, T, Hq, Hkv, D, scale, dt, None)


@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_noncausal"])
def test_fwd_validation(L, fn):
    def fwd(L, **kw):
        return globals()["fwd"](L, fn=fn, **kw)
    for name in ("q", "k", "v", "o", "lse"):
        assert fwd(L, **{name: None}) == NULL, name
    for kw in (dict(B=0), dict(T=0), dict(Hq=0), dict(Hkv=0), dict(Hq=3, Hkv=2),
               dict(scale=0.0), dict(scale=-1.0), dict(scale=float("nan")), dict(scale=float("inf"))):
        assert fwd(L, **kw) == INVALID, kw
    for D in (16, 48, 96, 256):
        assert fwd(L, D=D) == UNSUP
    assert fwd(L, dt=3) == UNSUP
    assert fwd(L, v=fake(2) + 8) == ALIGN
    assert fwd(L, lse=fake(4) + 4) == ALIGN
    assert fwd(L, o=fake(0)) == ALIAS
    assert fwd(L, lse=fake(1) + 256) == ALIAS
    assert fwd(L, lse=fake(3) + 1024) == ALIAS   # lse inside o


def test_workspace_size(L):
    # fp32 D_t [B, Hq, T] rounded to 256 bytes; linear in T.
    def ws(B, T, Hq, Hkv, D, dt=BF16):
        return L.attn_bwd_workspace_size(B, T, Hq, Hkv, D, dt)

    def up(x):
        return (x + 255) // 256 * 256
    assert ws(4, 1024, 12, 4, 64) == up(4 * 12 * 1024 * 4)
    assert ws(1, 3, 1, 1, 32) == up(3 * 4)
    assert ws(8, 4096, 32, 8, 128) == 2 * ws(8, 2048, 32, 8, 128)
    assert ws(0, 4, 1, 1, 32) == 0
    assert ws(1, 4, 3, 2, 32) == 0


def bwd(L, q=fake(0), k=fake(1), v=fake(2), o=fake(3), lse=fake(4), do=fake(5), dq=fake(6),
        dk=fake(7), dv=fake(8), ws=fake(9), wsb=None, B=2, T=16, Hq=4, Hkv=2, D=64, scale=0.125,
        dt=BF16, fn="attn_bwd"):
    if wsb is None:
        wsb = L.attn_bwd_workspace_size(B, T, Hq, Hkv, D, dt)
    return getattr(L, fn)(q, k, v, o, lse, do, dq, dk, dv, ws, wsb, B, T, Hq, Hkv, D, scale, dt, None)


@pytest.mark.parametrize("fn", ["attn_bwd", "attn_bwd_noncausal"])
def test_bwd_validation(L, fn):
    def bwd(L, **kw):
        return globals()["bwd"](L, fn=fn, **kw)
    for name in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "ws"):
        assert bwd(L, **{name: None}) == NULL, name
    for kw in (dict(B=0), dict(T=0), dict(Hq=6, Hkv=4), dict(scale=0.0)):
        assert bwd(L, **kw) == INVALID, kw
    assert bwd(L, D=80) == UNSUP
    assert bwd(L, dk=fake(7) + 2) == ALIGN
    assert bwd(L, ws=fake(9) + 16) == ALIGN          # workspace needs 256-byte alignment
    assert bwd(L, wsb=L.attn_bwd_workspace_size(2, 16, 4, 2, 64, BF16) - 1) == WS
    assert bwd(L, dq=fake(0)) == ALIAS                # output over an input
    assert bwd(L, dv=fake(7)) == ALIAS                # two outputs
    assert bwd(L, ws=fake(6)) == ALIAS                # workspace over an output


def test_bwd_stage_validation(L):
    ws = L.attn_bwd_workspace_size(2, 16, 4, 2, 64, BF16)
    pre = lambda o=fake(0), do=fake(1), w=fake(2), wb=ws, D=64, Hq=4: L.attn_bwd_preprocess(  # noqa
        o, do, w, wb, 2, 16, Hq, 2, D, BF16, None)
    assert pre(o=None) == NULL
    assert pre(D=48) == UNSUP
    assert pre(Hq=3) == INVALID
    assert pre(w=fake(2) + 64) == ALIGN
    assert pre(wb=ws - 1) == WS
    assert pre(w=fake(1)) == ALIAS
    dkdv = lambda dk=fake(5), dv=fake(6), w=fake(7), scale=0.1: L.attn_bwd_dkdv(  # noqa
        fake(0), fake(1), fake(2), fake(3), fake(4), dk, dv, w, ws, 2, 16, 4, 2, 64, scale, BF16, None)
    assert dkdv(dk=None) == NULL
    assert dkdv(scale=-1.0) == INVALID
    assert dkdv(dv=fake(5)) == ALIAS
    assert dkdv(dk=fake(7)) == ALIAS           # output over the workspace
    assert dkdv(w=fake(7) + 32) == ALIGN
    mn = lambda dq=fake(5), dk=fake(6), dv=fake(7), w=fake(8): L.attn_bwd_main(  # noqa
        fake(0), fake(1), fake(2), fake(3), fake(4), dq, dk, dv, w, ws, 2, 16, 4, 2, 64, 0.1, BF16, None)
    assert mn(dv=None) == NULL
    assert mn(dq=fake(6)) == ALIAS
    assert mn(dk=fake(2)) == ALIAS
    assert mn(w=fake(8) + 16) == ALIGN
    dq = lambda dq=fake(5), w=fake(6), wb=ws: L.attn_bwd_dq(  # noqa
        fake(0), fake(1), fake(2), fake(3), fake(4), dq, w, wb, 2, 16, 4, 2, 64, 0.1, BF16, None)
    assert dq(dq=None) == NULL
    assert dq(wb=16) == WS
    assert dq(dq=fake(0) + 256) == ALIAS
    assert dq(dq=fake(6)) == ALIAS


def test_bwd_rope_workspace_size(L):
    # D_t as for attn_bwd, then the fp32 (cos, sin) table [T, D/2, 2], each rounded to 256 bytes.
    def up(x):
        return (x + 255) // 256 * 256
    for (B, T, Hq, Hkv, D) in ((4, 1024, 12, 4, 64), (1, 3, 1, 1, 32), (8, 4096, 32, 8, 128)):
        assert L.attn_bwd_rope_workspace_size(B, T, Hq, Hkv, D, BF16) == \
            L.attn_bwd_workspace_size(B, T, Hq, Hkv, D, BF16) + up(T * D * 4)
    assert L.attn_bwd_rope_workspace_size(1, 4, 3, 2, 32, BF16) == 0


def test_bwd_rope_validation(L):
    ws = L.attn_bwd_rope_workspace_size(2, 16, 4, 2, 64, BF16)

    def br(q=fake(0), dq=fake(6), dk=fake(7), w=fake(9), wb=ws, base=1e4, pos0=0, D=64, T=16):
        return L.attn_bwd_rope(q, fake(1), fake(2), fake(3), fake(4), fake(5), dq, dk, fake(8), w, wb,
                               2, T, 4, 2, D, 0.125, BF16, base, pos0, None)
    assert br(q=None) == NULL
    for kw in (dict(base=1.0), dict(base=0.5), dict(base=float("nan")), dict(base=float("inf")),
               dict(pos0=-1), dict(pos0=(1 << 31) - 8)):
        assert br(**kw) == INVALID, kw
    assert br(D=96) == UNSUP
    # the plain backward's workspace is too small for the table
    assert br(wb=L.attn_bwd_workspace_size(2, 16, 4, 2, 64, BF16)) == WS
    assert br(wb=ws - 1) == WS
    assert br(w=fake(9) + 128) == ALIGN
    assert br(dk=fake(6)) == ALIAS
    assert br(w=fake(7)) == ALIAS
    pre = lambda w=fake(2), wb=ws, base=1e4, pos0=0: L.attn_bwd_rope_preprocess(  # noqa
        fake(0), fake(1), w, wb, 2, 16, 4, 2, 64, BF16, base, pos0, None)
    assert pre(w=None) == NULL
    assert pre(base=1.0) == INVALID
    assert pre(pos0=-3) == INVALID
    assert pre(wb=ws - 1) == WS
    assert pre(w=fake(1)) == ALIAS
    mn = lambda dq=fake(5), w=fake(8), wb=ws: L.attn_bwd_rope_main(  # noqa
        fake(0), fake(1), fake(2), fake(3), fake(4), dq, fake(6), fake(7), w, wb, 2, 16, 4, 2, 64, 0.1,
        BF16, None)
    assert mn(dq=None) == NULL
    assert mn(wb=L.attn_bwd_workspace_size(2, 16, 4, 2, 64, BF16)) == WS
    assert mn(dq=fake(8)) == ALIAS


def test_fwd_rope_workspace_and_validation(L):
    # The (cos, sin) table of every (position, pair): fp32 [T, D/2, 2], rounded to 256 bytes.
    for (T, D) in ((1024, 64), (3, 32), (4096, 128)):
        assert L.attn_fwd_rope_workspace_size(T, D) == (T * D * 4 + 255) // 256 * 256
    assert L.attn_fwd_rope_workspace_size(0, 64) == 0
    assert L.attn_fwd_rope_workspace_size(16, 7) == 0
    ws = L.attn_fwd_rope_workspace_size(16, 64)

    def fr(q=fake(0), k=fake(1), v=fake(2), o=fake(3), lse=fake(4), qr=fake(5), kr=fake(6), w=fake(7),
           wb=ws, T=16, D=64, Hq=4, Hkv=2, scale=0.125, dt=BF16, base=1e4, pos0=0):
        return L.attn_fwd_rope(q, k, v, o, lse, qr, kr, w, wb, 2, T, Hq, Hkv, D, scale, dt, base, pos0, None)
    for name in ("q", "k", "v", "o", "lse", "qr", "kr", "w"):
        assert fr(**{name: None}) == NULL, name
    for kw in (dict(Hq=3), dict(scale=0.0), dict(base=1.0), dict(base=float("nan")), dict(pos0=-1),
               dict(pos0=(1 << 31) - 8)):
        assert fr(**kw) == INVALID, kw
    assert fr(D=96) == UNSUP
    assert fr(dt=3) == UNSUP
    assert fr(wb=ws - 1) == WS
    assert fr(qr=fake(5) + 8) == ALIGN
    assert fr(qr=fake(0)) == ALIAS        # in-place rotation of q is not allowed here
    assert fr(kr=fake(1)) == ALIAS
    assert fr(w=fake(3) + 256) == ALIAS   # workspace inside o
    assert fr(kr=fake(5)) == ALIAS        # q_r and k_r overlap


def test_fwd_rope_fuses_q(L):
    # Host-only: the queries are rotated inside the forward for sequences of 2048 positions or
    # more, except where the forward splits each query block's keys over two waves (bf16,
    # head_dim <= 64, at most 2048 blocks of 32 query rows).
    assert L.attn_fwd_rope_fuses_q(4, 1024, 12, 4, 64, BF16) == 0     # short
    assert L.attn_fwd_rope_fuses_q(16, 512, 12, 4, 64, BF16) == 0     # short
    assert L.attn_fwd_rope_fuses_q(2, 8192, 12, 4, 64, BF16) == 1     # 6144 blocks: no split
    assert L.attn_fwd_rope_fuses_q(8, 4096, 32, 8, 128, BF16) == 1    # head_dim 128: no split
    assert L.attn_fwd_rope_fuses_q(1, 2048, 12, 4, 64, BF16) == 0     # 768 blocks: key split
    assert L.attn_fwd_rope_fuses_q(1, 2048, 12, 4, 64, 0) == 1        # fp32: no split
    assert L.attn_fwd_rope_fuses_q(1, 64, 3, 2, 64, BF16) == -1       # Hq not a multiple of Hkv
    assert L.attn_fwd_rope_fuses_q(1, 64, 4, 2, 96, BF16) == -1       # unsupported head_dim


def test_decode_workspace_and_validation(L):
    ws = L.attn_decode_workspace_size(8, 1, 8192, 32, 8, 128, BF16)
    assert ws >= 256 and ws % 256 == 0
    assert L.attn_decode_workspace_size(1, 2, 1, 4, 2, 64, BF16) == 0      # Tq > Tk
    assert L.attn_decode_workspace_size(1, 1, 10, 3, 2, 64, BF16) == 0     # Hq % Hkv
    assert L.attn_decode_workspace_size(1, 1, 10, 4, 2, 48, BF16) == 0     # head_dim

    def dec(q=fake(0), k=fake(1), v=fake(2), o=fake(3), lse=fake(4), w=fake(5), wb=None, Tq=1, Tk=64,
            D=64, scale=0.125):
        if wb is None:
            wb = max(256, L.attn_decode_workspace_size(2, Tq, Tk, 4, 2, 64, BF16))
        return L.attn_decode(q, k, v, o, lse, w, wb, 2, Tq, Tk, 4, 2, D, scale, BF16, None)
    assert dec(k=None) == NULL
    assert dec(w=None) == NULL
    for kw in (dict(Tq=0), dict(Tq=65), dict(Tk=0, Tq=1), dict(scale=0.0)):
        assert dec(**kw) == INVALID, kw
    assert dec(D=96) == UNSUP
    assert dec(o=fake(3) + 8) == ALIGN
    assert dec(w=fake(5) + 64) == ALIGN
    big = L.attn_decode_workspace_size(2, 1, 4096, 4, 2, 64, BF16)
    assert big > 256
    assert dec(Tk=4096, wb=big - 1) == WS
    assert dec(o=fake(0)) == ALIAS
    assert dec(lse=fake(3) + 64) == ALIAS
    assert dec(w=fake(1)) == ALIAS


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 64)
    with pytest.raises(RuntimeError):
        ea.rope_apply(x)
    with pytest.raises(RuntimeError):
        ea.attn_fwd(x, x[:, :, :1].contiguous(), x[:, :, :1].contiguous())
    with pytest.raises(RuntimeError):
        ea.attn_fwd_noncausal(x, x[:, :, :1].contiguous(), x[:, :, :1].contiguous())


def gemm_call(L, a=fake(0), b=fake(1), c=fake(2), M=64, N=64, K=64, lda=None, ldb=None, ldc=None,
              ta=0, tb=0, dt=BF16):
    lda = (M if ta else K) if lda is None else lda
    ldb = (K if tb else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return L.gemm(a, b, c, M, N, K, lda, ldb, ldc, ta, tb, dt, None)


def test_gemm_validation(L):
    for name in ("a", "b", "c"):
        assert gemm_call(L, **{name: None}) == NULL, name
    for kw in (dict(M=0), dict(N=0), dict(K=0), dict(ta=2), dict(tb=-1), dict(lda=32), dict(ldb=8),
               dict(ldc=56), dict(ta=1, lda=32)):
        assert gemm_call(L, **kw) == INVALID, kw
    assert gemm_call(L, ta=1, tb=1) == UNSUP
    assert gemm_call(L, dt=5) == UNSUP
    assert gemm_call(L, N=60) == UNSUP                  # N not a multiple of 8 bf16 elements
    assert gemm_call(L, K=60) == UNSUP                  # K along rows of A
    assert gemm_call(L, M=60, ta=1) == UNSUP            # M along rows of A^T
    assert gemm_call(L, lda=68) == ALIGN
    assert gemm_call(L, c=fake(2) + 8) == ALIGN
    assert gemm_call(L, c=fake(0) + 1024) == ALIAS      # C inside A
    assert gemm_call(L, b=fake(2) + 64 * 64 * 2 - 16) == ALIAS


def test_gemm_workspace_sizes(L):
    # Split-K engages only for few output tiles (64 x 64) and a long K: slices from
    # ceil(512 / tiles), at most K steps / 8 and 8; 4 bytes per element of each partial tile.
    assert L.gemm_workspace_size(768, 768, 4096, 1, 0, BF16) == 144 * 4 * 64 * 64 * 4
    assert L.gemm_workspace_size(768, 1280, 4096, 1, 0, BF16) == 240 * 3 * 64 * 64 * 4
    assert L.gemm_workspace_size(64, 64, 8192, 0, 0, BF16) == 8 * 64 * 64 * 4
    assert L.gemm_workspace_size(64, 64, 8192, 0, 0, F32) == 8 * 64 * 64 * 4
    assert L.gemm_workspace_size(64, 64, 1024, 0, 0, BF16) == 2 * 64 * 64 * 4   # 16 K steps
    assert L.gemm_workspace_size(64, 64, 960, 0, 0, BF16) == 0                  # 15 K steps
    assert L.gemm_workspace_size(4096, 768, 1280, 0, 1, BF16) == 0              # 768 tiles
    assert L.gemm_workspace_size(8192, 8192, 8192, 0, 0, BF16) == 0             # 128 x 128 tiles
    assert L.gemm_workspace_size(64, 64, 8192, 1, 1, BF16) == 0                 # unsupported
    assert L.gemm_workspace_size(64, 60, 8192, 0, 0, BF16) == 0
    assert L.qkv_proj_bwd_workspace_size(4, 1024, 768, 12, 4, 64, BF16) == 240 * 3 * 64 * 64 * 4
    assert L.qkv_proj_bwd_workspace_size(4, 1024, 768, 12, 5, 64, BF16) == 0    # Hq % Hkv


def test_gemm_ws_validation(L):
    need = 8 * 64 * 64 * 4

    def call(ws=fake(3), nbytes=need, **kw):
        a = dict(a=fake(0), b=fake(1), c=fake(2), M=64, N=64, K=8192, ta=0, tb=0, dt=BF16)
        a.update(kw)
        lda = a["M"] if a["ta"] else a["K"]
        ldb = a["K"] if a["tb"] else a["N"]
        return L.gemm_ws(a["a"], a["b"], a["c"], a["M"], a["N"], a["K"], lda, ldb, a["N"], a["ta"], a["tb"],
                         a["dt"], ws, nbytes, None)
    assert call(a=None) == NULL
    assert call(ws=None) == NULL
    assert call(ws=fake(3) + 16) == ALIGN
    assert call(nbytes=need - 1) == WS
    assert call(ws=fake(0) + 4096) == ALIAS             # workspace inside A
    assert call(ws=fake(2) - 256) == ALIAS              # workspace running into C
    assert call(N=60) == UNSUP
    assert call(M=0) == INVALID
    # A shape that does not split needs no workspace: NULL is accepted up to the launch,
    # so only the shape checks are exercised here.
    assert call(ws=None, nbytes=0, K=512, N=60) == UNSUP


def test_qkv_proj_bwd_ws_validation(L):
    need = 240 * 3 * 64 * 64 * 4

    def call(ws=fake(7), nbytes=need, **kw):
        a = dict(x=fake(0), w=fake(1), dq=fake(2), dk=fake(3), dv=fake(4), dx=fake(5), dw=fake(6), B=4, T=1024,
                 C=768, Hq=12, Hkv=4, D=64, dt=BF16)
        a.update(kw)
        return L.qkv_proj_bwd_ws(a["x"], a["w"], a["dq"], a["dk"], a["dv"], a["dx"], a["dw"], a["B"], a["T"],
                                 a["C"], a["Hq"], a["Hkv"], a["D"], a["dt"], ws, nbytes, None)
    assert call(dx=None) == NULL
    assert call(ws=None) == NULL
    assert call(ws=fake(7) + 128) == ALIGN
    assert call(nbytes=need - 256) == WS
    assert call(ws=fake(6)) == ALIAS                    # workspace over dw
    assert call(Hq=5) == INVALID


def qkv(L, x=fake(0), w=fake(1), q=fake(2), k=fake(3), v=fake(4), B=2, T=16, C=64, Hq=4, Hkv=2, D=16,
        dt=BF16, rope=1, base=1e4, pos0=0):
    return L.qkv_proj(x, w, q, k, v, B, T, C, Hq, Hkv, D, dt, rope, base, pos0, None)


def test_qkv_proj_validation(L):
    for name in ("x", "w", "q", "k", "v"):
        assert qkv(L, **{name: None}) == NULL, name
    for kw in (dict(B=0), dict(T=0), dict(C=0), dict(Hq=3), dict(D=1), dict(rope=2), dict(base=1.0),
               dict(base=float("nan")), dict(pos0=-1)):
        assert qkv(L, **kw) == INVALID, kw
    for kw in (dict(C=60), dict(D=12), dict(D=264), dict(dt=3)):
        assert qkv(L, **kw) == UNSUP, kw
    assert qkv(L, k=fake(3) + 4) == ALIGN
    assert qkv(L, q=fake(0) + 256) == ALIAS             # q over x
    assert qkv(L, v=fake(3) + 512) == ALIAS             # v over k


def test_qkv_proj_bwd_validation(L):
    def call(**kw):
        a = dict(x=fake(0), w=fake(1), dq=fake(2), dk=fake(3), dv=fake(4), dx=fake(5), dw=fake(6), B=2, T=16,
                 C=64, Hq=4, Hkv=2, D=16, dt=BF16)
        a.update(kw)
        return L.qkv_proj_bwd(a["x"], a["w"], a["dq"], a["dk"], a["dv"], a["dx"], a["dw"], a["B"], a["T"],
                              a["C"], a["Hq"], a["Hkv"], a["D"], a["dt"], None)
    for name in ("x", "w", "dq", "dk", "dv", "dx", "dw"):
        assert call(**{name: None}) == NULL, name
    assert call(Hq=3) == INVALID
    assert call(C=20) == UNSUP
    assert call(dx=fake(5) + 2) == ALIGN
    assert call(dx=fake(1)) == ALIAS                    # dx over w
    assert call(dw=fake(5) + 64) == ALIAS               # dw over dx


def test_noalloc_validation(L):
    # attn_bwd_noalloc validates like attn_bwd (no workspace) and rejects a problem whose D_t
    # exceeds the static scratch before any HIP call.
    def nb(q=fake(0), dq=fake(6), dk=fake(7), B=2, T=16, Hq=4, Hkv=2, D=64, scale=0.125, dt=BF16):
        return L.attn_bwd_noalloc(q, fake(1), fake(2), fake(3), fake(4), fake(5), dq, dk, fake(8),
                                  B, T, Hq, Hkv, D, scale, dt, None)
    assert nb(q=None) == NULL
    assert nb(Hq=3) == INVALID
    assert nb(D=48) == UNSUP
    assert nb(dk=fake(7) + 4) == ALIGN
    assert nb(dq=fake(0)) == ALIAS
    # B * Hq * T = 4 Mi rows fits exactly (16 MiB of D_t); one more position does not.  With
    # these sizes the fake tensors overlap, so the scratch check must come first.
    assert nb(B=64, Hq=64, Hkv=64, T=1025, D=32) == SCRATCH
    assert ea.NOALLOC_SCRATCH_BYTES == 16 << 20
    assert L.attn_bwd_workspace_size(64, 1024, 64, 64, 32, BF16) == ea.NOALLOC_SCRATCH_BYTES
