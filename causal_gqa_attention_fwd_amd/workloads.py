"""Seeded synthetic inputs shaped like the attention layers the NanoEuler pages describe.

This module draws random numbers and casts them; it holds none of the attention or RoPE
arithmetic, so both the HIP path and the CPU oracle can be fed from it.

Recipe (per workload): ``numpy.random.default_rng(seed)`` draws ``standard_normal`` in
float32 for Q_raw, K_raw, V and dO, in that order.  Then the workload's structure is
applied (a 1/sqrt(2) scale, or a set of "peaky" key rows multiplied by 8, chosen with
``rng.choice`` without replacement after dO), and bf16 workloads are rounded with
torch's round-to-nearest-even cast.  Everything is returned as CPU torch tensors.

Shapes come from the pages: the small CPU model (dim 128, 4 query / 2 KV heads, context
128) and the GPU model (dim 768, 12 query / 4 KV heads, context 512) of the NanoEuler model
table ("NanoEuler: CとCUDAでゼロから構築されたGPT-2スケールのLLM", "モデル構成"), and the
batch-4 / 1024-token benchmark shape of the blog's performance comparison (smartinfralog,
"性能对比" and its JSON model config).  The long-context and 32/8-head, head-dim-128
workloads extend those shapes; there is no dataset behind any of them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    dtype: str            # "f32" or "bf16"
    seed: int
    base: float = 10000.0
    qkv_scale: float = 1.0        # multiply Q_raw, K_raw, V by this (in fp32) before casting
    peaky_frac: float = 0.0       # fraction of (b, t, kv) key rows multiplied by peaky_mult
    peaky_mult: float = 8.0
    note: str = field(default="", compare=False)

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def pairs(self) -> int:
        """Unmasked causal (t, s) pairs over all batches and query heads."""
        return self.B * self.Hq * self.T * (self.T + 1) // 2

    def flops_fwd(self) -> int:
        return 4 * self.D * self.pairs

    def flops_bwd(self) -> int:
        return 10 * self.D * self.pairs

    def flops_total(self) -> int:
        return 14 * self.D * self.pairs

    def describe(self) -> dict:
        return {"workload": self.name, "batch": self.B, "seq_len": self.T, "q_heads": self.Hq,
                "kv_heads": self.Hkv, "head_dim": self.D, "io_dtype": self.dtype,
                "rope_base": self.base, "seed": self.seed}


WORKLOADS = {
    # Small CPU model attention layer: dim 128, 4 Q / 2 KV heads (head_dim 32), context 128.
    "tiny_cpu_model": Workload("tiny_cpu_model", 4, 128, 4, 2, 32, "f32", 1001),
    # GPU pipeline attention layer: dim 768, 12 Q / 4 KV heads (head_dim 64), context 512.
    "gpu_model_f32": Workload("gpu_model_f32", 16, 512, 12, 4, 64, "f32", 1002),
    "gpu_model_bf16": Workload("gpu_model_bf16", 16, 512, 12, 4, 64, "bf16", 1002),
    # Blog benchmark shape: batch 4, sequence 1024, 12 Q / 4 KV heads, head_dim 64.
    "blog_t1024": Workload("blog_t1024", 4, 1024, 12, 4, 64, "bf16", 1003,
                           qkv_scale=1.0 / math.sqrt(2.0)),
    # Long context with 1% of key rows scaled by 8 (peaky logits for the online softmax).
    "long_t8192": Workload("long_t8192", 2, 8192, 12, 4, 64, "bf16", 1004, peaky_frac=0.01),
    # Scaled GQA: 32 Q / 8 KV heads, head_dim 128, RoPE base 500000.
    "gqa_t4096_d128": Workload("gqa_t4096_d128", 8, 4096, 32, 8, 128, "bf16", 1005, base=500000.0),
}


def torch_dtype(dt: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dt]


def peaky_rows(w: Workload, rng: np.random.Generator) -> np.ndarray:
    """Flat (b*T + t)*Hkv + kv indices of the key rows to scale (drawn from rng)."""
    n_rows = w.B * w.T * w.Hkv
    count = int(round(w.peaky_frac * n_rows))
    if count == 0:
        return np.zeros((0,), dtype=np.int64)
    return np.sort(rng.choice(n_rows, size=count, replace=False)).astype(np.int64)


def make_inputs(w: Workload | str, dtype: str | None = None) -> dict:
    """Seeded raw inputs of a workload as CPU torch tensors.

    Returns {"q_raw", "k_raw", "v", "dout"} ([B,T,H,D], the workload's dtype unless
    ``dtype`` overrides it) and "peaky" (the scaled key-row indices).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    dt = dtype or w.dtype
    rng = np.random.default_rng(w.seed)
    qshape = (w.B, w.T, w.Hq, w.D)
    kshape = (w.B, w.T, w.Hkv, w.D)
    q = rng.standard_normal(qshape, dtype=np.float32)
    k = rng.standard_normal(kshape, dtype=np.float32)
    v = rng.standard_normal(kshape, dtype=np.float32)
    do = rng.standard_normal(qshape, dtype=np.float32)
    if w.qkv_scale != 1.0:
        s = np.float32(w.qkv_scale)
        q *= s
        k *= s
        v *= s
    rows = peaky_rows(w, rng)
    if rows.size:
        k.reshape(-1, w.D)[rows] *= np.float32(w.peaky_mult)
    tdt = torch_dtype(dt)
    out = {name: torch.from_numpy(a).to(tdt) for name, a in
           (("q_raw", q), ("k_raw", k), ("v", v), ("dout", do))}
    out["peaky"] = torch.from_numpy(rows)
    return out


def make_random(shape, seed: int, dtype: str = "f32", scale: float = 1.0) -> torch.Tensor:
    """One seeded N(0, scale^2) tensor (for edge-shape sweeps)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return torch.from_numpy(a).to(torch_dtype(dtype))


@dataclass(frozen=True)
class DecodeWorkload:
    """One generation step against a KV cache: Tq new query rows per sequence and a cache
    of Tk positions (those rows included)."""
    name: str
    B: int
    Tq: int
    Tk: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    seed: int

    def hbm_bytes(self) -> int:
        """Algorithmic bytes of one call: read q and the K/V cache, write o and lse."""
        es = 4 if self.dtype == "f32" else 2
        return (2 * self.B * self.Tq * self.Hq * self.D * es + 2 * self.B * self.Tk * self.Hkv * self.D * es
                + self.B * self.Hq * self.Tq * 4)

    def describe(self) -> dict:
        return {"workload": self.name, "batch": self.B, "new_tokens": self.Tq, "cache_len": self.Tk,
                "q_heads": self.Hq, "kv_heads": self.Hkv, "head_dim": self.D, "io_dtype": self.dtype,
                "seed": self.seed}


DECODE_WORKLOADS = {
    # One new token per sequence against an 8192-position cache, 32 Q / 8 KV heads, head_dim 128
    # (the scaled GQA shape above, generating).
    "decode_b8_tk8192": DecodeWorkload("decode_b8_tk8192", 8, 1, 8192, 32, 8, 128, "bf16", 1006),
    # Four new tokens (multi-token speculative decoding) for the 12 Q / 4 KV GPU model.
    "decode_mtp4_b16_tk1024": DecodeWorkload("decode_mtp4_b16_tk1024", 16, 4, 1024, 12, 4, 64, "bf16", 1007),
}


def make_decode_inputs(w: DecodeWorkload | str) -> dict:
    """Seeded N(0,1) q [B,Tq,Hq,D] and cache k, v [B,Tk,Hkv,D] (drawn in that order) as CPU
    torch tensors of the workload's dtype."""
    if isinstance(w, str):
        w = DECODE_WORKLOADS[w]
    rng = np.random.default_rng(w.seed)
    q = rng.standard_normal((w.B, w.Tq, w.Hq, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, w.Tk, w.Hkv, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, w.Tk, w.Hkv, w.D), dtype=np.float32)
    tdt = torch_dtype(w.dtype)
    return {"q": torch.from_numpy(q).to(tdt), "k": torch.from_numpy(k).to(tdt), "v": torch.from_numpy(v).to(tdt)}



def make_proj_inputs(w: Workload | str, seed_offset: int = 500) -> dict:
    """Seeded inputs of the projections around one attention layer of workload w: hidden
    states x [B, T, C] and upstream gradient dy [B, T, C] ~ N(0, 1), and random-init weights
    w_qkv [C, (Hq + 2 Hkv) D] and w_o [Hq D, C] ~ N(0, 1/C) (model dimension C = Hq D),
    drawn in that order from ``default_rng(seed + seed_offset)`` in float32, then cast to the
    workload's dtype.  There are no trained weights behind them."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    C = w.Hq * w.D
    rng = np.random.default_rng(w.seed + seed_offset)
    x = rng.standard_normal((w.B, w.T, C), dtype=np.float32)
    wq = rng.standard_normal((C, (w.Hq + 2 * w.Hkv) * w.D), dtype=np.float32) * np.float32(1.0 / math.sqrt(C))
    wo = rng.standard_normal((w.Hq * w.D, C), dtype=np.float32) * np.float32(1.0 / math.sqrt(C))
    dy = rng.standard_normal((w.B, w.T, C), dtype=np.float32)
    tdt = torch_dtype(w.dtype)
    return {k: torch.from_numpy(a).to(tdt) for k, a in (("x", x), ("w_qkv", wq), ("w_o", wo), ("dy", dy))}
