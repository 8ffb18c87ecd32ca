#!/usr/bin/env python3
"""Benchmark of libeuler_attn: one step = the whole causal-GQA-attention hot path on one
batch of seeded synthetic inputs already resident in HBM:

    RoPE(Q), RoPE(K) (one launch) -> attn_fwd -> attn_bwd_rope: pre-pass (D_t and the RoPE
    table), then dQ/dK/dV with RoPE^-1 applied to dQ and dK as they are stored

Throughput is reported as TFLOP/s at the exact causal FLOP count 14 * D * B * Hq * T(T+1)/2
(4D forward + 10D backward per unmasked query/key pair) and as a fraction of the MI355X
dense bf16 MFMA peak.  Default workload: batch 4, T = 1024, 12 query / 4 KV heads,
head_dim 64, bf16 I/O (the blog's benchmark shape).

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--extra NAMES]
                    [--decode NAMES] [--noncausal NAMES] [--proj NAMES]

Besides the headline step, the line carries the other timed paths of the library: the same
step on the other workloads ('extra': by default T = 8192, the head_dim-128 GQA shape, the
GPU-pipeline layer in bf16 and fp32, and the tiny CPU model), attention against a KV cache
('decode'), the
attention without the causal mask ('noncausal') and the projections on either side of the
attention, forward and backward ('projections').
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal GQA attention fwd+bwd TFLOP/s and % of MFMA peak (T=1024, 12Q/4KV, d=64)"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}   # MI355X dense MFMA (256 CU x 2.4 GHz)
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = {
    "attn_fwd": ["causal_gqa_attention_fwd_amd/csrc/attn_fwd.hip", "causal_gqa_attention_fwd_amd/csrc/ea_common.h"],
    "attn_bwd_main": ["causal_gqa_attention_fwd_amd/csrc/attn_bwd.hip", "causal_gqa_attention_fwd_amd/csrc/ea_common.h"],
    "attn_decode": ["causal_gqa_attention_fwd_amd/csrc/attn_decode.hip", "causal_gqa_attention_fwd_amd/csrc/ea_common.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sources_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Step:
    """Preallocated buffers and the five launches of one step, called through the C ABI."""

    def __init__(self, w, inp, torch, ea):
        self.w = w
        dev = torch.device("cuda", 0)
        self.q_raw = inp["q_raw"].to(dev)
        self.k_raw = inp["k_raw"].to(dev)
        self.v = inp["v"].to(dev)
        self.do = inp["dout"].to(dev)
        self.qr = torch.empty_like(self.q_raw)
        self.kr = torch.empty_like(self.k_raw)
        self.o = torch.empty_like(self.q_raw)
        self.lse = torch.empty((w.B, w.Hq, w.T), device=dev, dtype=torch.float32)
        self.dq_raw = torch.empty_like(self.q_raw)
        self.dk_raw = torch.empty_like(self.k_raw)
        self.dv = torch.empty_like(self.v)
        dtc = ea.EA_F32 if w.dtype == "f32" else ea.EA_BF16
        nws = ea.attn_bwd_rope_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D, self.q_raw.dtype)
        self.ws = torch.empty(nws, device=dev, dtype=torch.uint8)
        L = ea.lib()
        scale = 1.0 / (w.D ** 0.5)
        stream = torch.cuda.current_stream(dev).cuda_stream
        B, T, Hq, Hkv, D, base = w.B, w.T, w.Hq, w.Hkv, w.D, w.base
        p = lambda t: t.data_ptr()  # noqa: E731
        # (name, ctypes function, arguments) for each launch, in order.  The backward returns the
        # gradients of the raw (pre-RoPE) Q and K: the RoPE backward is fused into its stores.
        self.calls = [
            ("rope_qk", L.rope_apply_qk, (p(self.q_raw), p(self.qr), Hq, p(self.k_raw), p(self.kr), Hkv, B, T,
                                          D, dtc, base, 0, 0, stream)),
            ("attn_fwd", L.attn_fwd, (p(self.qr), p(self.kr), p(self.v), p(self.o), p(self.lse), B, T, Hq,
                                      Hkv, D, scale, dtc, stream)),
            ("attn_bwd_pre", L.attn_bwd_rope_preprocess, (p(self.o), p(self.do), p(self.ws), nws, B, T, Hq,
                                                          Hkv, D, dtc, base, 0, stream)),
            ("attn_bwd_main", L.attn_bwd_rope_main, (p(self.qr), p(self.kr), p(self.v), p(self.lse),
                                                     p(self.do), p(self.dq_raw), p(self.dk_raw), p(self.dv),
                                                     p(self.ws), nws, B, T, Hq, Hkv, D, scale, dtc, stream)),
        ]

    def run(self):
        for name, fn, args in self.calls:
            st = fn(*args)
            if st != 0:
                raise RuntimeError("%s returned status %d" % (name, st))

    def run_with_events(self, torch, events):
        for (name, fn, args), (e0, e1) in zip(self.calls, events):
            e0.record()
            st = fn(*args)
            e1.record()
            if st != 0:
                raise RuntimeError("%s returned status %d" % (name, st))


def algorithmic(w) -> dict:
    """Per-launch algorithmic FLOPs / bytes of each kernel of the step."""
    es = 4 if w.dtype == "f32" else 2
    qb = w.B * w.T * w.Hq * w.D * es
    kb = w.B * w.T * w.Hkv * w.D * es
    lse = w.B * w.Hq * w.T * 4
    return {
        "rope_qk": {"bytes": 2 * qb + 2 * kb},
        "attn_fwd": {"flops": w.flops_fwd(), "bytes": qb + 2 * kb + qb + lse},
        # D_t (read O and dO, write D_t) and the RoPE (cos, sin) table, fp32 [T, D/2, 2].
        "attn_bwd_pre": {"bytes": 2 * qb + lse + w.T * w.D * 4},
        # The backward's 10D per pair (S recompute, dP, dV, dK, dQ); the dQ-role workgroups
        # recompute S and dP once more (4D per pair executed, not counted as algorithmic).
        # The inverse RoPE on dQ and dK is applied before their stores (no extra HBM pass).
        "attn_bwd_main": {"flops": 10 * w.D * w.pairs, "executed_flops": 14 * w.D * w.pairs,
                          "bytes": 2 * qb + 2 * kb + 2 * lse + qb + 2 * kb},
    }


def time_workload(name, steps, warmup, torch, ea, W):
    w = W.WORKLOADS[name]
    log("[bench] workload %s: generating inputs" % name)
    inp = W.make_inputs(w)
    step = Step(w, inp, torch, ea)
    log("[bench] %s: %d warmup steps" % (name, warmup))
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    # Timed region: exactly `steps` steps, synchronised on both sides.
    log("[bench] %s: timing %d steps" % (name, steps))
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        step.run()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / steps
    # Per-kernel durations: the same steps again with HIP events around every launch, on the
    # stream the kernels are launched on (the current stream).
    log("[bench] %s: per-kernel events over %d steps" % (name, steps))
    per = {n: [] for n, _, _ in step.calls}
    for _ in range(steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in step.calls]
        step.run_with_events(torch, ev)
        torch.cuda.synchronize()
        for (n, _, _), (a, b) in zip(step.calls, ev):
            per[n].append(a.elapsed_time(b))
    kern_us = {n: 1000.0 * statistics.mean(v) for n, v in per.items()}
    return w, step, ms, wall, kern_us


def measured_traffic(name, workload):
    """HBM bytes per launch of entry point `name` on `workload` from the committed counter
    summary, or None: entries are keyed "<entry point>@<workload>" and count only while the
    kernel sources still hash to the value recorded with them."""
    try:
        with open(TRAFFIC_FILE) as f:
            tc = json.load(f)
        ent = tc.get("kernels", {}).get("%s@%s" % (name, workload))
        if (ent and name in KERNEL_SOURCES
                and ent.get("source_sha") == sources_sha(KERNEL_SOURCES[name])):
            return ent.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        pass
    return None


def roofline_for(w, kern_us, name):
    alg = algorithmic(w)[name]
    dur_s = kern_us[name] * 1e-6
    traffic = measured_traffic(name, w.name)
    if "flops" in alg:
        achieved = alg["flops"] / dur_s / 1e12
        peak = PEAK_TFLOPS[w.dtype]
        out = {"kernel": name, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
               "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
               "algorithmic_flops_per_launch": alg["flops"], "algorithmic_bytes_per_launch": alg["bytes"],
               "avg_launch_us": round(kern_us[name], 2)}
        if "executed_flops" in alg:
            out["executed_flops_per_launch"] = alg["executed_flops"]
            out["executed_tflops"] = round(alg["executed_flops"] / dur_s / 1e12, 2)
        return out
    achieved = alg["bytes"] / dur_s / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": alg["bytes"], "avg_launch_us": round(kern_us[name], 2)}


def time_decode(name, steps, warmup, torch, ea, W):
    """attn_decode on a decode workload: average microseconds per call over `steps` calls with
    inputs resident in HBM, and the algorithmic HBM rate (q and the K/V cache read, o and lse
    written) against the 8 TB/s peak."""
    w = W.DECODE_WORKLOADS[name]
    log("[bench] decode workload %s" % name)
    inp = W.make_decode_inputs(w)
    dev = torch.device("cuda", 0)
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Tq), device=dev, dtype=torch.float32)
    L = ea.lib()
    dtc = ea.EA_F32 if w.dtype == "f32" else ea.EA_BF16
    nws = max(256, L.attn_decode_workspace_size(w.B, w.Tq, w.Tk, w.Hq, w.Hkv, w.D, dtc))
    ws = torch.empty(nws, device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr(), nws,
            w.B, w.Tq, w.Tk, w.Hq, w.Hkv, w.D, 1.0 / (w.D ** 0.5), dtc, stream)
    for _ in range(warmup):
        if L.attn_decode(*args) != 0:
            raise RuntimeError("attn_decode failed")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        L.attn_decode(*args)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1000.0 / steps
    gbs = w.hbm_bytes() / (us * 1e-6) / 1e9
    return {"config": w.describe(), "calls": steps, "us_per_call": round(us, 2),
            "hbm_bytes_per_call": w.hbm_bytes(),
            "roofline": {"kernel": "attn_decode (one launch, or chunk partials + merge)", "bound": "hbm",
                         "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("attn_decode", name)}}


def time_fwd_rope(name, steps, warmup, torch, ea, W):
    """The forward half of the step two ways on a workload's raw inputs: rope_apply_qk then
    attn_fwd (the headline step's form), and attn_fwd_rope (K rotated in its own launch, which
    also writes the (cos, sin) table; Q rotated inside the forward as it loads).  Microseconds
    per call from HIP events around `steps` back-to-back calls on the launch stream."""
    w = W.WORKLOADS[name]
    log("[bench] fused-RoPE forward, workload %s" % name)
    inp = W.make_inputs(w)
    dev = torch.device("cuda", 0)
    q, k, v = (inp[x].to(dev) for x in ("q_raw", "k_raw", "v"))
    qr, kr, o = torch.empty_like(q), torch.empty_like(k), torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.T), device=dev, dtype=torch.float32)
    L = ea.lib()
    dtc = ea.EA_F32 if w.dtype == "f32" else ea.EA_BF16
    nws = L.attn_fwd_rope_workspace_size(w.T, w.D)
    ws = torch.empty(nws, device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev).cuda_stream
    scale = 1.0 / (w.D ** 0.5)
    p = lambda t: t.data_ptr()  # noqa: E731

    def unfused():
        if (L.rope_apply_qk(p(q), p(qr), w.Hq, p(k), p(kr), w.Hkv, w.B, w.T, w.D, dtc, w.base, 0, 0, stream)
                or L.attn_fwd(p(qr), p(kr), p(v), p(o), p(lse), w.B, w.T, w.Hq, w.Hkv, w.D, scale, dtc, stream)):
            raise RuntimeError("rope_apply_qk / attn_fwd failed")

    def fused():
        if L.attn_fwd_rope(p(q), p(k), p(v), p(o), p(lse), p(qr), p(kr), p(ws), nws, w.B, w.T, w.Hq, w.Hkv,
                           w.D, scale, dtc, w.base, 0, stream):
            raise RuntimeError("attn_fwd_rope failed")

    res = {}
    for label, fn in (("us_unfused", unfused), ("us_fused", fused)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        res[label] = round(1000.0 * t0.elapsed_time(t1) / steps, 2)
    return {"config": w.describe(), "calls": steps, **res,
            "note": "two launches either way (attn_fwd_rope rotates Q with K in its first launch where attn_fwd_rope_fuses_q is 0); the steps keep rope_apply_qk + attn_fwd, since inside the whole step the two forms measured the same"}


def time_noncausal(name, steps, warmup, torch, ea, W):
    """attn_fwd_noncausal then attn_bwd_noncausal (its pre-pass and main launch) on the inputs
    of a workload (no RoPE): TFLOP/s at 14 * D * B * Hq * T^2 (every query/key pair), with the
    forward's and the backward's average durations from HIP events on the launch stream."""
    w = W.WORKLOADS[name]
    log("[bench] non-causal workload %s" % name)
    inp = W.make_inputs(w)
    dev = torch.device("cuda", 0)
    q, k, v, do = (inp[x].to(dev) for x in ("q_raw", "k_raw", "v", "dout"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.T), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    L = ea.lib()
    dtc = ea.EA_F32 if w.dtype == "f32" else ea.EA_BF16
    nws = L.attn_bwd_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D, dtc)
    ws = torch.empty(nws, device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev).cuda_stream
    scale = 1.0 / (w.D ** 0.5)
    p = lambda t: t.data_ptr()  # noqa: E731
    fwd = (p(q), p(k), p(v), p(o), p(lse), w.B, w.T, w.Hq, w.Hkv, w.D, scale, dtc, stream)
    bwd = (p(q), p(k), p(v), p(o), p(lse), p(do), p(dq), p(dk), p(dv), p(ws), nws, w.B, w.T, w.Hq,
           w.Hkv, w.D, scale, dtc, stream)

    def run(ev=None):
        for i, (fn, a) in enumerate(((L.attn_fwd_noncausal, fwd), (L.attn_bwd_noncausal, bwd))):
            if ev:
                ev[i][0].record()
            if fn(*a) != 0:
                raise RuntimeError("non-causal attention failed")
            if ev:
                ev[i][1].record()
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        run()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    per = [[], []]
    for _ in range(steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2)]
        run(ev)
        torch.cuda.synchronize()
        for i in range(2):
            per[i].append(ev[i][0].elapsed_time(ev[i][1]))
    pairs = w.B * w.Hq * w.T * w.T
    flops = 14 * w.D * pairs
    tf = flops / (ms * 1e-3) / 1e12
    fwd_us, bwd_us = (1000.0 * statistics.mean(x) for x in per)
    return {"config": dict(w.describe(), causal=False), "steps": steps, "ms_per_step": round(ms, 4),
            "value": round(tf, 3), "unit": "TFLOP/s", "frac_of_peak": round(tf / PEAK_TFLOPS[w.dtype], 4),
            "flops_convention": "14*D*B*Hq*T^2",
            "kernel_us": {"attn_fwd_noncausal": round(fwd_us, 2), "attn_bwd_noncausal": round(bwd_us, 2)},
            "fwd_tflops": round(4 * w.D * pairs / (fwd_us * 1e-6) / 1e12, 2),
            "bwd_tflops": round(10 * w.D * pairs / (bwd_us * 1e-6) / 1e12, 2)}


def time_projections(name, steps, warmup, torch, ea, W):
    """The projections around one attention layer of a workload (model dimension C = Hq D):
    qkv_proj with RoPE (x [B*T, C] by w_qkv [C, (Hq + 2 Hkv) D]), the output projection
    y = o W_o, its backward (do = dy W_o^T, dW_o = o^T dy) and qkv_proj_bwd (dx and dW_qkv).
    The two weight gradients are timed plain and with split K (gemm_ws, qkv_proj_bwd_ws); the
    totals count the split ones, which a layer would call.  Average microseconds per call from
    HIP events on the launch stream, and TFLOP/s at 2 M N K per product against the dense
    MFMA peak of the dtype."""
    w = W.WORKLOADS[name]
    log("[bench] projections of workload %s" % name)
    inp = W.make_proj_inputs(w)
    dev = torch.device("cuda", 0)
    x, wq, wo, dy = (inp[k].to(dev) for k in ("x", "w_qkv", "w_o", "dy"))
    B, T, C, Hq, Hkv, D = w.B, w.T, w.Hq * w.D, w.Hq, w.Hkv, w.D
    M, Nq = B * T, (Hq + 2 * Hkv) * D
    q = torch.empty((B, T, Hq, D), device=dev, dtype=x.dtype)
    k = torch.empty((B, T, Hkv, D), device=dev, dtype=x.dtype)
    v = torch.empty_like(k)
    o = W.make_random((B * T, Hq * D), w.seed + 700, w.dtype).to(dev)
    y = torch.empty((M, C), device=dev, dtype=x.dtype)
    do = torch.empty_like(o)
    dwo = torch.empty_like(wo)
    dx = torch.empty_like(x)
    dwq = torch.empty_like(wq)
    L = ea.lib()
    dtc = ea.EA_F32 if w.dtype == "f32" else ea.EA_BF16
    stream = torch.cuda.current_stream(dev).cuda_stream
    p = lambda t: t.data_ptr()  # noqa: E731
    # Split-K workspaces of the two weight gradients (few output tiles, K = B T).
    ws_o = L.gemm_workspace_size(Hq * D, C, M, 1, 0, dtc)
    ws_q = L.qkv_proj_bwd_workspace_size(B, T, C, Hq, Hkv, D, dtc)
    ws = torch.empty(max(ws_o, ws_q, 256), device=dev, dtype=torch.uint8)
    calls = [
        ("qkv_proj_rope", 2 * M * Nq * C, L.qkv_proj,
         (p(x), p(wq), p(q), p(k), p(v), B, T, C, Hq, Hkv, D, dtc, 1, w.base, 0, stream)),
        ("out_proj", 2 * M * C * Hq * D, L.gemm,
         (p(o), p(wo), p(y), M, C, Hq * D, Hq * D, C, C, 0, 0, dtc, stream)),
        ("out_proj_bwd_dx", 2 * M * C * Hq * D, L.gemm,
         (p(dy), p(wo), p(do), M, Hq * D, C, C, C, Hq * D, 0, 1, dtc, stream)),
        ("out_proj_bwd_dw", 2 * M * C * Hq * D, L.gemm,
         (p(o), p(dy), p(dwo), Hq * D, C, M, Hq * D, C, C, 1, 0, dtc, stream)),
        ("out_proj_bwd_dw_splitk", 2 * M * C * Hq * D, L.gemm_ws,
         (p(o), p(dy), p(dwo), Hq * D, C, M, Hq * D, C, C, 1, 0, dtc, p(ws), ws.numel(), stream)),
        ("qkv_proj_bwd", 2 * 2 * M * Nq * C, L.qkv_proj_bwd,
         (p(x), p(wq), p(q), p(k), p(v), p(dx), p(dwq), B, T, C, Hq, Hkv, D, dtc, stream)),
        ("qkv_proj_bwd_splitk", 2 * 2 * M * Nq * C, L.qkv_proj_bwd_ws,
         (p(x), p(wq), p(q), p(k), p(v), p(dx), p(dwq), B, T, C, Hq, Hkv, D, dtc, p(ws), ws.numel(), stream)),
    ]
    out = {"config": dict(w.describe(), model_dim=C), "calls": steps, "kernels": {}}
    total_us, total_flops = 0.0, 0
    for cname, flops, fn, args in calls:
        for _ in range(warmup):
            if fn(*args) != 0:
                raise RuntimeError("%s failed" % cname)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn(*args)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / steps
        tf = flops / (us * 1e-6) / 1e12
        if cname not in ("out_proj_bwd_dw", "qkv_proj_bwd"):  # superseded by the split-K calls
            total_us += us
            total_flops += flops
        out["kernels"][cname] = {"us_per_call": round(us, 2), "flops": flops, "tflops": round(tf, 2),
                                 "frac_of_peak": round(tf / PEAK_TFLOPS[w.dtype], 4)}
    out["total_us"] = round(total_us, 2)
    out["total_tflops"] = round(total_flops / (total_us * 1e-6) / 1e12, 2)
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, W):
    """The oracle (plain float64 C++, OpenMP) on the host cores, timed as it stands.

    On the headline workload with every available thread: the whole step (RoPE on Q and K,
    forward, analytic backward, inverse RoPE on dQ and dK) and the forward alone (RoPE and
    forward).  Then one thread on the three smaller workloads' whole step (the tiny CPU model
    in full; the GPU-pipeline layer and the T=1024 shape on one (batch, K/V head) slice, scaled
    by B * Hkv: every slice does the same work).  Inputs are the bench's seeded inputs in
    float64; generation and conversion are outside the timed calls."""
    import numpy as np
    import torch
    from oracle import oracle

    def arrays(wl, b=None, kv=None):
        inp = W.make_inputs(wl)
        out = {}
        for k_, v_ in inp.items():
            if k_ == "peaky":
                continue
            a = v_.to(dtype=torch.float64).numpy()
            if b is not None:
                g = wl.Hq // wl.Hkv
                hs = slice(kv * g, (kv + 1) * g) if v_.shape[2] == wl.Hq else slice(kv, kv + 1)
                a = a[b:b + 1, :, hs]
            out[k_] = np.ascontiguousarray(a)
        return out

    def fwd(wl, a):
        qr = oracle.rope(a["q_raw"], wl.base)
        kr = oracle.rope(a["k_raw"], wl.base)
        oracle.attn_fwd(qr, kr, a["v"])
        return qr, kr

    def whole(wl, a):
        qr, kr = fwd(wl, a)
        dq, dk, _ = oracle.attn_bwd(qr, kr, a["v"], a["dout"])
        oracle.rope(dq, wl.base, inverse=True)
        oracle.rope(dk, wl.base, inverse=True)

    def timed(fn, budget=10.0, reps=3):
        times, t_all = [], time.perf_counter()
        while True:
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
            spent = time.perf_counter() - t_all
            if len(times) >= reps or spent + times[-1] > budget:
                break
        return statistics.median(times), len(times)

    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    oracle.set_num_threads(threads)
    cores = oracle.num_threads()
    a = arrays(w)
    t_step, n_step = timed(lambda: whole(w, a))
    t_fwd, n_fwd = timed(lambda: fwd(w, a))
    single = {}
    oracle.set_num_threads(1)
    try:
        for name in ("tiny_cpu_model", "gpu_model_f32", "blog_t1024"):
            wl = W.WORKLOADS[name]
            sliced = name != "tiny_cpu_model"
            aa = arrays(wl, 0, 0) if sliced else arrays(wl)
            scale = wl.B * wl.Hkv if sliced else 1
            ts, _ = timed(lambda: whole(wl, aa), budget=5.0, reps=1)
            single[name] = {"seconds_per_step": round(ts * scale, 3),
                            "tflops": round(wl.flops_total() / (ts * scale) / 1e12, 6),
                            "timed": ("one (batch, K/V head) slice x %d" % scale) if sliced else "whole step"}
    finally:
        oracle.set_num_threads(threads)
    return {"value": round(w.flops_total() / t_step / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": "whole step of workload %s (RoPE q/k, fwd, analytic bwd, inverse RoPE), float64, "
                      "%d threads, median of %d run(s)" % (w.name, cores, n_step),
            "seconds_per_step": round(t_step, 3),
            "forward_only": {"seconds": round(t_fwd, 3), "tflops": round(w.flops_fwd() / t_fwd / 1e12, 6),
                             "runs": n_fwd, "what": "RoPE on q and k, then the forward"},
            "single_thread": single}


def time_extra(args, torch, ea, W) -> dict:
    """The other workloads, each timed like the headline step (fewer steps)."""
    extra = {}
    for name in [x for x in args.extra.split(",") if x and x != args.workload]:
        steps = max(5, args.steps // 5)
        we, _, mse, _, ke = time_workload(name, steps, max(2, args.warmup // 5), torch, ea, W)
        tf = we.flops_total() / (mse * 1e-3) / 1e12
        dom = max(ke, key=ke.get)
        extra[name] = {"value": round(tf, 3), "unit": "TFLOP/s", "ms_per_step": round(mse, 4),
                       "frac_of_peak": round(tf / PEAK_TFLOPS[we.dtype], 4), "steps": steps,
                       "config": we.describe(),
                       "kernel_us": {k: round(v, 2) for k, v in ke.items()},
                       "roofline": roofline_for(we, ke, dom),
                       "roofline_attn_fwd": roofline_for(we, ke, "attn_fwd"),
                       "roofline_attn_bwd_main": roofline_for(we, ke, "attn_bwd_main")}
    return extra


def time_cold(name, steps, warmup, torch, ea, W):
    """The headline step with cold caches: before every step a 512 MiB buffer is written
    (twice the 256 MB last-level cache of the chip), so the step's inputs come from HBM; HIP
    events on the launch stream bracket the step alone, not the eviction."""
    w = W.WORKLOADS[name]
    log("[bench] cold-cache step, workload %s" % name)
    inp = W.make_inputs(w)
    step = Step(w, inp, torch, ea)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    evs = []
    for i in range(steps):
        flush.fill_(i & 0xff)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        step.run()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = statistics.mean(a.elapsed_time(b) for a, b in evs)
    tf = w.flops_total() / (ms * 1e-3) / 1e12
    return {"value": round(tf, 3), "unit": "TFLOP/s", "ms_per_step": round(ms, 4),
            "frac_of_peak": round(tf / PEAK_TFLOPS[w.dtype], 4), "steps": steps,
            "flush_bytes_between_steps": 512 << 20, "config": w.describe()}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="blog_t1024")
    ap.add_argument("--extra", default="long_t8192,gqa_t4096_d128,gpu_model_bf16,gpu_model_f32,tiny_cpu_model",
                    help="comma-separated extra workloads timed the same way (reported under 'extra')")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", default="decode_b8_tk8192,decode_mtp4_b16_tk1024",
                    help="comma-separated decode workloads (attn_decode against a KV cache) reported "
                         "under 'decode'; empty to skip")
    ap.add_argument("--noncausal", default="blog_t1024,long_t8192",
                    help="comma-separated workloads run through attn_fwd_noncausal + attn_bwd_noncausal, "
                         "reported under 'noncausal'; empty to skip")
    ap.add_argument("--fwd-rope", default="blog_t1024,long_t8192",
                    help="comma-separated workloads whose forward half is timed both as rope_apply_qk + "
                         "attn_fwd and as attn_fwd_rope, reported under 'fwd_rope'; empty to skip")
    ap.add_argument("--proj", default="blog_t1024",
                    help="comma-separated workloads whose QKV / output projections (forward and backward) "
                         "are timed under 'projections'; empty to skip")
    ap.add_argument("--cold", default="blog_t1024,long_t8192",
                    help="comma-separated workloads whose step is also timed with cold caches (512 MiB "
                         "written before every step), reported under 'cold_cache'; empty to skip")
    ap.add_argument("--only", default="",
                    help="profiling aid: comma-separated subset of extra,decode,projections,noncausal,fwd_rope,cold to run "
                         "WITHOUT the headline step (prints those sections only, not the benchmark line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy (known bytes) five times, for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters of a profiler run")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    import causal_gqa_attention_fwd_amd as ea
    from causal_gqa_attention_fwd_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 2
    ea.lib()  # fail loudly when the HIP library is missing
    if args.calibrate_copy:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n, "launches": 5}))
        return 0

    if args.only:
        # Kernel-trace runs of the secondary paths, so that their kernels (some shared with the
        # headline step) appear in a profile by themselves.
        want = set(x for x in args.only.split(",") if x)
        out = {"only": sorted(want)}
        if "extra" in want:
            out["extra"] = time_extra(args, torch, ea, W)
        if "decode" in want:
            out["decode"] = {name: time_decode(name, max(20, args.steps), max(3, args.warmup // 2), torch, ea, W)
                             for name in [x for x in args.decode.split(",") if x]}
        if "projections" in want:
            out["projections"] = {name: time_projections(name, max(20, args.steps), max(3, args.warmup // 2),
                                                         torch, ea, W)
                                  for name in [x for x in args.proj.split(",") if x]}
        if "noncausal" in want:
            out["noncausal"] = {name: time_noncausal(name, max(5, args.steps // 5), max(2, args.warmup // 5),
                                                     torch, ea, W)
                                for name in [x for x in args.noncausal.split(",") if x]}
        if "cold" in want:
            out["cold_cache"] = {name: time_cold(name, max(10, args.steps // 2), max(2, args.warmup // 5), torch,
                                                 ea, W) for name in [x for x in args.cold.split(",") if x]}
        if "fwd_rope" in want:
            out["fwd_rope"] = {name: time_fwd_rope(name, max(20, args.steps), max(3, args.warmup // 2), torch, ea, W)
                               for name in [x for x in args.fwd_rope.split(",") if x]}
        print(json.dumps(out), flush=True)
        return 0

    w, step, ms, wall, kern_us = time_workload(args.workload, args.steps, args.warmup, torch, ea, W)
    tflops = w.flops_total() / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    dominant = max(kern_us, key=kern_us.get)
    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": dict(w.describe(), causal=True,
                       step="rope_qk,attn_fwd,attn_bwd_rope_preprocess,attn_bwd_rope_main"),
        "frac_of_peak": round(tflops / peak, 4),
        "flops_per_step": w.flops_total(),
        "flops_convention": "exact causal: 14*D*B*Hq*T(T+1)/2",
        "host_wall_s": round(wall, 4),
        "kernel_us": {k: round(v, 2) for k, v in kern_us.items()},
        "roofline": roofline_for(w, kern_us, dominant),
        "roofline_attn_fwd": roofline_for(w, kern_us, "attn_fwd"),
        "roofline_attn_bwd_main": roofline_for(w, kern_us, "attn_bwd_main"),
    }
    out["extra"] = time_extra(args, torch, ea, W)
    out["decode"] = {name: time_decode(name, max(20, args.steps), max(3, args.warmup // 2), torch, ea, W)
                     for name in [x for x in args.decode.split(",") if x]}
    out["projections"] = {name: time_projections(name, max(20, args.steps), max(3, args.warmup // 2), torch, ea, W)
                          for name in [x for x in args.proj.split(",") if x]}
    out["noncausal"] = {name: time_noncausal(name, max(5, args.steps // 5), max(2, args.warmup // 5), torch, ea, W)
                        for name in [x for x in args.noncausal.split(",") if x]}
    out["fwd_rope"] = {name: time_fwd_rope(name, max(20, args.steps), max(3, args.warmup // 2), torch, ea, W)
                       for name in [x for x in args.fwd_rope.split(",") if x]}
    out["cold_cache"] = {name: time_cold(name, max(10, args.steps // 2), max(2, args.warmup // 5), torch, ea, W)
                         for name in [x for x in args.cold.split(",") if x]}
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) on host cores")
        out["cpu_baseline"] = cpu_baseline(w, W)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
