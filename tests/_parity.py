"""Shared helpers of the GPU parity tests: error metrics, tolerances and the pipeline that
runs the HIP path (through the C ABI binding) on seeded inputs.  The oracle is called by the
tests themselves; nothing here computes attention."""
from __future__ import annotations

import sys

import numpy as np
import torch

import causal_gqa_attention_fwd_amd as ea

# Tolerances.  fp32 I/O: normwise max|x-r|/max|r| <= 1e-4 (O, LSE) and <= 1e-3 (dQ, dK, dV).
# bf16 I/O (fp32 accumulation): max|O - O_ref| <= 2e-2; gradients normwise <= 2e-2; LSE
# normwise <= 1e-4 (fp32 arithmetic on exactly representable inputs).
TOL = {
    "f32": {"o": 1e-4, "lse": 1e-4, "grad": 1e-3},
    "bf16": {"o_abs": 2e-2, "lse": 1e-4, "grad": 2e-2},
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def normwise(x: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    return float(np.max(np.abs(x - ref)) / den) if den > 0 else float(np.max(np.abs(x - ref), initial=0.0))


def maxabs(x: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(x - ref), initial=0.0))


def gpu_forward_pipeline(inp: dict, base: float, device="cuda"):
    """RoPE on q/k then attn_fwd, all on the GPU; returns device tensors."""
    q = inp["q_raw"].to(device)
    k = inp["k_raw"].to(device)
    v = inp["v"].to(device)
    qr = ea.rope_apply(q, base)
    kr = ea.rope_apply(k, base)
    o, lse = ea.attn_fwd(qr, kr, v)
    return q, k, v, qr, kr, o, lse


def check_fwd(dt: str, o_gpu, lse_gpu, o_ref, lse_ref, what: str):
    o, lse = f64(o_gpu), f64(lse_gpu)
    eo, el = normwise(o, o_ref), normwise(lse, lse_ref)
    ea_ = maxabs(o, o_ref)
    say("  %s: O normwise %.3g maxabs %.3g, LSE normwise %.3g" % (what, eo, ea_, el))
    if dt == "f32":
        assert eo <= TOL["f32"]["o"], (what, "O", eo)
        assert el <= TOL["f32"]["lse"], (what, "LSE", el)
    else:
        assert ea_ <= TOL["bf16"]["o_abs"], (what, "O", ea_)
        assert el <= TOL["bf16"]["lse"], (what, "LSE", el)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def check_grads(dt: str, got: dict, ref: dict, what: str):
    tol = TOL[dt]["grad"]
    errs = {n: normwise(f64(got[n]) if torch.is_tensor(got[n]) else got[n], ref[n]) for n in ref}
    say("  %s: grads normwise %s" % (what, " ".join("%s %.3g" % kv for kv in errs.items())))
    for n, e in errs.items():
        assert e <= tol, (what, n, e)
