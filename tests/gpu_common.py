"""Helpers shared by the GPU tests: move generator output to the device, run
the HIP path through the C-ABI binding, run the oracle, compare."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from delta_rule_linear_amd import inputs

# Parity bounds on max|x - y| / max|y| per output tensor: 1e-4 for fp32
# inputs, 3e-3 for bf16 inputs with an fp32 state.
TOL = {"f32": 1e-4, "bf16": 3e-3}


def announce(*what):
    print("[gpu case]", *what, file=sys.stderr, flush=True)


def rel_err(x, y) -> float:
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    scale = np.max(np.abs(y)) if y.size else 0.0
    if scale == 0.0:
        return float(np.max(np.abs(x))) if x.size else 0.0
    return float(np.max(np.abs(x - y)) / scale)


def per_head_errors(x, y):
    """max|x - y| / max|y| of every (b, h) slice of [B, H, ...] arrays."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    B, H = y.shape[:2]
    xe = x.reshape(B, H, -1)
    ye = y.reshape(B, H, -1)
    if ye.shape[2] == 0:
        return np.zeros((B, H))
    num = np.abs(xe - ye).max(axis=2)
    den = np.abs(ye).max(axis=2)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def to_dev(a, dtype: str, device="cuda"):
    import torch
    if a is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(inputs.bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def problem_to_dev(p):
    """The problem's tensors on the device, keyed as dr_chunk_fwd's arguments
    (plus beta_v and key_scale when the problem has them)."""
    t = dict(q=to_dev(p.q, p.in_dtype), k=to_dev(p.k, p.in_dtype), v=to_dev(p.v, p.in_dtype),
             log_alpha=to_dev(p.log_alpha, "f32"), beta=to_dev(p.beta, "f32"), S0=to_dev(p.S0, "f32"))
    if getattr(p, "beta_v", None) is not None:
        t["beta_v"] = to_dev(p.beta_v, "f32")
    if getattr(p, "key_scale", None) is not None:
        t["key_scale"] = to_dev(p.key_scale, "f32")
    return t


def run_hip(p, out_dtype=None, **kw):
    """Chunked forward of a ChunkProblem on the GPU (dr_chunk_fwd_kv when it
    has a separate write strength); returns device tensors."""
    import delta_rule_linear_amd as drl
    t = problem_to_dev(p)
    kw.setdefault("qk_l2norm", getattr(p, "qk_l2norm", False))
    kw.setdefault("beta_logit", getattr(p, "beta_logit", False))
    if "key_scale" in t:
        return drl.dr_chunk_fwd_precond(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["key_scale"],
                                        t["S0"], gate=p.gate, beta_mode=p.beta_mode, out_dtype=out_dtype,
                                        **kw)
    if "beta_v" in t:
        return drl.dr_chunk_fwd_kv(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["beta_v"],
                                   t["S0"], gate=p.gate, beta_mode=p.beta_mode, out_dtype=out_dtype, **kw)
    return drl.dr_chunk_fwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["S0"],
                            gate=p.gate, beta_mode=p.beta_mode, out_dtype=out_dtype, **kw)


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def run_oracle(p, nthreads=0):
    return oracle.forward_problem(p, nthreads=nthreads)
