"""fp64 CPU oracle of the delta-rule forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The library path never does, and this package imports nothing
from the library: the two share no code.  The arithmetic lives in
``dr_oracle.c`` (plain C, fp64, one token at a time); this file builds it with
gcc and calls it through ctypes.

Recurrence (FG2-GDN page, section 2, the scaled key/value and state-update
equations; DeltaNet page, step list, step 6 for the output):
    kt = sqrt(beta) * k,  vt = sqrt(beta) * v
    S_t = (I - kt kt^T) Diag(alpha_t) S_{t-1} + kt vt^T,   o_t = S_t^T q_t
With separate erase and write strengths (FG2-GDN page, section "Erweiterung:
FG2-GDN+"; the page prints no equation, the reading taken is) kt = sqrt(beta^k)
* k in both terms and vt = sqrt(beta^v) * v.
Optional input preparation in front of it (DeltaNet page, step list, step 2
and its notes on the key/query map and on choosing beta): qk_l2norm replaces q
and k by unit vectors (a zero vector stays zero); beta_logit takes the
strength arrays as logits, beta = sigmoid(x).
backward() gives the gradients of the forward, with one strength or separate
erase and write strengths, write-side key scales and the input preparation
(reverse-mode differentiation of the token recurrence; the pages print no
backward).
Write-side key scaling (OSDN page, "Method"; the preconditioned delta rule
page, abstract): a diagonal preconditioner s_t on the gradient step, given as
an input; the write key is w = s * kt:
    S_t = (I - w kt^T) Diag(alpha_t) S_{t-1} + w vt^T.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dr_oracle.c")
LIB_PATH = os.path.join(_HERE, "libdr_oracle.so")

GATE_CODES = {"none": 0, "scalar": 1, "channel": 2}
IN_QK_L2NORM, IN_BETA_LOGIT = 1, 2
BETA_CODES = {"scalar": 0, "channel": 1}

_lib = None


def build(src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (fp64, OpenMP over sequences)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = LIB_PATH):
    """Load (building if absent) an oracle library and declare its entry points."""
    if not os.path.exists(path):
        build(out=path)
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.dro_forward.argtypes = [ctypes.c_int] * 5 + [dp, dp, dp, dp, ctypes.c_int, dp,
                                                      ctypes.c_int, dp, dp, dp, ctypes.c_int]
    lib.dro_forward.restype = ctypes.c_int
    lib.dro_forward_kv.argtypes = [ctypes.c_int] * 5 + [dp, dp, dp, dp, ctypes.c_int, dp, dp,
                                                         ctypes.c_int, dp, dp, dp, ctypes.c_int]
    lib.dro_forward_kv.restype = ctypes.c_int
    lib.dro_forward_ex.argtypes = [ctypes.c_int] * 5 + [dp, dp, dp, dp, ctypes.c_int, dp, dp,
                                                        ctypes.c_int, dp, ctypes.c_int, dp, dp, dp,
                                                        ctypes.c_int]
    lib.dro_forward_ex.restype = ctypes.c_int
    lib.dro_backward.argtypes = [ctypes.c_int] * 5 + [dp, dp, dp, dp, ctypes.c_int, dp, ctypes.c_int, dp, dp,
                                                      dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.dro_backward.restype = ctypes.c_int
    lib.dro_backward_kv.argtypes = [ctypes.c_int] * 5 + [dp, dp, dp, dp, ctypes.c_int, dp, dp, ctypes.c_int, dp, dp,
                                                         dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.dro_backward_kv.restype = ctypes.c_int
    lib.dro_backward_ex.argtypes = [ctypes.c_int] * 5 + [dp, dp, dp, dp, ctypes.c_int, dp, dp, ctypes.c_int, dp,
                                                         ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                                         ctypes.c_int]
    lib.dro_backward_ex.restype = ctypes.c_int
    lib.dro_max_threads.restype = ctypes.c_int
    return lib


def _get():
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


def _f64(a: Optional[np.ndarray]):
    if a is None:
        return None, None
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def forward(q, k, v, log_alpha, beta, S0=None, *, gate: str, beta_mode: str,
            nthreads: int = 0, lib=None, beta_v=None, qk_l2norm: bool = False,
            beta_logit: bool = False, key_scale=None):
    """Run the recurrence over [B, H, L, D] inputs; returns (o, S_final) in fp64.

    log_alpha is [B,H,L] (scalar gate), [B,H,L,Dk] (channel gate) or None
    (gate "none"); beta is [B,H,L] or [B,H,L,Dk]; S0 is [B,H,Dk,Dv] or None.
    beta_v (beta's shape) is a separate write strength; None means beta.
    qk_l2norm and beta_logit switch on the input preparation.  key_scale
    ([B,H,L,Dk]) scales the write-side key.
    """
    lib = lib or _get()
    q = np.asarray(q)
    B, H, L, Dk = q.shape
    Dv = np.asarray(v).shape[-1]
    qa, qp = _f64(q)
    ka, kp = _f64(k)
    va, vp = _f64(v)
    la, lp = _f64(log_alpha)
    ba, bp = _f64(beta)
    sa, sp = _f64(S0)
    o = np.empty((B, H, L, Dv), np.float64)
    Sf = np.empty((B, H, Dk, Dv), np.float64)
    op = o.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    fp = Sf.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    flags = (IN_QK_L2NORM if qk_l2norm else 0) | (IN_BETA_LOGIT if beta_logit else 0)
    if flags or key_scale is not None:
        if key_scale is not None and np.shape(key_scale) != (B, H, L, Dk):
            raise ValueError("key_scale must be [B, H, L, Dk]")
        ksa, ksp = _f64(key_scale)
        bva, bvp = _f64(beta if beta_v is None else beta_v)
        if np.shape(bva) != np.shape(ba):
            raise ValueError("beta_v must have beta's shape")
        rc = lib.dro_forward_ex(B, H, L, Dk, Dv, qp, kp, vp, lp, GATE_CODES[gate], bp, bvp,
                                BETA_CODES[beta_mode], ksp, flags, sp, op, fp, int(nthreads))
    elif beta_v is None:
        rc = lib.dro_forward(B, H, L, Dk, Dv, qp, kp, vp, lp, GATE_CODES[gate], bp,
                             BETA_CODES[beta_mode], sp, op, fp, int(nthreads))
    else:
        if np.shape(beta_v) != np.shape(beta):
            raise ValueError("beta_v must have beta's shape")
        bva, bvp = _f64(beta_v)
        rc = lib.dro_forward_kv(B, H, L, Dk, Dv, qp, kp, vp, lp, GATE_CODES[gate], bp, bvp,
                                BETA_CODES[beta_mode], sp, op, fp, int(nthreads))
    if rc != 0:
        raise ValueError(f"dro_forward rejected its arguments (code {rc})")
    return o, Sf


def backward(q, k, v, log_alpha, beta, S0, dO, dS_final=None, *, gate: str, beta_mode: str,
             nthreads: int = 0, lib=None, beta_v=None, key_scale=None, qk_l2norm: bool = False,
             beta_logit: bool = False):
    """Gradients of the forward for the loss whose gradients with respect to o
    and S_final are dO and dS_final, with respect to the inputs as passed (raw
    q, k and strength logits when the input preparation is on).  Returns a
    dict with dq, dk, dv, dlog_alpha (None for gate "none"), dbeta and dS0, in
    fp64 and in the inputs' shapes.  With a separate write strength beta_v
    (beta's shape) dbeta is the erase strength's gradient and dbeta_v the write
    strength's; with key_scale ([B,H,L,Dk]) dkey_scale is its gradient."""
    lib = lib or _get()
    q = np.asarray(q)
    B, H, L, Dk = q.shape
    Dv = np.asarray(v).shape[-1]
    qa, qp = _f64(q)
    ka, kp = _f64(k)
    va, vp = _f64(v)
    la, lp = _f64(log_alpha)
    ba, bp = _f64(beta)
    sa, sp = _f64(S0)
    da, dp_ = _f64(dO)
    fa, fp = _f64(dS_final)
    out = {"dq": np.empty((B, H, L, Dk)), "dk": np.empty((B, H, L, Dk)), "dv": np.empty((B, H, L, Dv)),
           "dlog_alpha": None if log_alpha is None else np.empty(np.shape(log_alpha)),
           "dbeta": np.empty(np.shape(beta)), "dS0": np.empty((B, H, Dk, Dv))}
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    flags = (IN_QK_L2NORM if qk_l2norm else 0) | (IN_BETA_LOGIT if beta_logit else 0)
    if flags or key_scale is not None:
        if key_scale is not None and np.shape(key_scale) != (B, H, L, Dk):
            raise ValueError("key_scale must be [B, H, L, Dk]")
        ksa, ksp = _f64(key_scale)
        bva, bvp = _f64(beta_v)
        if beta_v is not None:
            if np.shape(beta_v) != np.shape(beta):
                raise ValueError("beta_v must have beta's shape")
            out["dbeta_v"] = np.empty(np.shape(beta))
        if key_scale is not None:
            out["dkey_scale"] = np.empty((B, H, L, Dk))
        rc = lib.dro_backward_ex(B, H, L, Dk, Dv, qp, kp, vp, lp, GATE_CODES[gate], bp, bvp, BETA_CODES[beta_mode],
                                 ksp, flags, sp, dp_, fp, ptr(out["dq"]), ptr(out["dk"]), ptr(out["dv"]),
                                 ptr(out["dlog_alpha"]), ptr(out["dbeta"]), ptr(out.get("dbeta_v")),
                                 ptr(out.get("dkey_scale")), ptr(out["dS0"]), int(nthreads))
        if rc != 0:
            raise ValueError(f"dro_backward_ex rejected its arguments (code {rc})")
        return out
    if beta_v is None:
        rc = lib.dro_backward(B, H, L, Dk, Dv, qp, kp, vp, lp, GATE_CODES[gate], bp, BETA_CODES[beta_mode], sp,
                              dp_, fp, ptr(out["dq"]), ptr(out["dk"]), ptr(out["dv"]), ptr(out["dlog_alpha"]),
                              ptr(out["dbeta"]), ptr(out["dS0"]), int(nthreads))
    else:
        if np.shape(beta_v) != np.shape(beta):
            raise ValueError("beta_v must have beta's shape")
        bva, bvp = _f64(beta_v)
        out["dbeta_v"] = np.empty(np.shape(beta))
        rc = lib.dro_backward_kv(B, H, L, Dk, Dv, qp, kp, vp, lp, GATE_CODES[gate], bp, bvp, BETA_CODES[beta_mode],
                                 sp, dp_, fp, ptr(out["dq"]), ptr(out["dk"]), ptr(out["dv"]),
                                 ptr(out["dlog_alpha"]), ptr(out["dbeta"]), ptr(out["dbeta_v"]), ptr(out["dS0"]),
                                 int(nthreads))
    if rc != 0:
        raise ValueError(f"dro_backward rejected its arguments (code {rc})")
    return out


def forward_problem(p, nthreads: int = 0, lib=None):
    """Oracle over a ChunkProblem-like object (fields as the input generator's)."""
    return forward(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, gate=p.gate,
                   beta_mode=p.beta_mode, nthreads=nthreads, lib=lib,
                   beta_v=getattr(p, "beta_v", None), qk_l2norm=getattr(p, "qk_l2norm", False),
                   beta_logit=getattr(p, "beta_logit", False), key_scale=getattr(p, "key_scale", None))


def decode_step(S, q, k, v, log_alpha, beta, *, gate: str, beta_mode: str,
                nthreads: int = 0, lib=None, beta_v=None, qk_l2norm: bool = False,
                beta_logit: bool = False, key_scale=None):
    """One recurrent step for a batch of states: S [N,H,Dk,Dv], q/k/v [N,H,D].

    The decode step is the forward with a single token, started from S.
    Returns (o [N,H,Dv], S_new [N,H,Dk,Dv]) in fp64.
    """
    ex = lambda a: None if a is None else np.asarray(a)[:, :, None]
    o, Sn = forward(ex(q), ex(k), ex(v), ex(log_alpha), ex(beta), S, gate=gate,
                    beta_mode=beta_mode, nthreads=nthreads, lib=lib, beta_v=ex(beta_v),
                    qk_l2norm=qk_l2norm, beta_logit=beta_logit, key_scale=ex(key_scale))
    return o[:, :, 0], Sn


def max_threads(lib=None) -> int:
    return int((lib or _get()).dro_max_threads())
