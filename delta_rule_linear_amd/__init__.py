"""delta_rule_linear_amd -- MI355X (gfx950) delta-rule linear-attention forward.

Thin Python binding over the C ABI in include/deltarule.h, with the same names.
It only marshals arguments (shape checks, output and workspace allocation with
PyTorch, the current HIP stream); every step of the computation runs in the
HIP kernels of libdeltarule.so.  If the library is missing the binding raises:
there is no fallback path.

    o, S = dr_chunk_fwd(q, k, v, log_alpha, beta, S0, gate="scalar", beta_mode="scalar")
    o = dr_decode_step(S, q, k, v, log_alpha, beta, gate="scalar", beta_mode="scalar")

With separate channel-wise erase and write strengths (FG2-GDN+):

    o, S = dr_chunk_fwd_kv(q, k, v, log_alpha, beta_k, beta_v, S0, gate="channel")
    o = dr_decode_step_kv(S, q, k, v, log_alpha, beta_k, beta_v, gate="channel")

With a diagonal preconditioner on the gradient step (write-side key scales):

    o, S = dr_chunk_fwd_precond(q, k, v, log_alpha, beta, key_scale, S0, gate="scalar",
                                beta_mode="scalar")

Gradients of the chunked forward (any gate and beta mode):

    g = dr_chunk_bwd(q, k, v, log_alpha, beta, S0, dO, dS_final, gate="scalar")
    g["dq"], g["dk"], g["dv"], g["dlog_alpha"], g["dbeta"], g["dS0"]
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdeltarule.so")

DR_ABI_VERSION = 10
DR_OK, DR_ERR_NULL, DR_ERR_SHAPE, DR_ERR_UNSUPPORTED, DR_ERR_ALIGN, DR_ERR_WORKSPACE, DR_ERR_HIP = range(7)
DR_F32, DR_BF16 = 0, 1
GATES = {"none": 0, "scalar": 1, "channel": 2}
BETAS = {"scalar": 0, "channel": 1}
DR_IN_QK_L2NORM, DR_IN_BETA_LOGIT = 1, 2
EXPORTS = ("dr_chunk_fwd_workspace_bytes", "dr_chunk_fwd", "dr_chunk_fwd_kv", "dr_decode_step",
           "dr_decode_step_kv", "dr_chunk_fwd_precond_workspace_bytes", "dr_chunk_fwd_precond",
           "dr_decode_step_precond", "dr_status_str", "dr_last_error", "dr_abi_version",
           "dr_profile_begin", "dr_profile_end", "dr_chunk_bwd_workspace_bytes", "dr_chunk_bwd",
           "dr_chunk_bwd_kv", "dr_chunk_fwd_noalloc", "dr_chunk_fwd_kv_workspace_bytes",
           "dr_chunk_bwd_kv_workspace_bytes", "dr_chunk_bwd_precond_workspace_bytes", "dr_chunk_bwd_precond",
           "dr_chunk_bwd_workspace_bytes_min")
DR_NOALLOC_SCRATCH_BYTES = 256 << 20


class DeltaRuleError(RuntimeError):
    """A dr_* call returned an error status."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{dr_status_str(status)} ({detail})")


class ChunkDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("L", ctypes.c_int), ("Dk", ctypes.c_int),
                ("Dv", ctypes.c_int), ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("gate", ctypes.c_int), ("beta", ctypes.c_int), ("input_flags", ctypes.c_uint)]


class ProfileReport(ctypes.Structure):
    _fields_ = [("chunk_calls", ctypes.c_int), ("decode_calls", ctypes.c_int), ("prep_ms", ctypes.c_double),
                ("scan_ms", ctypes.c_double), ("decode_ms", ctypes.c_double), ("bwd_calls", ctypes.c_int),
                ("bwd_prep_ms", ctypes.c_double), ("bwd_fscan_ms", ctypes.c_double),
                ("bwd_rscan_ms", ctypes.c_double), ("bwd_post_ms", ctypes.c_double)]


class DecodeDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int), ("H", ctypes.c_int), ("Dk", ctypes.c_int), ("Dv", ctypes.c_int),
                ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int), ("gate", ctypes.c_int),
                ("beta", ctypes.c_int), ("input_flags", ctypes.c_uint)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m delta_rule_linear_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.dr_chunk_fwd_workspace_bytes.argtypes = [ctypes.POINTER(ChunkDesc)]
        L.dr_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
        L.dr_chunk_fwd.argtypes = [ctypes.POINTER(ChunkDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   ctypes.c_size_t, vp]
        L.dr_chunk_fwd.restype = ctypes.c_int
        L.dr_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(ChunkDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.dr_chunk_fwd_noalloc.restype = ctypes.c_int
        L.dr_chunk_fwd_kv.argtypes = [ctypes.POINTER(ChunkDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, ctypes.c_size_t, vp]
        L.dr_chunk_fwd_kv.restype = ctypes.c_int
        L.dr_decode_step.argtypes = [ctypes.POINTER(DecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp]
        L.dr_decode_step.restype = ctypes.c_int
        L.dr_decode_step_kv.argtypes = [ctypes.POINTER(DecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.dr_decode_step_kv.restype = ctypes.c_int
        L.dr_chunk_fwd_precond_workspace_bytes.argtypes = [ctypes.POINTER(ChunkDesc)]
        L.dr_chunk_fwd_precond_workspace_bytes.restype = ctypes.c_size_t
        L.dr_chunk_fwd_precond.argtypes = [ctypes.POINTER(ChunkDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           vp, ctypes.c_size_t, vp]
        L.dr_chunk_fwd_precond.restype = ctypes.c_int
        L.dr_decode_step_precond.argtypes = [ctypes.POINTER(DecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp,
                                             vp]
        L.dr_decode_step_precond.restype = ctypes.c_int
        L.dr_chunk_bwd_workspace_bytes.argtypes = [ctypes.POINTER(ChunkDesc)]
        L.dr_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.dr_chunk_bwd_workspace_bytes_min.argtypes = [ctypes.POINTER(ChunkDesc)]
        L.dr_chunk_bwd_workspace_bytes_min.restype = ctypes.c_size_t
        L.dr_chunk_fwd_kv_workspace_bytes.argtypes = [ctypes.POINTER(ChunkDesc)]
        L.dr_chunk_fwd_kv_workspace_bytes.restype = ctypes.c_size_t
        L.dr_chunk_bwd_kv_workspace_bytes.argtypes = [ctypes.POINTER(ChunkDesc)]
        L.dr_chunk_bwd_kv_workspace_bytes.restype = ctypes.c_size_t
        L.dr_chunk_bwd.argtypes = [ctypes.POINTER(ChunkDesc)] + [vp] * 15 + [ctypes.c_size_t, vp]
        L.dr_chunk_bwd.restype = ctypes.c_int
        L.dr_chunk_bwd_kv.argtypes = [ctypes.POINTER(ChunkDesc)] + [vp] * 17 + [ctypes.c_size_t, vp]
        L.dr_chunk_bwd_kv.restype = ctypes.c_int
        L.dr_chunk_bwd_precond_workspace_bytes.argtypes = [ctypes.POINTER(ChunkDesc)]
        L.dr_chunk_bwd_precond_workspace_bytes.restype = ctypes.c_size_t
        L.dr_chunk_bwd_precond.argtypes = [ctypes.POINTER(ChunkDesc)] + [vp] * 17 + [ctypes.c_size_t, vp]
        L.dr_chunk_bwd_precond.restype = ctypes.c_int
        L.dr_status_str.argtypes = [ctypes.c_int]
        L.dr_status_str.restype = ctypes.c_char_p
        L.dr_last_error.argtypes = []
        L.dr_last_error.restype = ctypes.c_char_p
        L.dr_abi_version.argtypes = []
        L.dr_abi_version.restype = ctypes.c_int
        L.dr_profile_begin.argtypes = []
        L.dr_profile_begin.restype = ctypes.c_int
        L.dr_profile_end.argtypes = [ctypes.POINTER(ProfileReport)]
        L.dr_profile_end.restype = ctypes.c_int
        if L.dr_abi_version() != DR_ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI {L.dr_abi_version()}, binding expects {DR_ABI_VERSION}")
        _lib = L
    return _lib


def dr_abi_version() -> int:
    return int(lib().dr_abi_version())


def dr_status_str(status: int) -> str:
    return lib().dr_status_str(int(status)).decode()


def dr_last_error() -> str:
    return lib().dr_last_error().decode()


def _check(status: int):
    if status != DR_OK:
        raise DeltaRuleError(status, dr_last_error())


def dr_profile_begin() -> None:
    """Start recording per-kernel HIP events in later calls."""
    _check(lib().dr_profile_begin())


def dr_profile_end() -> dict:
    """Stop recording; wait for the events and return the summed kernel times (ms)."""
    rep = ProfileReport()
    _check(lib().dr_profile_end(ctypes.byref(rep)))
    return {f: getattr(rep, f) for f, _ in ProfileReport._fields_}


# ---------------------------------------------------------------------------
# torch-facing wrappers (argument marshalling only)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.bfloat16:
        return DR_BF16
    if dt == torch.float32:
        return DR_F32
    raise TypeError(f"unsupported dtype {dt}: use torch.bfloat16 or torch.float32")


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t, name, dtype=None, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def input_flags(qk_l2norm: bool = False, beta_logit: bool = False) -> int:
    return (DR_IN_QK_L2NORM if qk_l2norm else 0) | (DR_IN_BETA_LOGIT if beta_logit else 0)


def chunk_desc(B, H, L, Dk, Dv, in_dtype, out_dtype, gate: str, beta_mode: str,
               flags: int = 0) -> ChunkDesc:
    return ChunkDesc(B, H, L, Dk, Dv, in_dtype, out_dtype, GATES[gate], BETAS[beta_mode], flags)


def dr_chunk_fwd_workspace_bytes(desc: ChunkDesc) -> int:
    return int(lib().dr_chunk_fwd_workspace_bytes(ctypes.byref(desc)))


def dr_chunk_fwd_precond_workspace_bytes(desc: ChunkDesc) -> int:
    return int(lib().dr_chunk_fwd_precond_workspace_bytes(ctypes.byref(desc)))


def dr_chunk_fwd(q, k, v, log_alpha, beta, S0=None, *, gate: str, beta_mode: str,
                 out_dtype=None, o=None, S_final=None, want_state: bool = True,
                 workspace=None, stream=None, qk_l2norm: bool = False, beta_logit: bool = False):
    """Chunked forward over [B, H, L, D] device tensors; returns (o, S_final).

    q, k: [B,H,L,Dk]; v: [B,H,L,Dv] (bf16 or fp32, same dtype); log_alpha:
    [B,H,L] / [B,H,L,Dk] fp32 or None for gate "none"; beta: [B,H,L] /
    [B,H,L,Dk] fp32; S0: [B,H,Dk,Dv] fp32 or None.  S_final may be passed in
    (it may be S0 itself for an in-place carry); with want_state=False no
    final state is written and None is returned for it.  qk_l2norm and
    beta_logit switch on the input preparation (DR_IN_QK_L2NORM,
    DR_IN_BETA_LOGIT).
    """
    return _chunk(q, k, v, log_alpha, beta, None, S0, gate, beta_mode, out_dtype, o, S_final,
                  want_state, workspace, stream, input_flags(qk_l2norm, beta_logit))


def dr_chunk_fwd_precond(q, k, v, log_alpha, beta, key_scale, S0=None, *, gate: str, beta_mode: str,
                         out_dtype=None, o=None, S_final=None, want_state: bool = True, workspace=None,
                         stream=None, qk_l2norm: bool = False, beta_logit: bool = False):
    """dr_chunk_fwd with write-side key scales key_scale [B,H,L,Dk] fp32 (the
    diagonal preconditioner of the gradient step)."""
    if key_scale is None:
        raise ValueError("key_scale is required")
    return _chunk(q, k, v, log_alpha, beta, None, S0, gate, beta_mode, out_dtype, o, S_final,
                  want_state, workspace, stream, input_flags(qk_l2norm, beta_logit), key_scale)


def dr_chunk_fwd_kv(q, k, v, log_alpha, beta_k, beta_v, S0=None, *, gate: str, beta_mode: str = "channel",
                    out_dtype=None, o=None, S_final=None, want_state: bool = True, workspace=None, stream=None,
                    qk_l2norm: bool = False, beta_logit: bool = False):
    """dr_chunk_fwd with separate erase (beta_k) and write (beta_v)
    strengths, both [B,H,L,Dk] (beta_mode "channel") or both [B,H,L]
    (beta_mode "scalar") fp32; Dv == Dk."""
    if beta_v is None:
        raise ValueError("beta_v is required")
    return _chunk(q, k, v, log_alpha, beta_k, beta_v, S0, gate, beta_mode, out_dtype, o, S_final,
                  want_state, workspace, stream, input_flags(qk_l2norm, beta_logit))


def dr_chunk_fwd_kv_workspace_bytes(desc: ChunkDesc) -> int:
    return int(lib().dr_chunk_fwd_kv_workspace_bytes(ctypes.byref(desc)))


def dr_chunk_bwd_workspace_bytes_min(desc: ChunkDesc) -> int:
    """The least workspace dr_chunk_bwd accepts (segments of chunks below
    dr_chunk_bwd_workspace_bytes; equal to it where segments do not apply)."""
    return int(lib().dr_chunk_bwd_workspace_bytes_min(ctypes.byref(desc)))


def dr_chunk_bwd_kv_workspace_bytes(desc: ChunkDesc) -> int:
    return int(lib().dr_chunk_bwd_kv_workspace_bytes(ctypes.byref(desc)))


def dr_chunk_fwd_noalloc(q, k, v, log_alpha, beta, S0=None, *, gate: str, beta_mode: str, o, S_final=None,
                         stream=None, qk_l2norm: bool = False, beta_logit: bool = False):
    """dr_chunk_fwd without a workspace: the library's per-GPU scratch array
    (DR_NOALLOC_SCRATCH_BYTES) takes its place, for callers that cannot
    allocate.  o (and S_final, or None to skip it) are the caller's tensors;
    nothing is allocated here or in the library.  Calls that overlap in time
    on one GPU race on the scratch array.  Returns (o, S_final)."""
    return _chunk(q, k, v, log_alpha, beta, None, S0, gate, beta_mode, o.dtype, o, S_final,
                  False, None, stream, input_flags(qk_l2norm, beta_logit), noalloc=True)


def _chunk(q, k, v, log_alpha, beta, beta_v, S0, gate, beta_mode, out_dtype, o, S_final, want_state,
           workspace, stream, flags, key_scale=None, noalloc=False):
    torch = _torch()
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    _need(q, "q")
    _need(k, "k", q.dtype, (B, H, L, Dk))
    _need(v, "v", q.dtype, (B, H, L, Dv))
    gshape = {"none": None, "scalar": (B, H, L), "channel": (B, H, L, Dk)}[gate]
    if gshape is None:
        if log_alpha is not None:
            raise ValueError("gate 'none' takes no log_alpha")
    else:
        _need(log_alpha, "log_alpha", torch.float32, gshape)
    bshape = (B, H, L) if beta_mode == "scalar" else (B, H, L, Dk)
    _need(beta, "beta", torch.float32, bshape)
    if beta_v is not None:
        _need(beta_v, "beta_v", torch.float32, bshape)
    if key_scale is not None:
        _need(key_scale, "key_scale", torch.float32, (B, H, L, Dk))
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, Dk, Dv))
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, H, L, Dv), dtype=out_dtype, device=q.device)
    else:
        _need(o, "o", out_dtype, (B, H, L, Dv))
    if want_state and S_final is None:
        S_final = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    elif S_final is not None:
        _need(S_final, "S_final", torch.float32, (B, H, Dk, Dv))
    desc = chunk_desc(B, H, L, Dk, Dv, _dtype_code(q.dtype), _dtype_code(out_dtype), gate, beta_mode,
                      flags)
    if noalloc:
        _check(lib().dr_chunk_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                          _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_final), _stream(stream)))
        return o, S_final
    nbytes = (dr_chunk_fwd_precond_workspace_bytes(desc) if key_scale is not None
              else dr_chunk_fwd_kv_workspace_bytes(desc) if beta_v is not None
              else dr_chunk_fwd_workspace_bytes(desc))
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if key_scale is not None:
        _check(lib().dr_chunk_fwd_precond(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                          _ptr(beta), _ptr(key_scale), _ptr(S0), _ptr(o), _ptr(S_final),
                                          _ptr(workspace), wbytes, _stream(stream)))
    elif beta_v is None:
        _check(lib().dr_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                  _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_final), _ptr(workspace),
                                  wbytes, _stream(stream)))
    else:
        _check(lib().dr_chunk_fwd_kv(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                     _ptr(beta), _ptr(beta_v), _ptr(S0), _ptr(o), _ptr(S_final),
                                     _ptr(workspace), wbytes, _stream(stream)))
    return o, S_final


def dr_chunk_bwd_workspace_bytes(desc: ChunkDesc) -> int:
    return int(lib().dr_chunk_bwd_workspace_bytes(ctypes.byref(desc)))


def dr_chunk_bwd_kv(q, k, v, log_alpha, beta_k, beta_v, S0, dO, dS_final=None, *, gate: str,
                    beta_mode: str = "channel", want_dS0: bool = True, workspace=None, stream=None,
                    qk_l2norm: bool = False, beta_logit: bool = False):
    """Gradients of dr_chunk_fwd_kv (separate erase and write strengths, both
    [B,H,L,Dk] or both [B,H,L] fp32): as dr_chunk_bwd, with dbeta the erase
    strength's gradient and dbeta_v the write strength's."""
    if beta_v is None:
        raise ValueError("beta_v is required")
    return dr_chunk_bwd(q, k, v, log_alpha, beta_k, S0, dO, dS_final, gate=gate, beta_mode=beta_mode,
                        want_dS0=want_dS0, workspace=workspace, stream=stream, qk_l2norm=qk_l2norm,
                        beta_logit=beta_logit, _beta_v=beta_v)


def dr_chunk_bwd_precond_workspace_bytes(desc: ChunkDesc) -> int:
    return int(lib().dr_chunk_bwd_precond_workspace_bytes(ctypes.byref(desc)))


def dr_chunk_bwd_precond(q, k, v, log_alpha, beta, key_scale, S0, dO, dS_final=None, *, gate: str,
                         beta_mode: str = "scalar", want_dS0: bool = True, workspace=None, stream=None,
                         qk_l2norm: bool = False, beta_logit: bool = False):
    """Gradients of dr_chunk_fwd_precond (write-side key scales key_scale,
    [B,H,L,Dk] fp32): as dr_chunk_bwd, with dkey_scale the scales' gradient."""
    if key_scale is None:
        raise ValueError("key_scale is required")
    return dr_chunk_bwd(q, k, v, log_alpha, beta, S0, dO, dS_final, gate=gate, beta_mode=beta_mode,
                        want_dS0=want_dS0, workspace=workspace, stream=stream, qk_l2norm=qk_l2norm,
                        beta_logit=beta_logit, _key_scale=key_scale)


def dr_chunk_bwd(q, k, v, log_alpha, beta, S0, dO, dS_final=None, *, gate: str, beta_mode: str = "scalar",
                 want_dS0: bool = True, workspace=None, stream=None, qk_l2norm: bool = False,
                 beta_logit: bool = False, _beta_v=None, _key_scale=None):
    """Gradients of dr_chunk_fwd (any gate and beta mode) for the
    loss whose gradients with respect to o and S_final are dO [B,H,L,Dv] and
    dS_final [B,H,Dk,Dv] (fp32; dS_final None means zero).  q, k, v and the
    other inputs are as for dr_chunk_fwd, with the same input preparation
    (qk_l2norm, beta_logit): the gradients are those of the raw inputs.
    Returns a dict of fp32 device tensors dq, dk, dv, dlog_alpha (None for
    gate "none"), dbeta and dS0 (None with want_dS0=False).  workspace: a
    device uint8 tensor (None: one of dr_chunk_bwd_workspace_bytes bytes is
    allocated); one smaller than that, down to dr_chunk_bwd_workspace_bytes_min,
    makes the library run the backward in segments of chunks."""
    torch = _torch()
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    _need(q, "q")
    _need(k, "k", q.dtype, (B, H, L, Dk))
    _need(v, "v", q.dtype, (B, H, L, Dv))
    gshape = {"none": None, "scalar": (B, H, L), "channel": (B, H, L, Dk)}[gate]
    if gshape is None:
        if log_alpha is not None:
            raise ValueError("gate 'none' takes no log_alpha")
    else:
        _need(log_alpha, "log_alpha", torch.float32, gshape)
    bshape = (B, H, L) if beta_mode == "scalar" else (B, H, L, Dk)
    _need(beta, "beta", torch.float32, bshape)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (B, H, Dk, Dv))
    if _beta_v is not None:
        _need(_beta_v, "beta_v", torch.float32, bshape)
    if _key_scale is not None:
        _need(_key_scale, "key_scale", torch.float32, (B, H, L, Dk))
    _need(dO, "dO", torch.float32, (B, H, L, Dv))
    if dS_final is not None:
        _need(dS_final, "dS_final", torch.float32, (B, H, Dk, Dv))
    f32 = dict(dtype=torch.float32, device=q.device)
    out = {"dq": torch.empty((B, H, L, Dk), **f32), "dk": torch.empty((B, H, L, Dk), **f32),
           "dv": torch.empty((B, H, L, Dv), **f32),
           "dlog_alpha": torch.empty(gshape, **f32) if gshape is not None else None,
           "dbeta": torch.empty(bshape, **f32),
           "dS0": torch.empty((B, H, Dk, Dv), **f32) if want_dS0 else None}
    desc = chunk_desc(B, H, L, Dk, Dv, _dtype_code(q.dtype), DR_F32, gate, beta_mode,
                      input_flags(qk_l2norm, beta_logit))
    if _key_scale is not None:
        nbytes = dr_chunk_bwd_precond_workspace_bytes(desc)
    elif _beta_v is not None:
        nbytes = dr_chunk_bwd_kv_workspace_bytes(desc)
    else:
        nbytes = dr_chunk_bwd_workspace_bytes(desc)
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if _key_scale is not None:
        out["dkey_scale"] = torch.empty((B, H, L, Dk), **f32)
        _check(lib().dr_chunk_bwd_precond(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                          _ptr(beta), _ptr(_key_scale), _ptr(S0), _ptr(dO), _ptr(dS_final),
                                          _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                          _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]), _ptr(out["dkey_scale"]),
                                          _ptr(out["dS0"]), _ptr(workspace), wbytes, _stream(stream)))
    elif _beta_v is None:
        _check(lib().dr_chunk_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                  _ptr(S0), _ptr(dO), _ptr(dS_final), _ptr(out["dq"]), _ptr(out["dk"]),
                                  _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]), _ptr(out["dS0"]),
                                  _ptr(workspace), wbytes, _stream(stream)))
    else:
        out["dbeta_v"] = torch.empty(bshape, **f32)
        _check(lib().dr_chunk_bwd_kv(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                     _ptr(_beta_v), _ptr(S0), _ptr(dO), _ptr(dS_final), _ptr(out["dq"]),
                                     _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]),
                                     _ptr(out["dbeta_v"]), _ptr(out["dS0"]), _ptr(workspace), wbytes,
                                     _stream(stream)))
    return out


def dr_decode_step(S, q, k, v, log_alpha, beta, *, gate: str, beta_mode: str, out_dtype=None,
                   o=None, stream=None, qk_l2norm: bool = False, beta_logit: bool = False):
    """One decode step for N x H states (updated in place); returns o [N,H,Dv].

    S: [N,H,Dk,Dv] fp32; q, k: [N,H,Dk]; v: [N,H,Dv]; log_alpha: [N,H] /
    [N,H,Dk] or None; beta: [N,H] / [N,H,Dk].
    """
    return _decode(S, q, k, v, log_alpha, beta, None, gate, beta_mode, out_dtype, o, stream,
                   input_flags(qk_l2norm, beta_logit))


def dr_decode_step_precond(S, q, k, v, log_alpha, beta, key_scale, *, gate: str, beta_mode: str,
                           out_dtype=None, o=None, stream=None, qk_l2norm: bool = False,
                           beta_logit: bool = False):
    """dr_decode_step with write-side key scales key_scale [N,H,Dk] fp32."""
    if key_scale is None:
        raise ValueError("key_scale is required")
    return _decode(S, q, k, v, log_alpha, beta, None, gate, beta_mode, out_dtype, o, stream,
                   input_flags(qk_l2norm, beta_logit), key_scale)


def dr_decode_step_kv(S, q, k, v, log_alpha, beta_k, beta_v, *, gate: str, beta_mode: str = "channel",
                      out_dtype=None, o=None, stream=None, qk_l2norm: bool = False, beta_logit: bool = False):
    """dr_decode_step with separate erase (beta_k) and write (beta_v)
    strengths, both [N,H,Dk] (beta_mode "channel", Dv == Dk) or both [N,H]
    (beta_mode "scalar") fp32."""
    if beta_v is None:
        raise ValueError("beta_v is required")
    return _decode(S, q, k, v, log_alpha, beta_k, beta_v, gate, beta_mode, out_dtype, o, stream,
                   input_flags(qk_l2norm, beta_logit))


def _decode(S, q, k, v, log_alpha, beta, beta_v, gate, beta_mode, out_dtype, o, stream, flags,
            key_scale=None):
    torch = _torch()
    N, H, Dk, Dv = S.shape
    _need(S, "S", torch.float32)
    _need(q, "q", None, (N, H, Dk))
    _need(k, "k", q.dtype, (N, H, Dk))
    _need(v, "v", q.dtype, (N, H, Dv))
    gshape = {"none": None, "scalar": (N, H), "channel": (N, H, Dk)}[gate]
    if gshape is None:
        if log_alpha is not None:
            raise ValueError("gate 'none' takes no log_alpha")
    else:
        _need(log_alpha, "log_alpha", torch.float32, gshape)
    bshape = (N, H) if beta_mode == "scalar" else (N, H, Dk)
    _need(beta, "beta", torch.float32, bshape)
    if beta_v is not None:
        _need(beta_v, "beta_v", torch.float32, bshape)
    if key_scale is not None:
        _need(key_scale, "key_scale", torch.float32, (N, H, Dk))
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((N, H, Dv), dtype=out_dtype, device=S.device)
    else:
        _need(o, "o", out_dtype, (N, H, Dv))
    desc = DecodeDesc(N, H, Dk, Dv, _dtype_code(q.dtype), _dtype_code(out_dtype), GATES[gate],
                      BETAS[beta_mode], flags)
    if key_scale is not None:
        _check(lib().dr_decode_step_precond(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                            _ptr(beta), _ptr(key_scale), _ptr(S), _ptr(o), _stream(stream)))
    elif beta_v is None:
        _check(lib().dr_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                    _ptr(beta), _ptr(S), _ptr(o), _stream(stream)))
    else:
        _check(lib().dr_decode_step_kv(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                       _ptr(beta), _ptr(beta_v), _ptr(S), _ptr(o), _stream(stream)))
    return o
