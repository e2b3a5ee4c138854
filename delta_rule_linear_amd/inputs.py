"""Seeded synthetic inputs for the delta-rule forward.

This module only draws and rounds numbers: it holds none of the recurrence's
arithmetic, so both the HIP path and the fp64 oracle can be fed from it.

Workloads (sizes as named by each function) and the draw recipe:

* One ``numpy.random.default_rng(seed)`` stream per problem, seed 0 by default.
* Tensors are drawn whole, in C order, in float64, in this order, skipping the
  ones the workload does not have: q ~ N(0,1), k ~ N(0,1), v ~ N(0,1),
  log alpha ~ U(lo, hi), beta logits ~ N(0,1), S0 ~ N(0, 0.01) (variance 0.01,
  i.e. sigma 0.1).
* q and k are L2-normalised per token in float64 (the DeltaNet page, the step
  list: the key map phi is "usually" followed by L2 normalisation), beta is the
  logistic sigmoid of its logit (the DeltaNet page lists a sigmoid projection
  among the ways to pick beta), then q, k, v are rounded to the input dtype
  (bf16 round-to-nearest-even, or fp32).  Gates, beta and S0 are fp32.
* Decode: the per-sequence states are drawn first, then for each step in order
  q, k, v, log alpha, beta logits of shape [N, H, .].

All arrays are returned as float32 numpy arrays whose values are exactly
representable in the named input dtype; ``bf16_bits`` gives the raw bf16 bit
patterns for handing to a device.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

GATES = ("none", "scalar", "channel")
BETAS = ("scalar", "channel")
DTYPES = ("bf16", "f32")


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even); returns float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-exact; round them first")
    return (u >> 16).astype(np.uint16)


def _l2norm(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x) if dtype == "bf16" else x.astype(np.float32)


@dataclass
class ChunkProblem:
    """One batch for the chunked forward: [B, H, L, D] tensors."""

    name: str
    B: int
    H: int
    L: int
    Dk: int
    Dv: int
    in_dtype: str
    gate: str
    beta_mode: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    log_alpha: Optional[np.ndarray]
    beta: np.ndarray
    S0: Optional[np.ndarray]
    meta: dict = field(default_factory=dict)
    beta_v: Optional[np.ndarray] = None   # separate write strength (FG2-GDN+), beta's shape
    qk_l2norm: bool = False               # q, k raw: the forward normalises them
    beta_logit: bool = False              # beta (and beta_v) hold logits
    key_scale: Optional[np.ndarray] = None   # write-side key scales [B, H, L, Dk]

    @property
    def token_heads(self) -> int:
        return self.B * self.H * self.L

    def head(self, b: int, h: int) -> "ChunkProblem":
        """The single (b, h) sequence as a B=H=1 problem (views, no copy)."""
        sl = lambda a: None if a is None else a[b : b + 1, h : h + 1]
        return ChunkProblem(
            f"{self.name}[b={b},h={h}]", 1, 1, self.L, self.Dk, self.Dv, self.in_dtype,
            self.gate, self.beta_mode, sl(self.q), sl(self.k), sl(self.v),
            sl(self.log_alpha), sl(self.beta), sl(self.S0), dict(self.meta), sl(self.beta_v),
            self.qk_l2norm, self.beta_logit, sl(self.key_scale))


def make_chunk_problem(B, H, L, Dk, Dv, *, in_dtype="bf16", gate="scalar", beta_mode="scalar",
                       log_alpha_range=(-0.1, -0.001), s0_var: Optional[float] = None,
                       seed: int = 0, name: str = "custom", beta_v: bool = False,
                       raw_inputs: bool = False, key_scale: bool = False) -> ChunkProblem:
    """Draw one chunked-forward batch following the module recipe.

    beta_v=True adds a separate write strength beta^v (FG2-GDN+), drawn like
    beta and after every other tensor, so the rest of the batch is unchanged.
    raw_inputs=True keeps the same draws before their last step: q and k
    are not normalised and the strengths are the logits, for a forward with
    the input preparation switched on.  key_scale=True adds write-side key
    scales (a diagonal preconditioner), U(0.5, 1.5) per token and channel,
    drawn after everything else.
    """
    if gate not in GATES or beta_mode not in BETAS or in_dtype not in DTYPES:
        raise ValueError("unknown mode")
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, L, Dk))
    k = rng.standard_normal((B, H, L, Dk))
    v = rng.standard_normal((B, H, L, Dv))
    la = None
    if gate == "scalar":
        la = rng.uniform(log_alpha_range[0], log_alpha_range[1], (B, H, L))
    elif gate == "channel":
        la = rng.uniform(log_alpha_range[0], log_alpha_range[1], (B, H, L, Dk))
    bshape = (B, H, L) if beta_mode == "scalar" else (B, H, L, Dk)
    beta_logits = rng.standard_normal(bshape)
    beta = beta_logits if raw_inputs else _sigmoid(beta_logits)
    S0 = None
    if s0_var is not None:
        S0 = (rng.standard_normal((B, H, Dk, Dv)) * np.sqrt(s0_var)).astype(np.float32)
    bv = rng.standard_normal(bshape) if beta_v else None
    if not raw_inputs:
        q, k = _l2norm(q), _l2norm(k)
        bv = None if bv is None else _sigmoid(bv)
    q = _to_dtype(q, in_dtype)
    k = _to_dtype(k, in_dtype)
    v = _to_dtype(v, in_dtype)
    return ChunkProblem(name, B, H, L, Dk, Dv, in_dtype, gate, beta_mode, q, k, v,
                        None if la is None else la.astype(np.float32),
                        beta.astype(np.float32), S0,
                        {"seed": seed, "log_alpha_range": log_alpha_range, "s0_var": s0_var},
                        None if bv is None else bv.astype(np.float32), raw_inputs, raw_inputs,
                        rng.uniform(0.5, 1.5, (B, H, L, Dk)).astype(np.float32) if key_scale else None)


def backward_cotangents(p: ChunkProblem, seed: int = 0, dS_final: bool = True):
    """Gradients of a loss with respect to the forward's outputs, for the
    backward: dO ~ N(0, 1) [B, H, L, Dv] and dS_final ~ N(0, 1)
    [B, H, Dk, Dv] (None with dS_final=False), fp32."""
    rng = np.random.default_rng([seed, 7919])
    dO = rng.standard_normal((p.B, p.H, p.L, p.Dv)).astype(np.float32)
    dSf = rng.standard_normal((p.B, p.H, p.Dk, p.Dv)).astype(np.float32) if dS_final else None
    return dO, dSf


# The named workloads.  Gate ranges are U(lo, hi) on log alpha.
GDN_GATE = (-0.1, -0.001)
KDA_GATE = (-0.2, -0.0005)

WORKLOADS = {
    # plain DeltaNet, fp32, alpha == 1, scalar beta, S0 = 0
    "deltanet_f32": dict(B=1, H=2, L=256, Dk=64, Dv=64, in_dtype="f32", gate="none",
                         beta_mode="scalar", s0_var=None),
    # Gated DeltaNet, scalar gate, bf16 inputs, S0 ~ N(0, 0.01)
    "gdn_b4h16_4k": dict(B=4, H=16, L=4096, Dk=128, Dv=128, in_dtype="bf16", gate="scalar",
                         beta_mode="scalar", log_alpha_range=GDN_GATE, s0_var=0.01),
    # KDA-style channel-wise gate, scalar beta, S0 = 0
    "kda_b2h32_16k": dict(B=2, H=32, L=16384, Dk=128, Dv=128, in_dtype="bf16", gate="channel",
                          beta_mode="scalar", log_alpha_range=KDA_GATE, s0_var=None),
    # FG2-GDN: channel-wise gate and channel-wise beta, S0 = 0
    "fg2_b2h16_16k": dict(B=2, H=16, L=16384, Dk=128, Dv=128, in_dtype="bf16", gate="channel",
                          beta_mode="channel", log_alpha_range=KDA_GATE, s0_var=None),
    # FG2-GDN+: as FG2-GDN with a separate channel-wise write strength beta^v
    "fg2plus_b2h16_16k": dict(B=2, H=16, L=16384, Dk=128, Dv=128, in_dtype="bf16", gate="channel",
                              beta_mode="channel", log_alpha_range=KDA_GATE, s0_var=None, beta_v=True),
    # the headline GDN shape with write-side key scales (a diagonal preconditioner)
    "gdn_precond_b2h16_16k": dict(B=2, H=16, L=16384, Dk=128, Dv=128, in_dtype="bf16", gate="scalar",
                                  beta_mode="scalar", log_alpha_range=GDN_GATE, s0_var=0.01, key_scale=True),
    # long-context GDN prefill, gating as the B=4 GDN workload
    "gdn_b1h16_64k": dict(B=1, H=16, L=65536, Dk=128, Dv=128, in_dtype="bf16", gate="scalar",
                          beta_mode="scalar", log_alpha_range=GDN_GATE, s0_var=0.01),
    # headline: scalar GDN gating at B=2, H=16, L=16K, d=128
    "gdn_b2h16_16k": dict(B=2, H=16, L=16384, Dk=128, Dv=128, in_dtype="bf16", gate="scalar",
                          beta_mode="scalar", log_alpha_range=GDN_GATE, s0_var=0.01),
}


def workload(name: str, seed: int = 0, **override) -> ChunkProblem:
    kw = dict(WORKLOADS[name])
    kw.update(override)
    return make_chunk_problem(seed=seed, name=name, **kw)


@dataclass
class DecodeProblem:
    """A batch of N sequences x H heads, each with its own state, stepped T times."""

    N: int
    H: int
    Dk: int
    Dv: int
    steps: int
    in_dtype: str
    gate: str
    beta_mode: str
    S: np.ndarray                 # [N, H, Dk, Dv] float32, the initial states
    q: np.ndarray                 # [steps, N, H, Dk]
    k: np.ndarray                 # [steps, N, H, Dk]
    v: np.ndarray                 # [steps, N, H, Dv]
    log_alpha: Optional[np.ndarray]   # [steps, N, H] or [steps, N, H, Dk]
    beta: np.ndarray              # [steps, N, H] or [steps, N, H, Dk]
    beta_v: Optional[np.ndarray] = None   # separate write strength (FG2-GDN+), beta's shape
    qk_l2norm: bool = False               # raw q, k and strength logits (see make_decode_problem)
    beta_logit: bool = False
    key_scale: Optional[np.ndarray] = None   # write-side key scales [steps, N, H, Dk]


def make_decode_problem(N=256, H=16, Dk=128, Dv=128, steps=512, *, in_dtype="bf16",
                        gate="scalar", beta_mode="scalar", log_alpha_range=GDN_GATE,
                        s0_var=0.01, seed=0, beta_v: bool = False,
                        raw_inputs: bool = False, key_scale: bool = False) -> DecodeProblem:
    """Decode batch: states first, then each step's tokens, in step order;
    with beta_v=True a separate write strength per step is drawn last, like
    beta, so the other arrays are those of beta_v=False.  raw_inputs=True
    keeps q and k unnormalised and the strengths as their logits."""
    rng = np.random.default_rng(seed)
    S = (rng.standard_normal((N, H, Dk, Dv)) * np.sqrt(s0_var)).astype(np.float32)
    qs, ks, vs, las, bs = [], [], [], [], []
    for _ in range(steps):
        q = rng.standard_normal((N, H, Dk))
        k = rng.standard_normal((N, H, Dk))
        v = rng.standard_normal((N, H, Dv))
        la = None
        if gate == "scalar":
            la = rng.uniform(log_alpha_range[0], log_alpha_range[1], (N, H))
        elif gate == "channel":
            la = rng.uniform(log_alpha_range[0], log_alpha_range[1], (N, H, Dk))
        bl = rng.standard_normal((N, H) if beta_mode == "scalar" else (N, H, Dk))
        qs.append(_to_dtype(q if raw_inputs else _l2norm(q), in_dtype))
        ks.append(_to_dtype(k if raw_inputs else _l2norm(k), in_dtype))
        vs.append(_to_dtype(v, in_dtype))
        las.append(None if la is None else la.astype(np.float32))
        bs.append((bl if raw_inputs else _sigmoid(bl)).astype(np.float32))
    bv = None
    if beta_v:
        bv = rng.standard_normal((steps,) + bs[0].shape)
        bv = (bv if raw_inputs else _sigmoid(bv)).astype(np.float32)
    return DecodeProblem(N, H, Dk, Dv, steps, in_dtype, gate, beta_mode, S,
                         np.stack(qs), np.stack(ks), np.stack(vs),
                         None if gate == "none" else np.stack(las), np.stack(bs), bv,
                         raw_inputs, raw_inputs,
                         rng.uniform(0.5, 1.5, (steps, N, H, Dk)).astype(np.float32) if key_scale else None)
