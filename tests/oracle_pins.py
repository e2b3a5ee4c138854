"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes a forward callable with the oracle's signature,
``fwd(q, k, v, log_alpha, beta, S0, gate=, beta_mode=) -> (o, S_final)``, and
raises AssertionError when the callable disagrees with what the pages and the
mathematics fix.  The same checks run against the real oracle
(test_oracle_pins.py) and against copies of it with planted mistakes
(test_oracle_mutants.py), which must each fail at least one of them.

Sources, cited by page and passage:
  [FG2-eq]   FG2-GDN page, section 2 "Kerninnovation": kt = sqrt(beta) (.) k,
             vt = sqrt(beta) (.) v; S_t = (I - kt kt^T) Diag(alpha_t) S_{t-1} + kt vt^T.
  [FG2-rk1]  same section, "Strukturelle Kompatibilitaet": the symmetric sqrt(beta)
             scaling keeps the transition a rank-one (Householder-type) update.
  [FG2-gate] FG2-GDN page, section 1: GDN's alpha is one scalar for all features,
             KDA's is a d_k-vector.
  [DN-steps] DeltaNet page, the seven-step list: read the map, error scaled by
             beta, outer-product update, output read from the updated state.
  [DN-beta]  DeltaNet page, property list: beta near 0 leaves the state almost
             unchanged, large beta overwrites.
  [DN-norm]  DeltaNet page, property list: without L2 normalisation the rule can
             diverge.
  [DN-inf]   DeltaNet page, property list: inference uses the recurrent form with
             a constant-size state (so a run can be resumed from its state).
  [QED]      The query-erase page: key-directed delta edits cannot change the
             key-orthogonal part of reads.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

RNG_SEED = 1234


def _rng(salt):
    return np.random.default_rng([RNG_SEED, salt])


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_case(salt, *, B=1, H=2, L=12, Dk=5, Dv=4, gate="scalar", beta_mode="scalar",
                s0=True, unit_keys=True):
    """Small fp64 case with generic values (no special structure)."""
    r = _rng(salt)
    q = r.standard_normal((B, H, L, Dk))
    k = r.standard_normal((B, H, L, Dk))
    if unit_keys:
        k = _unit(k)
    v = r.standard_normal((B, H, L, Dv))
    la = None
    if gate == "scalar":
        la = r.uniform(-0.7, -0.01, (B, H, L))
    elif gate == "channel":
        la = r.uniform(-0.7, -0.01, (B, H, L, Dk))
    beta = r.uniform(0.05, 1.0, (B, H, L) if beta_mode == "scalar" else (B, H, L, Dk))
    S0 = r.standard_normal((B, H, Dk, Dv)) if s0 else None
    return q, k, v, la, beta, S0


def _alpha_vec(la, t, gate, Dk):
    if gate == "none":
        return np.ones(Dk)
    if gate == "scalar":
        return np.full(Dk, np.exp(la[t]))
    return np.exp(la[t])


def _beta_vec(beta, t, beta_mode, Dk):
    return np.full(Dk, beta[t]) if beta_mode == "scalar" else beta[t]


def dense_reference(q, k, v, la, beta, S0, gate, beta_mode):
    """Literal [FG2-eq]: builds M_t = (I - kt kt^T) Diag(alpha_t) as a dense
    matrix and multiplies.  One (b, h) at a time; inputs [L, D]."""
    L, Dk = q.shape
    Dv = v.shape[1]
    S = np.zeros((Dk, Dv)) if S0 is None else S0.copy()
    o = np.zeros((L, Dv))
    for t in range(L):
        sb = np.sqrt(_beta_vec(beta, t, beta_mode, Dk))
        kt = sb * k[t]
        vt = (sb[:Dv] if beta_mode == "channel" else np.sqrt(beta[t])) * v[t]
        M = (np.eye(Dk) - np.outer(kt, kt)) @ np.diag(_alpha_vec(la, t, gate, Dk))
        S = M @ S + np.outer(kt, vt)
        o[t] = S.T @ q[t]
    return o, S


def _per_head(fn, q, k, v, la, beta, S0, gate, beta_mode):
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    o = np.zeros((B, H, L, Dv))
    S = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            o[b, h], S[b, h] = fn(q[b, h], k[b, h], v[b, h], None if la is None else la[b, h],
                                  beta[b, h], None if S0 is None else S0[b, h], gate, beta_mode)
    return o, S


def _close(x, y, tol, what):
    err = np.max(np.abs(np.asarray(x) - np.asarray(y)))
    scale = max(1.0, np.max(np.abs(y)))
    assert err <= tol * scale, f"{what}: max abs err {err:.3e} > {tol:.1e} * {scale:.3g}"


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------

def pin_dense_product(fwd):
    """Oracle == literal dense product (I - kt kt^T) Diag(alpha) S + kt vt^T
    [FG2-eq], every gate and beta mode, d_k != d_v where allowed."""
    salt = 0
    for gate in ("none", "scalar", "channel"):
        for beta_mode in ("scalar", "channel"):
            Dk, Dv = (6, 6) if beta_mode == "channel" else (6, 4)
            salt += 1
            args = random_case(salt, L=11, Dk=Dk, Dv=Dv, gate=gate, beta_mode=beta_mode)
            o, S = fwd(*args, gate=gate, beta_mode=beta_mode)
            oy, Sy = _per_head(dense_reference, *args, gate, beta_mode)
            _close(o, oy, 1e-12, f"o ({gate},{beta_mode})")
            _close(S, Sy, 1e-12, f"S ({gate},{beta_mode})")


def pin_transition_products(fwd):
    """Whole-sequence brute force [FG2-eq]: S_L = (prod_t M_t) S0 +
    sum_t (prod_{s>t} M_s) kt_t vt_t^T, o_t = S_t^T q_t with S_t from the
    same expansion, on d_k <= 8, L <= 16."""
    for salt, (gate, beta_mode) in enumerate([("scalar", "scalar"), ("channel", "channel"),
                                              ("channel", "scalar")]):
        q, k, v, la, beta, S0 = random_case(100 + salt, B=1, H=1, L=16, Dk=8, Dv=8,
                                            gate=gate, beta_mode=beta_mode)
        o, S = fwd(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode)
        qq, kk, vv, SS = q[0, 0], k[0, 0], v[0, 0], S0[0, 0]
        ll = None if la is None else la[0, 0]
        bb = beta[0, 0]
        Ms, ws = [], []
        for t in range(16):
            sb = np.sqrt(_beta_vec(bb, t, beta_mode, 8))
            kt, vt = sb * kk[t], sb * vv[t]
            Ms.append((np.eye(8) - np.outer(kt, kt)) @ np.diag(_alpha_vec(ll, t, gate, 8)))
            ws.append(np.outer(kt, vt))
        for t in range(16):
            prod_all = np.eye(8)
            for u in range(t + 1):
                prod_all = Ms[u] @ prod_all
            St = prod_all @ SS
            for s in range(t + 1):
                P = np.eye(8)
                for u in range(s + 1, t + 1):
                    P = Ms[u] @ P
                St = St + P @ ws[s]
            _close(o[0, 0, t], St.T @ qq[t], 1e-11, f"o_t t={t} ({gate},{beta_mode})")
        _close(S[0, 0], St, 1e-11, f"S_L ({gate},{beta_mode})")


def pin_exact_rational(fwd):
    """Exact rational arithmetic of [FG2-eq] (no floating point) on a DeltaNet
    case whose beta values are perfect squares, so sqrt(beta) is rational."""
    L, Dk, Dv = 5, 3, 2
    # integer key rows with integer norms, so the unit keys are rational
    kk = [[1, 2, 2], [3, 4, 0], [0, 3, 4], [1, 0, 0], [2, 2, 1]]
    norms = [3, 5, 5, 1, 3]
    kf = [[Fraction(x, n) for x in row] for row, n in zip(kk, norms)]
    vf = [[Fraction(1), Fraction(-2)], [Fraction(3, 2), Fraction(0)], [Fraction(-1), Fraction(1, 4)],
          [Fraction(2), Fraction(2)], [Fraction(0), Fraction(-3)]]
    qf = [[Fraction(1), Fraction(0), Fraction(1, 2)], [Fraction(0), Fraction(1), Fraction(0)],
          [Fraction(1, 4), Fraction(1, 4), Fraction(1, 4)], [Fraction(1), Fraction(1), Fraction(-1)],
          [Fraction(-1), Fraction(2), Fraction(0)]]
    sqrtb = [Fraction(1), Fraction(1, 2), Fraction(3, 4), Fraction(1, 3), Fraction(2, 3)]
    S = [[Fraction(1, 2), Fraction(-1)], [Fraction(0), Fraction(2)], [Fraction(1), Fraction(1, 8)]]
    S0 = [row[:] for row in S]
    o_exact = []
    for t in range(L):
        kt = [sqrtb[t] * x for x in kf[t]]
        vt = [sqrtb[t] * x for x in vf[t]]
        # M = I - kt kt^T ; S <- M S + kt vt^T
        newS = [[sum(((1 if c == d else 0) - kt[c] * kt[d]) * S[d][j] for d in range(Dk)) + kt[c] * vt[j]
                 for j in range(Dv)] for c in range(Dk)]
        S = newS
        o_exact.append([sum(S[c][j] * qf[t][c] for c in range(Dk)) for j in range(Dv)])
    f = lambda a: np.array([[float(x) for x in r] for r in a])
    q = f(qf)[None, None]
    k = f(kf)[None, None]
    v = f(vf)[None, None]
    beta = np.array([float(s * s) for s in sqrtb])[None, None]
    o, Sf = fwd(q, k, v, None, beta, f(S0)[None, None], gate="none", beta_mode="scalar")
    _close(o[0, 0], f(o_exact), 1e-13, "o vs exact rationals")
    _close(Sf[0, 0], f(S), 1e-13, "S vs exact rationals")


def pin_residual_and_orthogonal_reads(fwd):
    """Per step, with S' = Diag(alpha_t) S_{t-1}:
    (i) residual contraction S_t^T kt - vt = (1 - |kt|^2)(S'^T kt - vt) [DN-steps],
    (ii) reads along any x orthogonal to kt are unchanged, S_t^T x = S'^T x [QED].
    Together (i) and (ii) determine S_t uniquely."""
    for gate, beta_mode in (("scalar", "scalar"), ("channel", "channel"), ("none", "scalar")):
        q, k, v, la, beta, S0 = random_case(200, B=1, H=1, L=7, Dk=6, Dv=6, gate=gate,
                                            beta_mode=beta_mode, unit_keys=False)
        S_prev = S0[0, 0]
        r = _rng(201)
        for t in range(7):
            sl = lambda a: None if a is None else a[:, :, : t + 1]
            _, S_t = fwd(sl(q), sl(k), sl(v), sl(la), sl(beta), S0, gate=gate, beta_mode=beta_mode)
            S_t = S_t[0, 0]
            sb = np.sqrt(_beta_vec(beta[0, 0], t, beta_mode, 6))
            kt, vt = sb * k[0, 0, t], sb * v[0, 0, t]
            Sp = np.diag(_alpha_vec(None if la is None else la[0, 0], t, gate, 6)) @ S_prev
            _close(S_t.T @ kt - vt, (1 - kt @ kt) * (Sp.T @ kt - vt), 1e-12, f"residual t={t} {gate}")
            for _ in range(3):
                x = r.standard_normal(6)
                x -= (x @ kt) / (kt @ kt) * kt
                _close(S_t.T @ x, Sp.T @ x, 1e-12, f"orthogonal read t={t} {gate}")
            S_prev = S_t


def pin_beta_zero_pure_decay(fwd):
    """beta = 0 leaves the state at its decayed previous value [DN-beta]; over a
    whole sequence S_L = Diag(exp(sum_t log alpha_t)) S0 and o_t = S_t^T q_t."""
    for gate in ("scalar", "channel", "none"):
        q, k, v, la, beta, S0 = random_case(300, L=9, Dk=5, Dv=3, gate=gate)
        beta = np.zeros_like(beta)
        o, S = fwd(q, k, v, la, beta, S0, gate=gate, beta_mode="scalar")
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                for t in range(9):
                    if gate == "none":
                        g = np.zeros(5)
                    elif gate == "scalar":
                        g = np.full(5, la[b, h, : t + 1].sum())
                    else:
                        g = la[b, h, : t + 1].sum(axis=0)
                    St = np.exp(g)[:, None] * S0[b, h]
                    _close(o[b, h, t], St.T @ q[b, h, t], 1e-12, f"o t={t} {gate}")
                _close(S[b, h], St, 1e-12, f"S_L {gate}")


def pin_overwrite_recall(fwd):
    """alpha = 1, beta = 1, unit keys: the state overwrites, so querying with the
    key just written returns its value [DN-steps, DN-beta]; with orthonormal keys
    k_1..k_n, S_n = (I - K^T K) S0 + K^T V and S_n^T k_i = v_i (projection)."""
    r = _rng(400)
    Dk, Dv, n = 7, 5, 5
    Qm, _ = np.linalg.qr(r.standard_normal((Dk, Dk)))
    K = Qm[:n]                       # n orthonormal rows
    V = r.standard_normal((n, Dv))
    S0 = r.standard_normal((Dk, Dv))
    q = K.copy()                     # query each key right after writing it
    o, S = fwd(q[None, None], K[None, None], V[None, None], None, np.ones((1, 1, n)),
               S0[None, None], gate="none", beta_mode="scalar")
    _close(o[0, 0], V, 1e-12, "o_t == v_t when q_t == k_t")
    _close(S[0, 0], (np.eye(Dk) - K.T @ K) @ S0 + K.T @ V, 1e-12, "projection closed form")
    _close(K @ S[0, 0], V, 1e-12, "S_n^T k_i == v_i")
    # a generic (non-orthogonal) unit key sequence still recalls the last write
    q2, k2, v2, _, _, S02 = random_case(401, L=6, Dk=4, Dv=3, gate="none")
    o2, _ = fwd(k2, k2, v2, None, np.ones((1, 2, 6)), S02, gate="none", beta_mode="scalar")
    _close(o2, v2, 1e-12, "last write recalled")


def pin_transition_structure(fwd):
    """The transition's deviation from the decay is symmetric rank one with
    eigenvalue -|kt|^2 [FG2-rk1]: run one step from S0 = I with v = 0, read
    M = S_1, check M Diag(alpha)^-1 - I == -kt kt^T.  With |kt|^2 > 2 the
    eigenvalue 1 - |kt|^2 exceeds 1 in modulus and repeated writes of that key
    diverge; with |kt|^2 < 2 they contract [DN-norm]."""
    r = _rng(500)
    Dk = 6
    for gate in ("scalar", "channel"):
        k = r.standard_normal(Dk) * 0.6
        la = r.uniform(-0.5, -0.05, Dk if gate == "channel" else ())
        b = r.uniform(0.2, 1.0, Dk)
        alpha = np.exp(la) * np.ones(Dk)
        _, M = fwd(np.zeros((1, 1, 1, Dk)), k[None, None, None], np.zeros((1, 1, 1, Dk)),
                   np.asarray(la)[None, None, None], b[None, None, None], np.eye(Dk)[None, None],
                   gate=gate, beta_mode="channel")
        D = M[0, 0] @ np.diag(1 / alpha) - np.eye(Dk)
        kt = np.sqrt(b) * k
        _close(D, -np.outer(kt, kt), 1e-12, f"rank-one deviation ({gate})")
        ev = np.sort(np.linalg.eigvalsh((D + D.T) / 2))
        _close(ev[0], -(kt @ kt), 1e-12, "eigenvalue -|kt|^2")
        _close(ev[1:], np.zeros(Dk - 1), 1e-12, "other eigenvalues 0")
    for scale, grows in ((np.sqrt(2.5), True), (np.sqrt(1.5), False)):
        k = np.zeros(4)
        k[0] = scale                      # |k|^2 = 2.5 (diverges) or 1.5 (contracts)
        L = 30
        kk = np.tile(k, (L, 1))[None, None]
        _, S = fwd(np.zeros((1, 1, L, 4)), kk, np.zeros((1, 1, L, 2)), None, np.ones((1, 1, L)),
                   np.ones((1, 1, 4, 2)), gate="none", beta_mode="scalar")
        amp = abs(S[0, 0, 0, 0])
        want = abs(1 - k @ k) ** L
        assert abs(amp - want) <= 1e-9 * max(1, want), f"amplitude {amp} vs {want}"
        assert (amp > 1e3) == grows


def pin_fg2_as_scaled_deltanet(fwd):
    """Channel beta is a scalar DeltaNet step on the normalised key:
    kt = sqrt(beta) (.) k equals sqrt(b') k^ with k^ = kt/|kt|, b' = |kt|^2, and
    vt = sqrt(b') v' with v' = vt/|kt| [FG2-eq, FG2-rk1]."""
    for gate in ("channel", "scalar"):
        q, k, v, la, beta, S0 = random_case(600, L=10, Dk=6, Dv=6, gate=gate, beta_mode="channel",
                                            unit_keys=False)
        o1, S1 = fwd(q, k, v, la, beta, S0, gate=gate, beta_mode="channel")
        kt = np.sqrt(beta) * k
        vt = np.sqrt(beta) * v
        nk = np.linalg.norm(kt, axis=-1)
        o2, S2 = fwd(q, kt / nk[..., None], vt / nk[..., None], la, nk ** 2, S0, gate=gate,
                     beta_mode="scalar")
        _close(o1, o2, 1e-12, f"o channel-beta vs scalar form ({gate})")
        _close(S1, S2, 1e-12, f"S channel-beta vs scalar form ({gate})")


def pin_cross_mode(fwd):
    """A d_k-vector gate with equal entries is the scalar gate; a channel beta
    with equal entries is the scalar beta; gate none is log alpha = 0 [FG2-gate]."""
    q, k, v, la, beta, S0 = random_case(700, L=10, Dk=5, Dv=5, gate="scalar")
    ref = fwd(q, k, v, la, beta, S0, gate="scalar", beta_mode="scalar")
    lac = np.repeat(la[..., None], 5, axis=-1)
    bc = np.repeat(beta[..., None], 5, axis=-1)
    for got, what in ((fwd(q, k, v, lac, beta, S0, gate="channel", beta_mode="scalar"), "channel gate"),
                      (fwd(q, k, v, la, bc, S0, gate="scalar", beta_mode="channel"), "channel beta"),
                      (fwd(q, k, v, lac, bc, S0, gate="channel", beta_mode="channel"), "both")):
        _close(got[0], ref[0], 1e-12, f"o {what}")
        _close(got[1], ref[1], 1e-12, f"S {what}")
    a = fwd(q, k, v, None, beta, S0, gate="none", beta_mode="scalar")
    b = fwd(q, k, v, np.zeros_like(la), beta, S0, gate="scalar", beta_mode="scalar")
    _close(a[0], b[0], 0.0, "o none vs log alpha = 0")
    _close(a[1], b[1], 0.0, "S none vs log alpha = 0")


def pin_split_and_resume(fwd):
    """Running L tokens equals running L1 tokens then the rest from S_final
    [DN-inf]; equivalently prefill of L - n tokens followed by n one-token
    steps (decode) equals prefill of L."""
    for gate, beta_mode in (("scalar", "scalar"), ("channel", "channel")):
        q, k, v, la, beta, S0 = random_case(800, L=13, Dk=4, Dv=4, gate=gate, beta_mode=beta_mode)
        o, S = fwd(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode)
        cut = lambda a, s: None if a is None else a[:, :, s]
        for L1 in (1, 5, 12):
            a = slice(0, L1)
            b = slice(L1, 13)
            oa, Sa = fwd(cut(q, a), cut(k, a), cut(v, a), cut(la, a), cut(beta, a), S0,
                         gate=gate, beta_mode=beta_mode)
            ob, Sb = fwd(cut(q, b), cut(k, b), cut(v, b), cut(la, b), cut(beta, b), Sa,
                         gate=gate, beta_mode=beta_mode)
            _close(np.concatenate([oa, ob], axis=2), o, 1e-13, f"o split at {L1}")
            _close(Sb, S, 1e-13, f"S split at {L1}")
        Sc = S0
        outs = []
        for t in range(13):
            s = slice(t, t + 1)
            ot, Sc = fwd(cut(q, s), cut(k, s), cut(v, s), cut(la, s), cut(beta, s), Sc,
                         gate=gate, beta_mode=beta_mode)
            outs.append(ot)
        _close(np.concatenate(outs, axis=2), o, 1e-13, "o one token at a time")
        _close(Sc, S, 1e-13, "S one token at a time")


def pin_zero_state_defaults(fwd):
    """S0 absent means a zero initial state; a zero-length run returns S0."""
    q, k, v, la, beta, _ = random_case(900, L=6, Dk=4, Dv=3, gate="scalar")
    a = fwd(q, k, v, la, beta, None, gate="scalar", beta_mode="scalar")
    b = fwd(q, k, v, la, beta, np.zeros((1, 2, 4, 3)), gate="scalar", beta_mode="scalar")
    _close(a[0], b[0], 0.0, "o with S0 None vs zeros")
    _close(a[1], b[1], 0.0, "S with S0 None vs zeros")


ALL_PINS = [
    pin_dense_product,
    pin_transition_products,
    pin_exact_rational,
    pin_residual_and_orthogonal_reads,
    pin_beta_zero_pure_decay,
    pin_overwrite_recall,
    pin_transition_structure,
    pin_fg2_as_scaled_deltanet,
    pin_cross_mode,
    pin_split_and_resume,
    pin_zero_state_defaults,
]


# ---------------------------------------------------------------------------
# Separate erase and write strengths (FG2-GDN page, section "Erweiterung:
# FG2-GDN+").  The page prints no equation; the reading pinned here is
# kt = sqrt(beta^k) k in both the erase and the write term and
# vt = sqrt(beta^v) v.  Each pin takes fwd_kv(q, k, v, la, beta, beta_v, S0,
# *, gate, beta_mode).
# ---------------------------------------------------------------------------

def _dense_kv(q, k, v, la, beta, beta_v, S0, gate, beta_mode):
    L, Dk = q.shape
    Dv = v.shape[1]
    S = np.zeros((Dk, Dv)) if S0 is None else S0.copy()
    o = np.zeros((L, Dv))
    for t in range(L):
        sk = np.sqrt(_beta_vec(beta, t, beta_mode, Dk))
        sv = np.sqrt(_beta_vec(beta_v, t, beta_mode, Dk))
        kt = sk * k[t]
        vt = (sv[:Dv] if beta_mode == "channel" else sv[0]) * v[t]
        M = (np.eye(Dk) - np.outer(kt, kt)) @ np.diag(_alpha_vec(la, t, gate, Dk))
        S = M @ S + np.outer(kt, vt)
        o[t] = S.T @ q[t]
    return o, S


def pin_kv_dense_product(fwd_kv):
    """Oracle == literal dense product with vt scaled by sqrt(beta^v) and kt by
    sqrt(beta^k) in both terms, every gate and beta mode."""
    salt = 40
    for gate in ("none", "scalar", "channel"):
        for beta_mode in ("scalar", "channel"):
            Dk, Dv = (6, 6) if beta_mode == "channel" else (6, 4)
            salt += 1
            q, k, v, la, beta, S0 = random_case(salt, B=2, H=2, L=9, Dk=Dk, Dv=Dv, gate=gate,
                                                beta_mode=beta_mode)
            bv = _rng(salt + 100).uniform(0.05, 1.0, beta.shape)
            o, S = fwd_kv(q, k, v, la, beta, bv, S0, gate=gate, beta_mode=beta_mode)
            for b in range(2):
                for h in range(2):
                    oy, Sy = _dense_kv(q[b, h], k[b, h], v[b, h], None if la is None else la[b, h],
                                       beta[b, h], bv[b, h], S0[b, h], gate, beta_mode)
                    _close(o[b, h], oy, 1e-12, f"o ({gate},{beta_mode})")
                    _close(S[b, h], Sy, 1e-12, f"S ({gate},{beta_mode})")


def pin_kv_write_scaling(fwd_kv):
    """From S0 = 0 the recurrence is linear in vt for fixed kt and alpha:
    beta^v = c^2 beta^k scales every output and the final state by c."""
    for beta_mode in ("scalar", "channel"):
        q, k, v, la, beta, _ = random_case(60, L=14, Dk=6, Dv=6, gate="scalar",
                                           beta_mode=beta_mode, s0=False)
        c = 0.37
        o1, S1 = fwd_kv(q, k, v, la, beta, beta, None, gate="scalar", beta_mode=beta_mode)
        o2, S2 = fwd_kv(q, k, v, la, beta, c * c * beta, None, gate="scalar", beta_mode=beta_mode)
        _close(o2, c * o1, 1e-13, f"o ({beta_mode})")
        _close(S2, c * S1, 1e-13, f"S ({beta_mode})")


def pin_kv_superposition(fwd_kv):
    """The response to (S0, writes) is the response to (S0, no writes) plus the
    response to (0, writes): beta^v enters only the write term."""
    for beta_mode in ("scalar", "channel"):
        q, k, v, la, beta, S0 = random_case(61, L=13, Dk=5, Dv=5, gate="channel",
                                            beta_mode=beta_mode)
        bv = _rng(62).uniform(0.05, 1.0, beta.shape)
        o, S = fwd_kv(q, k, v, la, beta, bv, S0, gate="channel", beta_mode=beta_mode)
        oa, Sa = fwd_kv(q, k, v, la, beta, np.zeros_like(bv), S0, gate="channel",
                        beta_mode=beta_mode)
        ob, Sb = fwd_kv(q, k, v, la, beta, bv, None, gate="channel", beta_mode=beta_mode)
        _close(o, oa + ob, 1e-12, f"o ({beta_mode})")
        _close(S, Sa + Sb, 1e-12, f"S ({beta_mode})")


KV_PINS = [pin_kv_dense_product, pin_kv_write_scaling, pin_kv_superposition]


# ---------------------------------------------------------------------------
# Input preparation in front of the recurrence (DeltaNet page, step list,
# step 2 and its notes on the key/query map and on choosing beta): qk_l2norm
# makes q and k unit vectors, beta_logit reads the strengths as logits.
# Each pin takes fwd_ex(q, k, v, la, beta, beta_v, S0, *, gate, beta_mode,
# qk_l2norm, beta_logit); beta_v may be None (one strength).
# ---------------------------------------------------------------------------

def _modes():
    return [("none", "scalar"), ("scalar", "scalar"), ("channel", "scalar"), ("scalar", "channel"),
            ("channel", "channel")]


def pin_l2norm_ray_invariance(fwd_ex):
    """With qk_l2norm the result depends on q_t and k_t only through their
    directions: positive per-token rescaling changes nothing."""
    for n, (gate, beta_mode) in enumerate(_modes()):
        q, k, v, la, beta, S0 = random_case(70 + n, L=11, Dk=5, Dv=5, gate=gate, beta_mode=beta_mode,
                                            unit_keys=False)
        r = _rng(80 + n)
        cq = r.uniform(0.2, 5.0, q.shape[:-1] + (1,))
        ck = r.uniform(0.2, 5.0, k.shape[:-1] + (1,))
        kw = dict(gate=gate, beta_mode=beta_mode, qk_l2norm=True, beta_logit=False)
        o1, S1 = fwd_ex(q, k, v, la, beta, None, S0, **kw)
        o2, S2 = fwd_ex(q * cq, k * ck, v, la, beta, None, S0, **kw)
        _close(o2, o1, 1e-12, f"o ({gate},{beta_mode})")
        _close(S2, S1, 1e-12, f"S ({gate},{beta_mode})")


def pin_l2norm_fixes_unit_and_zero_vectors(fwd_ex):
    """Unit vectors, and the zero vector, pass through the normalisation
    unchanged.  With the ray invariance above this fixes the map x / |x|_2."""
    for n, (gate, beta_mode) in enumerate(_modes()):
        q, k, v, la, beta, S0 = random_case(90 + n, L=11, Dk=5, Dv=5, gate=gate, beta_mode=beta_mode)
        q = _unit(q)
        q[:, :, 3] = 0.0
        k[:, :, 5] = 0.0
        kw = dict(gate=gate, beta_mode=beta_mode, beta_logit=False)
        o1, S1 = fwd_ex(q, k, v, la, beta, None, S0, qk_l2norm=True, **kw)
        o2, S2 = fwd_ex(q, k, v, la, beta, None, S0, qk_l2norm=False, **kw)
        assert np.isfinite(o1).all() and np.isfinite(S1).all()
        _close(o1, o2, 1e-13, f"o ({gate},{beta_mode})")
        _close(S1, S2, 1e-13, f"S ({gate},{beta_mode})")


def pin_beta_logit_round_trip(fwd_ex):
    """Strengths given as logits log(b / (1 - b)) reproduce the run with the
    strengths b themselves, for one strength and for separate erase and
    write strengths."""
    for n, (gate, beta_mode) in enumerate(_modes()):
        q, k, v, la, beta, S0 = random_case(100 + n, L=11, Dk=5, Dv=5, gate=gate, beta_mode=beta_mode)
        bv = _rng(110 + n).uniform(0.05, 0.95, beta.shape)
        logit = lambda b: np.log(b) - np.log1p(-b)
        kw = dict(gate=gate, beta_mode=beta_mode, qk_l2norm=False)
        for b_v in (None, bv):
            o1, S1 = fwd_ex(q, k, v, la, beta, b_v, S0, beta_logit=False, **kw)
            o2, S2 = fwd_ex(q, k, v, la, logit(beta), None if b_v is None else logit(b_v), S0,
                            beta_logit=True, **kw)
            _close(o2, o1, 1e-12, f"o ({gate},{beta_mode})")
            _close(S2, S1, 1e-12, f"S ({gate},{beta_mode})")


def pin_beta_logit_saturation(fwd_ex):
    """Logit +60 is a full write (beta = 1 to 1e-26), logit -60 no write at
    all: the state only decays (the closed form of beta = 0)."""
    q, k, v, la, beta, S0 = random_case(120, L=9, Dk=5, Dv=5, gate="channel", beta_mode="channel")
    kw = dict(gate="channel", beta_mode="channel", qk_l2norm=False)
    o1, S1 = fwd_ex(q, k, v, la, np.full_like(beta, 60.0), None, S0, beta_logit=True, **kw)
    o2, S2 = fwd_ex(q, k, v, la, np.ones_like(beta), None, S0, beta_logit=False, **kw)
    _close(o1, o2, 1e-13, "o at logit +60")
    _close(S1, S2, 1e-13, "S at logit +60")
    _, S3 = fwd_ex(q, k, v, la, np.full_like(beta, -60.0), None, S0, beta_logit=True, **kw)
    decay = np.exp(la.sum(axis=2))                       # [B, H, Dk]
    _close(S3, decay[..., None] * S0, 1e-12, "S at logit -60")


PREP_PINS = [pin_l2norm_ray_invariance, pin_l2norm_fixes_unit_and_zero_vectors,
             pin_beta_logit_round_trip, pin_beta_logit_saturation]


# ---------------------------------------------------------------------------
# Write-side key scaling: a diagonal preconditioner s_t on the delta rule's
# gradient step (OSDN page, "Method"; the preconditioned delta rule page,
# abstract), given as an input.  Each pin takes
# fwd_ks(q, k, v, la, beta, key_scale, S0, *, gate, beta_mode).
# ---------------------------------------------------------------------------

def _dense_ks(q, k, v, la, beta, ks, S0, gate, beta_mode):
    L, Dk = q.shape
    Dv = v.shape[1]
    S = S0.copy()
    o = np.zeros((L, Dv))
    for t in range(L):
        sb = np.sqrt(_beta_vec(beta, t, beta_mode, Dk))
        kt = sb * k[t]
        vt = (sb[:Dv] if beta_mode == "channel" else sb[0]) * v[t]
        w = ks[t] * kt
        S = (np.eye(Dk) - np.outer(w, kt)) @ np.diag(_alpha_vec(la, t, gate, Dk)) @ S + np.outer(w, vt)
        o[t] = S.T @ q[t]
    return o, S


def pin_ks_dense_product(fwd_ks):
    """Oracle == literal dense (I - w kt^T) Diag(alpha) S + w vt^T, w = s (.) kt,
    every gate and beta mode."""
    salt = 150
    for gate in ("none", "scalar", "channel"):
        for beta_mode in ("scalar", "channel"):
            salt += 1
            q, k, v, la, beta, S0 = random_case(salt, B=2, H=2, L=9, Dk=6, Dv=6, gate=gate,
                                                beta_mode=beta_mode)
            ks = _rng(salt + 50).uniform(0.2, 2.0, q.shape)
            o, S = fwd_ks(q, k, v, la, beta, ks, S0, gate=gate, beta_mode=beta_mode)
            for b in range(2):
                for h in range(2):
                    oy, Sy = _dense_ks(q[b, h], k[b, h], v[b, h], None if la is None else la[b, h],
                                       beta[b, h], ks[b, h], S0[b, h], gate, beta_mode)
                    _close(o[b, h], oy, 1e-12, f"o ({gate},{beta_mode})")
                    _close(S[b, h], Sy, 1e-12, f"S ({gate},{beta_mode})")


def pin_ks_preconditioned_gradient_step(fwd_ks):
    """One token from S0 is S' - Diag(s) grad, with S' = Diag(alpha) S0 and grad
    the gradient at S' of the inner regression loss 1/2 |S^T kt - vt|^2, taken
    here by central differences (exact for a quadratic up to rounding)."""
    q, k, v, la, beta, S0 = random_case(160, B=1, H=1, L=1, Dk=5, Dv=4, gate="channel",
                                        beta_mode="scalar")
    ks = _rng(161).uniform(0.2, 2.0, q.shape)
    _, S1 = fwd_ks(q, k, v, la, beta, ks, S0, gate="channel", beta_mode="scalar")
    kt = np.sqrt(beta[0, 0, 0]) * k[0, 0, 0]
    vt = np.sqrt(beta[0, 0, 0]) * v[0, 0, 0]
    Sp = np.exp(la[0, 0, 0])[:, None] * S0[0, 0]
    loss = lambda S: 0.5 * np.sum((S.T @ kt - vt) ** 2)
    grad = np.zeros_like(Sp)
    h = 1e-3
    for i in range(Sp.shape[0]):
        for j in range(Sp.shape[1]):
            E = np.zeros_like(Sp)
            E[i, j] = h
            grad[i, j] = (loss(Sp + E) - loss(Sp - E)) / (2 * h)
    _close(S1[0, 0], Sp - ks[0, 0, 0][:, None] * grad, 1e-9, "S after one step")


def pin_ks_unit_and_zero_scales(fwd_ks):
    """s = 1 is the unscaled recurrence; s = 0 neither erases nor writes, so the
    state only decays: S_L = Diag(e^{sum log alpha}) S0."""
    q, k, v, la, beta, S0 = random_case(170, L=10, Dk=5, Dv=5, gate="channel", beta_mode="channel")
    kw = dict(gate="channel", beta_mode="channel")
    o1, S1 = fwd_ks(q, k, v, la, beta, np.ones_like(q), S0, **kw)
    o2, S2 = fwd_ks(q, k, v, la, beta, None, S0, **kw)
    _close(o1, o2, 1e-14, "o at s = 1")
    _close(S1, S2, 1e-14, "S at s = 1")
    _, S3 = fwd_ks(q, k, v, la, beta, np.zeros_like(q), S0, **kw)
    _close(S3, np.exp(la.sum(axis=2))[..., None] * S0, 1e-12, "S at s = 0")


KS_PINS = [pin_ks_dense_product, pin_ks_preconditioned_gradient_step, pin_ks_unit_and_zero_scales]


# ---------------------------------------------------------------------------
# The backward (gradients of the one-strength forward).  Each pin takes
# fwd(q, k, v, la, beta, S0, *, gate, beta_mode) -> (o, S_final) and
# bwd(q, k, v, la, beta, S0, dO, dS_final, *, gate, beta_mode) -> dict.
# ---------------------------------------------------------------------------

def _bwd_case(salt, gate, beta_mode, L=7, Dk=5, Dv=5):
    q, k, v, la, beta, S0 = random_case(salt, L=L, Dk=Dk, Dv=Dv, gate=gate, beta_mode=beta_mode)
    beta = 0.2 + 0.7 * beta   # away from 0, where sqrt has no derivative
    r = _rng(salt + 1000)
    Wo = r.standard_normal((1, 2, L, Dv))
    WS = r.standard_normal((1, 2, Dk, Dv))
    return q, k, v, la, beta, S0, Wo, WS


def pin_bwd_directional_derivatives(fwd, bwd):
    """For the loss <Wo, o> + <WS, S_final>, the gradients' inner product with
    a random direction, for each input alone and for all at once, equals the
    central difference of the loss along that direction."""
    salt = 200
    for gate in ("none", "scalar", "channel"):
        for beta_mode in ("scalar", "channel"):
            salt += 1
            q, k, v, la, beta, S0, Wo, WS = _bwd_case(salt, gate, beta_mode)
            kw = dict(gate=gate, beta_mode=beta_mode)
            g = bwd(q, k, v, la, beta, S0, Wo, WS, **kw)
            x = dict(q=q, k=k, v=v, la=la, beta=beta, S0=S0)
            grads = dict(q=g["dq"], k=g["dk"], v=g["dv"], la=g["dlog_alpha"], beta=g["dbeta"], S0=g["dS0"])
            r = _rng(salt + 2000)
            dirs = {n: (None if a is None else r.standard_normal(a.shape)) for n, a in x.items()}

            def loss(xx):
                o, S = fwd(xx["q"], xx["k"], xx["v"], xx["la"], xx["beta"], xx["S0"], **kw)
                return float(np.sum(Wo * o) + np.sum(WS * S))

            for which in [[n] for n in x if x[n] is not None] + [[n for n in x if x[n] is not None]]:
                h = 1e-5
                xp = {n: (a if a is None else (a + h * dirs[n] if n in which else a)) for n, a in x.items()}
                xm = {n: (a if a is None else (a - h * dirs[n] if n in which else a)) for n, a in x.items()}
                fd = (loss(xp) - loss(xm)) / (2 * h)
                an = sum(float(np.sum(grads[n] * dirs[n])) for n in which)
                assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), \
                    f"({gate},{beta_mode}) d/d{'+'.join(which)}: analytic {an:.10e} vs difference {fd:.10e}"


def pin_bwd_linear_inputs(fwd, bwd):
    """o and S_final are linear in (v, S0) jointly and o is linear in q, so the
    loss equals <dv, v> + <dS0, S0> exactly, and its o part <dq, q> (Euler's
    theorem for degree-1 homogeneous functions)."""
    # the last case has d_v well above d_k (value-sized scratch in the forward step)
    for n, (gate, beta_mode, Dk, Dv) in enumerate([("scalar", "scalar", 5, 5), ("channel", "channel", 5, 5),
                                                   ("scalar", "scalar", 3, 19)]):
        q, k, v, la, beta, S0, Wo, WS = _bwd_case(300 + n, gate, beta_mode, Dk=Dk, Dv=Dv)
        kw = dict(gate=gate, beta_mode=beta_mode)
        o, S = fwd(q, k, v, la, beta, S0, **kw)
        g = bwd(q, k, v, la, beta, S0, Wo, WS, **kw)
        total = np.sum(Wo * o) + np.sum(WS * S)
        _close(np.sum(g["dv"] * v) + np.sum(g["dS0"] * S0), total, 1e-12, f"v, S0 ({gate},{beta_mode})")
        g0 = bwd(q, k, v, la, beta, S0, Wo, np.zeros_like(WS), **kw)
        _close(np.sum(g0["dq"] * q), np.sum(Wo * o), 1e-12, f"q ({gate},{beta_mode})")


BWD_PINS = [pin_bwd_directional_derivatives, pin_bwd_linear_inputs]


# Backward with a separate write strength (FG2-GDN+).  Each pin takes
# fwd(q, k, v, la, beta, S0, *, gate, beta_mode, beta_v) -> (o, S_final) and
# bwd(q, k, v, la, beta, S0, dO, dS_final, *, gate, beta_mode, beta_v) -> dict
# (with dbeta_v).

def pin_bwd_kv_directional_derivatives(fwd, bwd):
    """With beta^v separate from beta^k: for <Wo, o> + <WS, S_final>, the
    gradients' inner product with random directions (each input alone, beta^v
    included, then all at once) equals the central difference of the loss,
    every gate, channel-wise strengths."""
    salt = 260
    for gate in ("none", "scalar", "channel"):
        salt += 1
        q, k, v, la, beta, S0, Wo, WS = _bwd_case(salt, gate, "channel")
        bv = 0.2 + 0.7 * _rng(salt + 3000).uniform(0.0, 1.0, beta.shape)
        kw = dict(gate=gate, beta_mode="channel")
        g = bwd(q, k, v, la, beta, S0, Wo, WS, beta_v=bv, **kw)
        x = dict(q=q, k=k, v=v, la=la, beta=beta, bv=bv, S0=S0)
        grads = dict(q=g["dq"], k=g["dk"], v=g["dv"], la=g["dlog_alpha"], beta=g["dbeta"], bv=g["dbeta_v"],
                     S0=g["dS0"])
        r = _rng(salt + 2000)
        dirs = {n: (None if a is None else r.standard_normal(a.shape)) for n, a in x.items()}

        def loss(xx):
            o, S = fwd(xx["q"], xx["k"], xx["v"], xx["la"], xx["beta"], xx["S0"], beta_v=xx["bv"], **kw)
            return float(np.sum(Wo * o) + np.sum(WS * S))

        for which in [[n] for n in x if x[n] is not None] + [[n for n in x if x[n] is not None]]:
            h = 1e-5
            xp = {n: (a if a is None else (a + h * dirs[n] if n in which else a)) for n, a in x.items()}
            xm = {n: (a if a is None else (a - h * dirs[n] if n in which else a)) for n, a in x.items()}
            fd = (loss(xp) - loss(xm)) / (2 * h)
            an = sum(float(np.sum(grads[n] * dirs[n])) for n in which)
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), \
                f"(kv, {gate}) d/d{'+'.join(which)}: analytic {an:.10e} vs difference {fd:.10e}"


def pin_bwd_kv_equal_strengths(fwd, bwd):
    """beta^v = beta^k is the one-strength rule: the gradients of q, k, v, log
    alpha and S0 are those of the one-strength backward, and dbeta^k + dbeta^v
    is its dbeta."""
    for n, gate in enumerate(("scalar", "channel")):
        q, k, v, la, beta, S0, Wo, WS = _bwd_case(280 + n, gate, "channel")
        kw = dict(gate=gate, beta_mode="channel")
        g2 = bwd(q, k, v, la, beta, S0, Wo, WS, beta_v=beta, **kw)
        g1 = bwd(q, k, v, la, beta, S0, Wo, WS, beta_v=None, **kw)
        for name in ("dq", "dk", "dv", "dlog_alpha", "dS0"):
            _close(g2[name], g1[name], 1e-12, f"kv {gate} {name}")
        _close(g2["dbeta"] + g2["dbeta_v"], g1["dbeta"], 1e-12, f"kv {gate} dbeta")


BWD_KV_PINS = [pin_bwd_kv_directional_derivatives, pin_bwd_kv_equal_strengths]


# Backward with write-side key scales and the input preparation.  Each pin
# takes fwd_ex(q, k, v, la, beta, beta_v, ks, S0, *, gate, beta_mode,
# qk_l2norm, beta_logit) -> (o, S_final) and bwd_ex(q, k, v, la, beta, beta_v,
# ks, S0, dO, dS_final, *, gate, beta_mode, qk_l2norm, beta_logit) -> dict
# (with dbeta_v when beta_v is given, dkey_scale when ks is).

def _bwd_ex_case(salt, gate, beta_mode, *, logits, ks, sepv, L=7, Dk=5, Dv=5):
    q, k, v, la, beta, S0, Wo, WS = _bwd_case(salt, gate, beta_mode, L=L, Dk=Dk, Dv=Dv)
    r = _rng(salt + 4000)
    q = q * r.uniform(0.5, 3.0, q.shape[:-1] + (1,))      # raw rows, not unit vectors
    k = k * r.uniform(0.5, 3.0, k.shape[:-1] + (1,))
    if logits:
        beta = r.standard_normal(beta.shape)
    bv = None
    if sepv:
        bv = r.standard_normal(beta.shape) if logits else 0.2 + 0.7 * r.uniform(0.0, 1.0, beta.shape)
    s = r.uniform(0.5, 1.5, q.shape) if ks else None
    return q, k, v, la, beta, bv, s, S0, Wo, WS


def pin_bwd_ex_directional_derivatives(fwd_ex, bwd_ex):
    """With key scales and/or the input preparation (raw q, k; strength
    logits): for <Wo, o> + <WS, S_final>, the gradients' inner product with
    random directions (each input alone, the key scales and the write strength
    included, then all at once) equals the central difference of the loss."""
    salt = 320
    cases = [("scalar", "scalar", True, False, False), ("channel", "channel", True, False, False),
             ("none", "scalar", False, True, False), ("channel", "scalar", False, True, False),
             ("scalar", "channel", True, True, True), ("channel", "channel", True, True, True),
             ("scalar", "scalar", True, True, True)]
    for gate, beta_mode, prep, ks, sepv in cases:
        salt += 1
        q, k, v, la, beta, bv, s, S0, Wo, WS = _bwd_ex_case(salt, gate, beta_mode, logits=prep, ks=ks, sepv=sepv)
        kw = dict(gate=gate, beta_mode=beta_mode, qk_l2norm=prep, beta_logit=prep)
        g = bwd_ex(q, k, v, la, beta, bv, s, S0, Wo, WS, **kw)
        x = dict(q=q, k=k, v=v, la=la, beta=beta, bv=bv, s=s, S0=S0)
        grads = dict(q=g["dq"], k=g["dk"], v=g["dv"], la=g["dlog_alpha"], beta=g["dbeta"], bv=g.get("dbeta_v"),
                     s=g.get("dkey_scale"), S0=g["dS0"])
        r = _rng(salt + 2000)
        dirs = {n: (None if a is None else r.standard_normal(a.shape)) for n, a in x.items()}

        def loss(xx):
            o, S = fwd_ex(xx["q"], xx["k"], xx["v"], xx["la"], xx["beta"], xx["bv"], xx["s"], xx["S0"], **kw)
            return float(np.sum(Wo * o) + np.sum(WS * S))

        live = [n for n in x if x[n] is not None]
        for which in [[n] for n in live] + [live]:
            h = 1e-5
            xp = {n: (a if a is None else (a + h * dirs[n] if n in which else a)) for n, a in x.items()}
            xm = {n: (a if a is None else (a - h * dirs[n] if n in which else a)) for n, a in x.items()}
            fd = (loss(xp) - loss(xm)) / (2 * h)
            an = sum(float(np.sum(grads[n] * dirs[n])) for n in which)
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), \
                f"(ex {gate},{beta_mode},prep={prep},ks={ks}) d/d{'+'.join(which)}: analytic {an:.10e} " \
                f"vs difference {fd:.10e}"


def pin_bwd_ex_normalisation_is_scale_free(fwd_ex, bwd_ex):
    """With q and k normalised, the loss does not change when q_t or k_t is
    scaled by a positive factor, so the gradient of each row is orthogonal to
    the row itself: sum_c dq_tc q_tc = 0 and sum_c dk_tc k_tc = 0 for every t."""
    for n, (gate, beta_mode) in enumerate((("scalar", "scalar"), ("channel", "channel"))):
        q, k, v, la, beta, bv, s, S0, Wo, WS = _bwd_ex_case(340 + n, gate, beta_mode, logits=True, ks=True,
                                                             sepv=False)
        g = bwd_ex(q, k, v, la, beta, bv, s, S0, Wo, WS, gate=gate, beta_mode=beta_mode, qk_l2norm=True,
                   beta_logit=True)
        scale = np.abs(g["dq"]).max() * np.abs(q).max()
        assert np.abs(np.sum(g["dq"] * q, axis=-1)).max() <= 1e-12 * scale, "dq not orthogonal to q"
        assert np.abs(np.sum(g["dk"] * k, axis=-1)).max() <= 1e-12 * np.abs(g["dk"]).max() * np.abs(k).max(), \
            "dk not orthogonal to k"


def pin_bwd_ex_off_is_the_plain_backward(fwd_ex, bwd_ex):
    """Unit key scales and no input preparation: the gradients of q, k, v,
    log alpha, beta and S0 are those of the plain backward (whose own pins fix
    it), and with the input preparation on already-normalised rows and
    strengths given as logits x, dbeta_x = dbeta sigmoid(x) (1 - sigmoid(x))
    while the row gradients lose their radial part only."""
    import oracle
    for n, (gate, beta_mode) in enumerate((("scalar", "scalar"), ("channel", "channel"), ("none", "scalar"))):
        q, k, v, la, beta, S0, Wo, WS = _bwd_case(350 + n, gate, beta_mode)
        kw = dict(gate=gate, beta_mode=beta_mode)
        ref = oracle.backward(q, k, v, la, beta, S0, Wo, WS, **kw)
        g = bwd_ex(q, k, v, la, beta, None, np.ones_like(q), S0, Wo, WS, qk_l2norm=False, beta_logit=False, **kw)
        for name in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"):
            if ref[name] is None:
                assert g[name] is None, name
                continue
            _close(g[name], ref[name], 1e-12, f"unit scales {gate} {name}")
        # rows already unit vectors, strengths as logits
        qu = q / np.linalg.norm(q, axis=-1, keepdims=True)
        ku = k / np.linalg.norm(k, axis=-1, keepdims=True)
        x = np.log(beta / (1.0 - beta))
        ref = oracle.backward(qu, ku, v, la, beta, S0, Wo, WS, **kw)
        g = bwd_ex(qu, ku, v, la, x, None, None, S0, Wo, WS, qk_l2norm=True, beta_logit=True, **kw)
        _close(g["dbeta"], ref["dbeta"] * beta * (1.0 - beta), 1e-10, f"logit {gate} dbeta")
        for name, rows in (("dq", qu), ("dk", ku)):
            radial = np.sum(ref[name] * rows, axis=-1, keepdims=True) * rows
            _close(g[name], ref[name] - radial, 1e-10, f"normalised {gate} {name}")
        for name in ("dv", "dlog_alpha", "dS0"):
            if ref[name] is not None:
                _close(g[name], ref[name], 1e-10, f"normalised {gate} {name}")


BWD_EX_PINS = [pin_bwd_ex_directional_derivatives, pin_bwd_ex_normalisation_is_scale_free,
               pin_bwd_ex_off_is_the_plain_backward]
