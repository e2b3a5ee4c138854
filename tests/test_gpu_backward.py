"""HIP backward (dr_chunk_bwd) vs the fp64 oracle's backward, element by
element, on seeded inputs and seeded output gradients.

Every call goes through the C ABI (ctypes binding) into libdeltarule.so.
Bounds (max|x - y| / max|y|, per gradient): 1e-4 for fp32 inputs, 3e-3 for
bf16 inputs (the backward computes in fp32 from the bf16 values either way).
"""
import numpy as np
import pytest

import oracle
from delta_rule_linear_amd import inputs
from gpu_common import TOL, announce, per_head_errors, problem_to_dev, rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GRADS = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_linear_amd as drl
    drl.lib()


def run_bwd(p, dO, dSf):
    import delta_rule_linear_amd as drl
    t = problem_to_dev(p)
    g = drl.dr_chunk_bwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["S0"], to_dev(dO, "f32"),
                         to_dev(dSf, "f32"), gate=p.gate, beta_mode=p.beta_mode)
    torch.cuda.synchronize()
    return g


def oracle_bwd(p, dO, dSf):
    return oracle.backward(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, dO, dSf, gate=p.gate,
                           beta_mode=p.beta_mode)


def _check(p, seed=0, dS_final=True, tol=None):
    announce("backward", p.name, p.B, p.H, p.L, p.Dk, p.Dv, p.in_dtype, p.gate, "dS_final" if dS_final else "")
    dO, dSf = inputs.backward_cotangents(p, seed, dS_final)
    g = run_bwd(p, dO, dSf)
    ref = oracle_bwd(p, dO, dSf)
    tol = TOL[p.in_dtype] if tol is None else tol
    errs = {}
    for n in GRADS:
        if ref[n] is None:
            assert g[n] is None, n
            continue
        errs[n] = rel_err(to_np(g[n]), ref[n])
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{p.name}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()) + f" (tol {tol:.0e})"
    return errs


def _every_sequence(name, g, ref, names):
    """Each (b, h) sequence of every gradient held to the bf16 bound on its own."""
    worst = {}
    for n in names:
        if ref.get(n) is None:
            continue
        e = per_head_errors(to_np(g[n]), ref[n])
        worst[n] = float(e.max())
        bh = np.unravel_index(np.argmax(e), e.shape)
        assert e.max() <= TOL["bf16"], f"{name} {n}: {e.max():.2e} at sequence {tuple(map(int, bh))}"
    print(f"{name}: every sequence within bounds, worst " + ", ".join(f"{n} {v:.1e}" for n, v in worst.items()))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("L", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("D", [64, 128])
def test_backward_sweep(dtype, gate, L, D):
    rng = inputs.KDA_GATE if gate == "channel" else inputs.GDN_GATE
    p = inputs.make_chunk_problem(2, 2, L, D, D, in_dtype=dtype, gate=gate, s0_var=0.01, seed=L + D,
                                  log_alpha_range=rng, name=f"bwd_{gate}_{dtype}")
    _check(p, seed=L)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("L", [1, 65, 200])
@pytest.mark.parametrize("D", [64, 128])
def test_backward_channel_beta_sweep(dtype, gate, L, D):
    # FG2-GDN: beta per channel scales k and v by its square root
    rng = inputs.KDA_GATE if gate == "channel" else inputs.GDN_GATE
    p = inputs.make_chunk_problem(2, 2, L, D, D, in_dtype=dtype, gate=gate, beta_mode="channel", s0_var=0.01,
                                  seed=L + D + 7, log_alpha_range=rng, name=f"bwd_cbeta_{gate}_{dtype}")
    _check(p, seed=L + 1)


@pytest.mark.parametrize("Dv", [16, 48, 256])
def test_backward_channel_gate_value_width(Dv):
    p = inputs.make_chunk_problem(1, 2, 130, 128, Dv, in_dtype="f32", gate="channel", s0_var=0.01, seed=Dv,
                                  log_alpha_range=inputs.KDA_GATE, name="bwd_cg_width")
    _check(p)


def test_backward_channel_gate_strong_decay():
    # log alpha down to -1 per token: within-chunk cumulative decays reach about -60
    p = inputs.make_chunk_problem(1, 2, 150, 64, 64, in_dtype="f32", gate="channel", s0_var=0.01,
                                  log_alpha_range=(-1.0, -0.05), seed=13, name="bwd_cg_strong")
    _check(p)


@pytest.mark.parametrize("mode", ["kda", "fg2", "kv", "precond_channel", "precond_scalar"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("la", [(-3.0, -0.5), (-1.6, -0.3)])
def test_backward_strong_channel_decay(la, dtype, mode):
    # log alpha in (-3, -0.5): a chunk's decay reaches about -110 in every
    # channel, past e^-G's fp32 range, so every chunk takes the shifted
    # operands; (-1.6, -0.3) puts chunks on both sides of the switch
    import delta_rule_linear_amd as drl
    bm = "channel" if mode in ("fg2", "kv") else "scalar"
    gate = "scalar" if mode == "precond_scalar" else "channel"
    p = inputs.make_chunk_problem(2, 2, 200, 128, 128, in_dtype=dtype, gate=gate, beta_mode=bm, s0_var=0.01,
                                  log_alpha_range=la, seed=53, beta_v=mode == "kv",
                                  key_scale=mode.startswith("precond"), name=f"bwd_strong_{mode}_{dtype}")
    # the first chunk's decay, below the switch at -60 in some channel
    assert p.log_alpha[:, :, :64].astype(np.float64).sum(axis=2).min() < -60
    if mode.startswith("precond"):
        _check_precond(p, seed=9)
    elif mode == "kv":
        _check_kv(p, seed=9)
    else:
        _check(p, seed=9)


@pytest.mark.parametrize("Dv", [16, 48, 256])
def test_backward_value_width(Dv):
    p = inputs.make_chunk_problem(1, 2, 130, 128, Dv, in_dtype="f32", gate="scalar", s0_var=0.01, seed=Dv,
                                  name="bwd_width")
    _check(p)


def test_backward_without_state_inputs():
    # S0 absent and dS_final absent: both read as zeros
    p = inputs.make_chunk_problem(1, 3, 150, 128, 128, in_dtype="f32", gate="scalar", seed=5,
                                  name="bwd_no_state")
    _check(p, dS_final=False)


def test_backward_many_heads_grid_mapping():
    # 9 sequences: the scans' column-tile mapping rounds up to whole groups of 8
    p = inputs.make_chunk_problem(3, 3, 100, 64, 64, in_dtype="bf16", gate="scalar", s0_var=0.01, seed=9,
                                  name="bwd_heads")
    _check(p)


def test_backward_strong_gate():
    p = inputs.make_chunk_problem(1, 2, 192, 128, 128, in_dtype="f32", gate="scalar", s0_var=0.01,
                                  log_alpha_range=(-3.0, -0.5), seed=11, name="bwd_strong_gate")
    _check(p)


def test_backward_no_tokens():
    import delta_rule_linear_amd as drl
    p = inputs.make_chunk_problem(1, 2, 0, 64, 64, in_dtype="f32", gate="scalar", s0_var=0.01, seed=3,
                                  name="bwd_empty")
    dO, dSf = inputs.backward_cotangents(p, 0)
    g = run_bwd(p, dO, dSf)
    assert g["dq"].numel() == 0
    assert np.array_equal(to_np(g["dS0"]), dSf.astype(np.float64))


@pytest.mark.timeout(900)
def test_backward_channel_gate_full_size_every_sequence():
    # the KDA shape (B=2, H=32, L=16384, d=128, bf16, channel gate) in one call
    p = inputs.workload("kda_b2h32_16k")
    announce("backward full size", p.name)
    dO, dSf = inputs.backward_cotangents(p, 0)
    g = run_bwd(p, dO, dSf)
    ref = oracle_bwd(p, dO, dSf)
    _every_sequence(p.name, g, ref, GRADS)
    del g, ref
    torch.cuda.empty_cache()


def _check_kv(p, seed=0, tol=None):
    import delta_rule_linear_amd as drl
    announce("backward kv", p.name, p.B, p.H, p.L, p.Dk, p.Dv, p.in_dtype, p.gate, p.beta_mode)
    dO, dSf = inputs.backward_cotangents(p, seed)
    t = problem_to_dev(p)
    g = drl.dr_chunk_bwd_kv(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["beta_v"], t["S0"],
                            to_dev(dO, "f32"), to_dev(dSf, "f32"), gate=p.gate, beta_mode=p.beta_mode)
    torch.cuda.synchronize()
    ref = oracle.backward(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, dO, dSf, gate=p.gate, beta_mode=p.beta_mode,
                          beta_v=p.beta_v)
    tol = TOL[p.in_dtype] if tol is None else tol
    errs = {n: rel_err(to_np(g[n]), ref[n]) for n in GRADS + ("dbeta_v",) if ref.get(n) is not None}
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{p.name}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()) + f" (tol {tol:.0e})"


@pytest.mark.parametrize("beta_mode", ["channel", "scalar"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("L", [1, 65, 200])
@pytest.mark.parametrize("D", [64, 128])
def test_backward_kv_sweep(dtype, gate, L, D, beta_mode):
    # FG2-GDN+: separate erase and write strengths, d_k-vectors or one scalar
    # each per token
    rng = inputs.KDA_GATE if gate == "channel" else inputs.GDN_GATE
    p = inputs.make_chunk_problem(2, 2, L, D, D, in_dtype=dtype, gate=gate, beta_mode=beta_mode, s0_var=0.01,
                                  seed=L + D + 11, log_alpha_range=rng, beta_v=True,
                                  name=f"bwd_kv_{beta_mode}_{gate}_{dtype}")
    _check_kv(p, seed=L + 2)


@pytest.mark.timeout(900)
def test_backward_kv_full_size_every_sequence():
    import delta_rule_linear_amd as drl
    p = inputs.workload("fg2plus_b2h16_16k")
    announce("backward kv full size", p.name)
    dO, dSf = inputs.backward_cotangents(p, 0)
    t = problem_to_dev(p)
    g = drl.dr_chunk_bwd_kv(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["beta_v"], t["S0"],
                            to_dev(dO, "f32"), to_dev(dSf, "f32"), gate=p.gate)
    torch.cuda.synchronize()
    ref = oracle.backward(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, dO, dSf, gate=p.gate, beta_mode="channel",
                          beta_v=p.beta_v)
    _every_sequence(p.name, g, ref, GRADS + ("dbeta_v",))
    del g, ref
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_backward_channel_beta_full_size_every_sequence():
    # the FG2-GDN shape (B=2, H=16, L=16384, d=128, bf16, channel gate and beta) in one call
    p = inputs.workload("fg2_b2h16_16k")
    announce("backward full size", p.name)
    dO, dSf = inputs.backward_cotangents(p, 0)
    g = run_bwd(p, dO, dSf)
    ref = oracle_bwd(p, dO, dSf)
    _every_sequence(p.name, g, ref, GRADS)
    del g, ref
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_backward_full_size_every_sequence():
    # the benchmark's GDN shape (B=2, H=16, L=16384, d=128, bf16) in one call;
    # every sequence checked whole against the oracle
    p = inputs.workload("gdn_b2h16_16k")
    announce("backward full size", p.name)
    dO, dSf = inputs.backward_cotangents(p, 0)
    g = run_bwd(p, dO, dSf)
    ref = oracle_bwd(p, dO, dSf)
    _every_sequence(p.name, g, ref, GRADS)
    del g, ref
    torch.cuda.empty_cache()



def _check_prepared(p, seed=0, tol=None):
    """The backward with the input preparation on, against the oracle's
    gradients with respect to the raw inputs (unnormalised q and k, strength
    logits)."""
    import delta_rule_linear_amd as drl
    announce("backward prepared", p.name, p.B, p.H, p.L, p.Dk, p.Dv, p.in_dtype, p.gate, p.beta_mode,
             p.qk_l2norm, p.beta_logit)
    dO, dSf = inputs.backward_cotangents(p, seed)
    t = problem_to_dev(p)
    flags = dict(qk_l2norm=p.qk_l2norm, beta_logit=p.beta_logit)
    if p.beta_v is None:
        g = drl.dr_chunk_bwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["S0"], to_dev(dO, "f32"),
                             to_dev(dSf, "f32"), gate=p.gate, beta_mode=p.beta_mode, **flags)
    else:
        g = drl.dr_chunk_bwd_kv(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["beta_v"], t["S0"],
                                to_dev(dO, "f32"), to_dev(dSf, "f32"), gate=p.gate, beta_mode=p.beta_mode,
                                **flags)
    torch.cuda.synchronize()
    ref = oracle.backward(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, dO, dSf, gate=p.gate, beta_mode=p.beta_mode,
                          beta_v=p.beta_v, **flags)
    tol = TOL[p.in_dtype] if tol is None else tol
    errs = {n: rel_err(to_np(g[n]), ref[n]) for n in GRADS + ("dbeta_v",) if ref.get(n) is not None}
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{p.name}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()) + f" (tol {tol:.0e})"


def _raw(p, qk_l2norm, beta_logit):
    """p drawn with raw_inputs=True, with one or both preparation steps on:
    a step that stays off gets its prepared values (normalised q, k; the
    strengths' sigmoid), so the forward sees the same recurrence."""
    import dataclasses

    def sig(x):
        return None if x is None else (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)

    def unit(x):
        x64 = x.astype(np.float32).astype(np.float64)
        n = np.linalg.norm(x64, axis=-1, keepdims=True)
        return inputs._to_dtype(np.where(n > 0, x64 / np.where(n > 0, n, 1), 0.0), p.in_dtype)

    upd = dict(qk_l2norm=qk_l2norm, beta_logit=beta_logit)
    if not qk_l2norm:
        upd.update(q=unit(p.q), k=unit(p.k))
    if not beta_logit:
        upd.update(beta=sig(p.beta), beta_v=sig(p.beta_v))
    return dataclasses.replace(p, **upd)


@pytest.mark.parametrize("prep", ["l2", "logit", "both"])
@pytest.mark.parametrize("beta_mode", ["scalar", "channel", "kv_scalar", "kv_channel"])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_input_preparation(prep, beta_mode, gate, dtype):
    # DeltaNet page, step list, step 2 and its notes: the gradients are those
    # of the raw q and k (through the normalisation) and of the strength
    # logits (through the sigmoid)
    kv = beta_mode.startswith("kv_")
    bm = beta_mode[3:] if kv else beta_mode
    rng = inputs.KDA_GATE if gate == "channel" else inputs.GDN_GATE
    D = 128 if dtype == "bf16" else 64
    p = inputs.make_chunk_problem(2, 2, 150, D, D, in_dtype=dtype, gate=gate, beta_mode=bm, s0_var=0.01,
                                  seed=17 + D, log_alpha_range=rng, beta_v=kv, raw_inputs=True,
                                  name=f"bwd_prep_{prep}_{beta_mode}_{gate}_{dtype}")
    p = _raw(p, prep in ("l2", "both"), prep in ("logit", "both"))
    _check_prepared(p, seed=3)


@pytest.mark.parametrize("Dv", [16, 48, 256])
def test_backward_input_preparation_value_width(Dv):
    p = inputs.make_chunk_problem(1, 2, 130, 128, Dv, in_dtype="f32", gate="scalar", s0_var=0.01, seed=Dv + 1,
                                  log_alpha_range=inputs.GDN_GATE, raw_inputs=True, name=f"bwd_prep_dv{Dv}")
    _check_prepared(p, seed=4)


def test_backward_input_preparation_zero_rows():
    # a zero q or k row normalises to zero (both sides take that reading),
    # and its gradient is zero
    p = inputs.make_chunk_problem(1, 2, 100, 64, 64, in_dtype="f32", gate="scalar", s0_var=0.01, seed=23,
                                  log_alpha_range=inputs.GDN_GATE, raw_inputs=True, name="bwd_prep_zero_rows")
    p.q[0, 0, 5] = 0
    p.k[0, 1, 70] = 0
    p.q[0, 1, 99] = 0
    p.k[0, 1, 99] = 0
    _check_prepared(p, seed=5)


@pytest.mark.timeout(900)
def test_backward_input_preparation_full_size_every_sequence():
    # the benchmark's GDN shape with raw q, k and strength logits
    import delta_rule_linear_amd as drl
    p = inputs.make_chunk_problem(2, 16, 16384, 128, 128, in_dtype="bf16", gate="scalar",
                                  log_alpha_range=inputs.GDN_GATE, s0_var=0.01, seed=0, raw_inputs=True,
                                  name="bwd_prep_gdn_b2h16_16k")
    announce("backward prepared full size", p.name)
    dO, dSf = inputs.backward_cotangents(p, 0)
    t = problem_to_dev(p)
    g = drl.dr_chunk_bwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["S0"], to_dev(dO, "f32"),
                         to_dev(dSf, "f32"), gate=p.gate, beta_mode=p.beta_mode, qk_l2norm=True, beta_logit=True)
    torch.cuda.synchronize()
    ref = oracle.backward(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, dO, dSf, gate=p.gate, beta_mode=p.beta_mode,
                          qk_l2norm=True, beta_logit=True)
    _every_sequence(p.name, g, ref, GRADS)
    del g, ref
    torch.cuda.empty_cache()


def _check_precond(p, seed=0, tol=None):
    """dr_chunk_bwd_precond against the oracle's gradients of the
    preconditioned rule, dkey_scale included."""
    import delta_rule_linear_amd as drl
    announce("backward precond", p.name, p.B, p.H, p.L, p.Dk, p.Dv, p.in_dtype, p.gate, p.beta_mode,
             p.qk_l2norm, p.beta_logit)
    dO, dSf = inputs.backward_cotangents(p, seed)
    t = problem_to_dev(p)
    flags = dict(qk_l2norm=p.qk_l2norm, beta_logit=p.beta_logit)
    g = drl.dr_chunk_bwd_precond(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["key_scale"], t["S0"],
                                 to_dev(dO, "f32"), to_dev(dSf, "f32"), gate=p.gate, beta_mode=p.beta_mode, **flags)
    torch.cuda.synchronize()
    ref = oracle.backward(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, dO, dSf, gate=p.gate, beta_mode=p.beta_mode,
                          key_scale=p.key_scale, **flags)
    tol = TOL[p.in_dtype] if tol is None else tol
    errs = {n: rel_err(to_np(g[n]), ref[n]) for n in GRADS + ("dkey_scale",) if ref.get(n) is not None}
    assert set(errs) >= {"dq", "dk", "dv", "dbeta", "dS0", "dkey_scale"}
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{p.name}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()) + f" (tol {tol:.0e})"
    return g, ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("beta_mode", ["scalar", "channel"])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("L", [1, 65, 200])
def test_backward_precond_sweep(L, gate, beta_mode, dtype):
    # OSDN page, "Method": the write-side key w = s (.) kt; every gate mode
    # runs the channel-gate kernels (a scalar or absent gate broadcast)
    rng = inputs.KDA_GATE if gate == "channel" else inputs.GDN_GATE
    D = 128 if dtype == "bf16" else 64
    p = inputs.make_chunk_problem(2, 2, L, D, D, in_dtype=dtype, gate=gate, beta_mode=beta_mode, s0_var=0.01,
                                  seed=L + D + 31, log_alpha_range=rng, key_scale=True,
                                  name=f"bwd_precond_{gate}_{beta_mode}_{dtype}")
    _check_precond(p, seed=L + 5)


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_backward_precond_input_preparation(gate):
    # raw q, k and strength logits with key scales: the normalisation and the
    # sigmoid in front of the preconditioned rule
    rng = inputs.KDA_GATE if gate == "channel" else inputs.GDN_GATE
    p = inputs.make_chunk_problem(1, 3, 150, 128, 128, in_dtype="bf16", gate=gate, s0_var=0.01, seed=41,
                                  log_alpha_range=rng, raw_inputs=True, key_scale=True,
                                  name=f"bwd_precond_prep_{gate}")
    _check_precond(p, seed=6)


def test_backward_precond_unit_scales_match_plain():
    # s = 1 is the unscaled rule: the same gradients as dr_chunk_bwd, and
    # dkey_scale = k (.) (the write key's gradient)
    import delta_rule_linear_amd as drl
    p = inputs.make_chunk_problem(1, 2, 130, 128, 128, in_dtype="bf16", gate="channel", s0_var=0.01, seed=43,
                                  log_alpha_range=inputs.KDA_GATE, key_scale=True, name="bwd_precond_unit")
    p.key_scale[:] = 1.0
    g, ref = _check_precond(p, seed=7)
    plain = run_bwd(p, *inputs.backward_cotangents(p, 7))
    for n in GRADS:
        assert rel_err(to_np(g[n]), to_np(plain[n])) <= 1e-5, n


def test_backward_precond_value_width():
    p = inputs.make_chunk_problem(1, 2, 130, 128, 48, in_dtype="f32", gate="scalar", s0_var=0.01, seed=47,
                                  log_alpha_range=inputs.GDN_GATE, key_scale=True, name="bwd_precond_dv48")
    _check_precond(p, seed=8)


@pytest.mark.timeout(900)
def test_backward_precond_full_size_every_sequence():
    # the headline GDN shape with write-side key scales U(0.5, 1.5), every sequence
    import delta_rule_linear_amd as drl
    p = inputs.workload("gdn_precond_b2h16_16k")
    announce("backward precond full size", p.name)
    dO, dSf = inputs.backward_cotangents(p, 0)
    t = problem_to_dev(p)
    g = drl.dr_chunk_bwd_precond(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["key_scale"], t["S0"],
                                 to_dev(dO, "f32"), to_dev(dSf, "f32"), gate=p.gate, beta_mode=p.beta_mode)
    torch.cuda.synchronize()
    ref = oracle.backward(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, dO, dSf, gate=p.gate, beta_mode=p.beta_mode,
                          key_scale=p.key_scale)
    _every_sequence(p.name, g, ref, GRADS + ("dkey_scale",))
    del g, ref
    torch.cuda.empty_cache()


# ------------------------------------- bounded workspace: segments of chunks

def _bwd_with_workspace(p, dO, dSf, nbytes, want_dS0=True):
    import delta_rule_linear_amd as drl
    t = problem_to_dev(p)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
    g = drl.dr_chunk_bwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["S0"], to_dev(dO, "f32"),
                         None if dSf is None else to_dev(dSf, "f32"), gate=p.gate, beta_mode=p.beta_mode,
                         want_dS0=want_dS0, workspace=ws)
    torch.cuda.synchronize()
    return g


def _same_gradients(name, g, f, what):
    for n in GRADS:
        if f[n] is None:
            assert g[n] is None, n
        else:
            assert torch.equal(g[n], f[n]), f"{name}: {n} differs ({what})"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_backward_is_deterministic(dtype, gate):
    # every sum of the backward runs in a fixed order (no float atomics), so
    # repeated calls give the same bits
    rng = inputs.KDA_GATE if gate == "channel" else inputs.GDN_GATE
    p = inputs.make_chunk_problem(2, 3, 64 * 9 + 5, 128, 128, in_dtype=dtype, gate=gate, s0_var=0.01, seed=11,
                                  log_alpha_range=rng, name=f"determinism-{dtype}-{gate}")
    announce("backward determinism", p.name)
    dO, dSf = inputs.backward_cotangents(p, 2)
    first = run_bwd(p, dO, dSf)
    for _ in range(3):
        _same_gradients(p.name, run_bwd(p, dO, dSf), first, "repeated call")


def _desc(p):
    import delta_rule_linear_amd as drl
    return drl.chunk_desc(p.B, p.H, p.L, p.Dk, p.Dv, drl.DR_BF16 if p.in_dtype == "bf16" else drl.DR_F32,
                          drl.DR_F32, p.gate, p.beta_mode, 0)


@pytest.mark.parametrize("gate", ["none", "scalar"])
@pytest.mark.parametrize("D", [64, 128])
def test_backward_segments_match_full_workspace(gate, D):
    # 76 chunks (a ragged last one): with the least workspace the call runs
    # segments of 32, 32 and 12 chunks; one byte short of the full workspace
    # gives segments of 75 and 1; in between 38 and 38.  Each segment starts
    # from a checkpoint of S and the carried state gradient, with the same
    # per-chunk arithmetic, so the gradients are bit-identical to those of
    # the call that keeps every chunk's states, and within bounds of the
    # oracle
    import delta_rule_linear_amd as drl
    p = inputs.make_chunk_problem(1, 3, 64 * 75 + 17, D, D, gate=gate, s0_var=0.01, seed=D + 5,
                                  name=f"segments-{gate}-D{D}")
    d = _desc(p)
    full, least = drl.dr_chunk_bwd_workspace_bytes(d), drl.dr_chunk_bwd_workspace_bytes_min(d)
    assert least < full
    dO, dSf = inputs.backward_cotangents(p, 1)
    announce("backward segments", p.name, full, least)
    ref_g = _bwd_with_workspace(p, dO, dSf, full)
    for nbytes in (least, full - 1, (least + full) // 2):
        g = _bwd_with_workspace(p, dO, dSf, nbytes)
        _same_gradients(p.name, g, ref_g, f"{nbytes} of {full} bytes")
    ref = oracle_bwd(p, dO, dSf)
    for n in GRADS:
        if ref[n] is not None:
            assert rel_err(to_np(g[n]), ref[n]) <= TOL["bf16"], n
    # without S0, dS_final and dS0
    p.S0 = None
    g0 = _bwd_with_workspace(p, dO, None, least, want_dS0=False)
    f0 = _bwd_with_workspace(p, dO, None, full, want_dS0=False)
    assert g0["dS0"] is None
    _same_gradients(p.name, g0, f0, "no S0, dS_final or dS0")


def test_backward_segments_full_size_every_sequence():
    # the benchmark's GDN shape with the least workspace (segments of 32
    # chunks): bit-identical to the full-workspace call, every sequence
    # within bounds of the oracle
    import delta_rule_linear_amd as drl
    p = inputs.workload("gdn_b2h16_16k")
    d = _desc(p)
    full, least = drl.dr_chunk_bwd_workspace_bytes(d), drl.dr_chunk_bwd_workspace_bytes_min(d)
    announce("backward segments full size", p.name, full, least)
    assert least < 0.6e9 < full
    dO, dSf = inputs.backward_cotangents(p, 0)
    g = _bwd_with_workspace(p, dO, dSf, least)
    f = _bwd_with_workspace(p, dO, dSf, full)
    _same_gradients(p.name, g, f, "least workspace")
    del f
    torch.cuda.empty_cache()
    ref = oracle_bwd(p, dO, dSf)
    _every_sequence(p.name, g, ref, GRADS)
    del g, ref
    torch.cuda.empty_cache()


def test_backward_workspace_below_least_is_rejected():
    import delta_rule_linear_amd as drl
    p = inputs.make_chunk_problem(1, 1, 64 * 40, 64, 64, gate="scalar", seed=2, name="segments-too-small")
    least = drl.dr_chunk_bwd_workspace_bytes_min(_desc(p))
    dO, dSf = inputs.backward_cotangents(p, 1)
    with pytest.raises(RuntimeError, match="at least"):
        _bwd_with_workspace(p, dO, dSf, least - 256)
