"""HIP path vs the fp64 oracle, element by element, on seeded inputs.

Every call goes through the C ABI (ctypes binding) into libdeltarule.so.
Bounds (max|x - y| / max|y|, per output tensor): 1e-4 for fp32 inputs,
3e-3 for bf16 inputs with an fp32 state.
"""
import numpy as np
import pytest

import oracle

from delta_rule_linear_amd import inputs
from gpu_common import TOL, announce, per_head_errors, rel_err, run_hip, run_oracle, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_linear_amd as drl
    drl.lib()


def _check(p, out_dtype=None, tol=None):
    announce(p.name, p.B, p.H, p.L, p.Dk, p.Dv, p.in_dtype, p.gate, p.beta_mode)
    o, S = run_hip(p, out_dtype=out_dtype)
    torch.cuda.synchronize()
    oy, Sy = run_oracle(p)
    tol = TOL[p.in_dtype] if tol is None else tol
    eo, es = rel_err(to_np(o), oy), rel_err(to_np(S), Sy)
    assert eo <= tol and es <= tol, f"{p.name}: o err {eo:.2e}, S err {es:.2e} (tol {tol:.0e})"
    return eo, es


MODES = [("none", "scalar"), ("scalar", "scalar"), ("scalar", "channel"), ("channel", "scalar"),
         ("channel", "channel")]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gate,beta_mode", MODES)
@pytest.mark.parametrize("L", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("D", [64, 128])
def test_small_sweep(dtype, gate, beta_mode, L, D):
    rng = (-0.2, -0.0005) if gate == "channel" else (-0.1, -0.001)
    p = inputs.make_chunk_problem(1, 2, L, D, D, in_dtype=dtype, gate=gate, beta_mode=beta_mode,
                                  log_alpha_range=rng, s0_var=0.01, seed=L + D,
                                  name=f"sweep-{dtype}-{gate}-{beta_mode}-L{L}-D{D}")
    # fp32 inputs run on two-term fp16 splits, whose arithmetic reaches ~1e-6:
    # hold them to 1e-5 (ten times inside the 1e-4 contract) so that a lost
    # low term anywhere shows up
    _check(p, tol=1e-5 if dtype == "f32" else None)


@pytest.mark.parametrize("Dv", [16, 48, 256])
def test_value_width(Dv):
    p = inputs.make_chunk_problem(2, 3, 130, 128, Dv, gate="scalar", s0_var=0.01, seed=3,
                                  name=f"dv{Dv}")
    _check(p)


def test_bf16_output():
    p = inputs.make_chunk_problem(1, 4, 300, 128, 128, gate="scalar", s0_var=0.01, seed=4,
                                  name="bf16-out")
    # rounding o to bf16 adds up to 2^-9 relative to each element
    _check(p, out_dtype=torch.bfloat16, tol=TOL["bf16"] + 2 ** -9)


def test_many_heads_grid_mapping():
    # nseq not a multiple of 8 exercises the sequence-to-XCD remapping tail
    p = inputs.make_chunk_problem(3, 5, 100, 64, 64, gate="scalar", s0_var=0.01, seed=5,
                                  name="b3h5")
    _check(p)


def test_strong_channel_gate_exact_path():
    # per-token log alpha down to -3: in-block decay exceeds the fp16 factor
    # range, so diagonal blocks take the exact path
    p = inputs.make_chunk_problem(1, 2, 128, 128, 128, gate="channel", beta_mode="scalar",
                                  log_alpha_range=(-3.0, -0.5), seed=6, name="strong-gate")
    _check(p)


@pytest.mark.parametrize("beta_mode", ["scalar", "channel"])
@pytest.mark.parametrize("D", [64, 128])
def test_channel_prep_loop_uneven_jobs(beta_mode, D):
    # channel-gate preparation runs a persistent loop over chunks with the next
    # chunk's inputs loaded ahead: 5 x 61 = 305 chunks on a grid of one
    # workgroup per compute unit, so some workgroups take two chunks and others
    # one, and the last chunk of each sequence is ragged
    p = inputs.make_chunk_problem(1, 5, 64 * 60 + 17, D, D, gate="channel", beta_mode=beta_mode,
                                  log_alpha_range=(-0.2, -0.0005), s0_var=0.01, seed=9,
                                  name=f"cg-loop-{beta_mode}-D{D}")
    _check(p)


def test_very_strong_scalar_gate():
    p = inputs.make_chunk_problem(1, 2, 128, 64, 64, gate="scalar", log_alpha_range=(-20.0, -5.0),
                                  s0_var=0.01, seed=7, name="very-strong-scalar")
    _check(p)


# ------------------------------------------------ magnitudes of v and S0
# The matrix-core operands derived from v and the state (R = V - gamma K S,
# U, and with a channel gate or beta the state and the gated operands) are
# fp16 terms: finite up to 65504, normal down to 2^-14.  The range below is the
# one the header states: v and S0 scaled by 2^e (exactly, a power of two)
# keep the parity bound for e in [-12, 13] with bf16 inputs and [-8, 13] with
# fp32 inputs; the run is homogeneous in (v, S0), so the oracle is simply
# rerun on the scaled values.

SCALE_EDGES = {"bf16": (-12, 13), "f32": (-8, 13)}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gate,beta_mode", MODES)
def test_value_and_state_magnitude_range(dtype, gate, beta_mode):
    rng = (-0.2, -0.0005) if gate == "channel" else (-0.1, -0.001)
    for e in SCALE_EDGES[dtype]:
        p = inputs.make_chunk_problem(1, 2, 200, 128, 128, in_dtype=dtype, gate=gate, beta_mode=beta_mode,
                                      log_alpha_range=rng, s0_var=0.01, seed=3,
                                      name=f"scale-2^{e}-{dtype}-{gate}-{beta_mode}")
        p.v = (p.v * np.float32(2.0 ** e)).astype(np.float32)
        p.S0 = (p.S0 * np.float32(2.0 ** e)).astype(np.float32)
        _check(p)
    # beyond the fp16 range the overflow shows: the output is not finite
    p = inputs.make_chunk_problem(1, 2, 200, 128, 128, in_dtype=dtype, gate=gate, beta_mode=beta_mode,
                                  log_alpha_range=rng, s0_var=0.01, seed=3)
    p.v = (p.v * np.float32(2.0 ** 16)).astype(np.float32)
    p.S0 = (p.S0 * np.float32(2.0 ** 16)).astype(np.float32)
    announce("scale 2^16", dtype, gate, beta_mode)
    o, S = run_hip(p)
    assert not (torch.isfinite(o).all().item() and torch.isfinite(S).all().item())


# ------------------------------------- separate erase and write strengths

@pytest.mark.parametrize("beta_mode", ["channel", "scalar"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("L", [1, 65, 200])
@pytest.mark.parametrize("D", [64, 128])
def test_kv_small_sweep(dtype, gate, L, D, beta_mode):
    # separate erase and write strengths, d_k-vectors or one scalar each per token
    rng = (-0.2, -0.0005) if gate == "channel" else (-0.1, -0.001)
    p = inputs.make_chunk_problem(1, 2, L, D, D, in_dtype=dtype, gate=gate, beta_mode=beta_mode,
                                  log_alpha_range=rng, s0_var=0.01, seed=L + D + 1, beta_v=True,
                                  name=f"kv-{beta_mode}-{dtype}-{gate}-L{L}-D{D}")
    _check(p, tol=1e-5 if dtype == "f32" else None)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_kv_scalar_strengths_uneven_jobs_and_input_prep(gate):
    # scalar separate strengths on the persistent channel-gate loop with a
    # ragged tail, and with raw q, k and strength logits
    for raw in (False, True):
        p = inputs.make_chunk_problem(1, 5, 64 * 60 + 17, 128, 128, gate=gate, beta_mode="scalar",
                                      log_alpha_range=(-0.2, -0.0005), s0_var=0.01, seed=23, beta_v=True,
                                      raw_inputs=raw, name=f"kv-scalar-loop-{gate}-raw{int(raw)}")
        _check(p)


def test_kv_scalar_equal_strengths_match_single_strength():
    # beta_v == beta_k (scalar) through the separate-strength entry point (the
    # channel-beta kernels) agrees with dr_chunk_fwd (the scalar-beta kernels)
    import delta_rule_linear_amd as drl
    from gpu_common import problem_to_dev
    for gate in ("scalar", "channel"):
        p = inputs.make_chunk_problem(1, 3, 300, 128, 128, gate=gate, beta_mode="scalar",
                                      log_alpha_range=(-0.2, -0.0005), s0_var=0.01, seed=24)
        announce("kv scalar equal strengths", gate)
        t = problem_to_dev(p)
        o1, S1 = drl.dr_chunk_fwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["S0"], gate=gate,
                                  beta_mode="scalar")
        o2, S2 = drl.dr_chunk_fwd_kv(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["beta"].clone(),
                                     t["S0"], gate=gate, beta_mode="scalar")
        assert rel_err(to_np(o2), to_np(o1)) <= 2e-3 and rel_err(to_np(S2), to_np(S1)) <= 2e-3


def test_kv_channel_prep_loop_uneven_jobs():
    p = inputs.make_chunk_problem(1, 5, 64 * 60 + 17, 128, 128, gate="channel", beta_mode="channel",
                                  log_alpha_range=(-0.2, -0.0005), s0_var=0.01, seed=10, beta_v=True,
                                  name="kv-cg-loop")
    _check(p)


def test_kv_equal_strengths_match_single_strength_bits():
    # beta_v == beta_k through the separate-strength entry point gives the
    # single-strength result bit for bit (same kernels, same operands)
    import delta_rule_linear_amd as drl
    from gpu_common import problem_to_dev
    for gate in ("scalar", "channel"):
        p = inputs.make_chunk_problem(1, 3, 300, 128, 128, gate=gate, beta_mode="channel",
                                      log_alpha_range=(-0.2, -0.0005), s0_var=0.01, seed=11)
        announce("kv equal strengths", gate)
        t = problem_to_dev(p)
        o1, S1 = drl.dr_chunk_fwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["S0"],
                                  gate=gate, beta_mode="channel")
        bv = t["beta"].clone()
        o2, S2 = drl.dr_chunk_fwd_kv(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], bv, t["S0"],
                                     gate=gate)
        assert torch.equal(o1, o2) and torch.equal(S1, S2)


# ------------------------------------------- input preparation in the kernels

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gate,beta_mode", MODES)
@pytest.mark.parametrize("L", [65, 200])
@pytest.mark.parametrize("D", [64, 128])
def test_input_prep_sweep(dtype, gate, beta_mode, L, D):
    # raw q, k (norms near sqrt(D)) and strength logits; the kernels normalise
    # and apply the sigmoid
    rng = (-0.2, -0.0005) if gate == "channel" else (-0.1, -0.001)
    p = inputs.make_chunk_problem(1, 2, L, D, D, in_dtype=dtype, gate=gate, beta_mode=beta_mode,
                                  log_alpha_range=rng, s0_var=0.01, seed=L + D + 2, raw_inputs=True,
                                  name=f"prep-{dtype}-{gate}-{beta_mode}-L{L}-D{D}")
    _check(p, tol=1e-5 if dtype == "f32" else None)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_input_prep_separate_strengths(gate):
    p = inputs.make_chunk_problem(1, 3, 200, 128, 128, gate=gate, beta_mode="channel",
                                  log_alpha_range=(-0.2, -0.0005), s0_var=0.01, seed=13, beta_v=True,
                                  raw_inputs=True, name=f"prep-kv-{gate}")
    _check(p)


@pytest.mark.parametrize("gate,beta_mode", MODES)
def test_input_prep_zero_vectors(gate, beta_mode):
    # a zero key writes and erases nothing, a zero query reads nothing
    p = inputs.make_chunk_problem(1, 2, 130, 128, 128, gate=gate, beta_mode=beta_mode,
                                  log_alpha_range=(-0.2, -0.0005), s0_var=0.01, seed=14,
                                  raw_inputs=True, name=f"prep-zero-{gate}-{beta_mode}")
    p.k[:, :, [5, 64, 129]] = 0
    p.q[:, :, [7, 63, 100]] = 0
    _check(p)
    o, _ = run_hip(p)
    assert torch.isfinite(o).all().item()
    assert to_np(o[:, :, [7, 63, 100]]).max() == 0.0


@pytest.mark.timeout(600)
def test_input_prep_full_headline_every_head():
    # the headline batch drawn raw: the normalisation and the sigmoid in the
    # kernels; every head recomputed by the oracle
    p = inputs.workload("gdn_b2h16_16k", raw_inputs=True)
    announce("full raw", p.name)
    o, S = run_hip(p)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(S).all().item()
    og, Sg = to_np(o), to_np(S)
    del o, S
    oy, Sy = run_oracle(p)
    eo, es = per_head_errors(og, oy), per_head_errors(Sg, Sy)
    print(f"raw headline, {p.B * p.H} heads: worst o {eo.max():.2e}, worst S {es.max():.2e}")
    assert eo.max() <= TOL["bf16"] and es.max() <= TOL["bf16"]


# ------------------------------- write-side key scales (diagonal preconditioner)

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gate,beta_mode", MODES)
@pytest.mark.parametrize("L", [65, 200])
@pytest.mark.parametrize("D", [64, 128])
def test_precond_sweep(dtype, gate, beta_mode, L, D):
    rng = (-0.2, -0.0005) if gate == "channel" else (-0.1, -0.001)
    p = inputs.make_chunk_problem(1, 2, L, D, D, in_dtype=dtype, gate=gate, beta_mode=beta_mode,
                                  log_alpha_range=rng, s0_var=0.01, seed=L + D + 3, key_scale=True,
                                  name=f"precond-{dtype}-{gate}-{beta_mode}-L{L}-D{D}")
    _check(p, tol=1e-5 if dtype == "f32" else None)


@pytest.mark.parametrize("gate,beta_mode", [("scalar", "scalar"), ("channel", "channel")])
def test_precond_with_input_prep_and_uneven_jobs(gate, beta_mode):
    # raw inputs and logits, and the persistent preparation loop with a ragged tail
    p = inputs.make_chunk_problem(1, 5, 64 * 60 + 17, 128, 128, gate=gate, beta_mode=beta_mode,
                                  log_alpha_range=(-0.2, -0.0005), s0_var=0.01, seed=16,
                                  raw_inputs=True, key_scale=True, name=f"precond-prep-{gate}")
    _check(p)


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("Dv", [48, 256])
def test_precond_and_channel_gate_value_widths(gate, Dv):
    # d_v != d_k on the channel-gate kernels (key scales, and KDA-style gates)
    for ks in (True, False):
        if gate != "channel" and not ks:
            continue
        p = inputs.make_chunk_problem(1, 3, 130, 128, Dv, gate=gate, beta_mode="scalar",
                                      log_alpha_range=(-0.2, -0.0005), s0_var=0.01, seed=19, key_scale=ks,
                                      name=f"width-{gate}-dv{Dv}-ks{int(ks)}")
        _check(p)


def test_precond_bf16_output():
    p = inputs.make_chunk_problem(1, 3, 200, 128, 128, gate="scalar", beta_mode="scalar",
                                  log_alpha_range=(-0.1, -0.001), s0_var=0.01, seed=20, key_scale=True,
                                  name="precond-bf16-out")
    _check(p, out_dtype=torch.bfloat16, tol=TOL["bf16"] + 2 ** -9)


def test_precond_strong_gate_exact_path():
    p = inputs.make_chunk_problem(1, 2, 128, 128, 128, gate="channel", beta_mode="scalar",
                                  log_alpha_range=(-3.0, -0.5), seed=17, key_scale=True,
                                  name="precond-strong-gate")
    _check(p)


@pytest.mark.parametrize("gate,beta_mode", MODES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_precond(gate, beta_mode, dtype):
    import delta_rule_linear_amd as drl
    import oracle
    from gpu_common import to_dev
    rng = (-0.2, -0.0005) if gate == "channel" else (-0.1, -0.001)
    dp = inputs.make_decode_problem(5, 3, 128, 128, 4, in_dtype=dtype, gate=gate, beta_mode=beta_mode,
                                    log_alpha_range=rng, seed=18, key_scale=True)
    announce("decode precond", gate, beta_mode, dtype)
    S = to_dev(dp.S, "f32")
    Sy = dp.S.astype(np.float64)
    for t in range(dp.steps):
        la = None if dp.log_alpha is None else dp.log_alpha[t]
        o = drl.dr_decode_step_precond(S, to_dev(dp.q[t], dtype), to_dev(dp.k[t], dtype),
                                       to_dev(dp.v[t], dtype), to_dev(la, "f32"), to_dev(dp.beta[t], "f32"),
                                       to_dev(dp.key_scale[t], "f32"), gate=gate, beta_mode=beta_mode)
        oy, Sy = oracle.decode_step(Sy, dp.q[t], dp.k[t], dp.v[t], la, dp.beta[t], gate=gate,
                                    beta_mode=beta_mode, key_scale=dp.key_scale[t])
        assert rel_err(to_np(o), oy) <= 1e-5, f"step {t} o"
    assert rel_err(to_np(S), Sy) <= 1e-5


# ---------------------------------------------------------------- full sizes

FULL = ["deltanet_f32", "gdn_b4h16_4k", "kda_b2h32_16k", "fg2_b2h16_16k", "fg2plus_b2h16_16k",
        "gdn_precond_b2h16_16k", "gdn_b2h16_16k", "gdn_b1h16_64k"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL)
def test_full_workload_every_head(name):
    """Each workload at its full size in one call; the oracle recomputes every
    (b, h) sequence and each is held to the bound on its own."""
    p = inputs.workload(name)
    announce("full", name, p.B, p.H, p.L, p.Dk, p.gate, p.beta_mode)
    o, S = run_hip(p)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(S).all().item()
    og, Sg = to_np(o), to_np(S)
    del o, S
    oy, Sy = run_oracle(p)
    tol = TOL[p.in_dtype]
    eo = per_head_errors(og, oy)
    es = per_head_errors(Sg, Sy)
    bo = np.unravel_index(np.argmax(eo), eo.shape)
    bs = np.unravel_index(np.argmax(es), es.shape)
    print(f"{name}: {p.B * p.H} heads; worst o {eo.max():.2e} at {tuple(map(int, bo))}, "
          f"worst S {es.max():.2e} at {tuple(map(int, bs))}")
    assert eo.max() <= tol and es.max() <= tol, \
        f"{name}: o {eo.max():.2e} at {bo}, S {es.max():.2e} at {bs} (tol {tol:.0e})"


# ---------------------------------------------------------------- decode

def _decode_case(N, H, D, gate, beta_mode, steps, dtype="bf16", seed=0):
    rng = (-0.2, -0.0005) if gate == "channel" else (-0.1, -0.001)
    return inputs.make_decode_problem(N, H, D, D, steps, in_dtype=dtype, gate=gate,
                                      beta_mode=beta_mode, log_alpha_range=rng, seed=seed)


@pytest.mark.parametrize("gate,beta_mode", MODES)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_steps(gate, beta_mode, D, dtype):
    import delta_rule_linear_amd as drl
    import oracle
    from gpu_common import to_dev
    dp = _decode_case(5, 3, D, gate, beta_mode, 4, dtype)
    announce("decode", gate, beta_mode, D, dtype)
    S = to_dev(dp.S, "f32")
    Sy = dp.S.astype(np.float64)
    for t in range(dp.steps):
        la = None if dp.log_alpha is None else dp.log_alpha[t]
        o = drl.dr_decode_step(S, to_dev(dp.q[t], dtype), to_dev(dp.k[t], dtype), to_dev(dp.v[t], dtype),
                               to_dev(la, "f32"), to_dev(dp.beta[t], "f32"), gate=gate,
                               beta_mode=beta_mode)
        oy, Sy = oracle.decode_step(Sy, dp.q[t], dp.k[t], dp.v[t], la, dp.beta[t], gate=gate,
                                    beta_mode=beta_mode)
        assert rel_err(to_np(o), oy) <= 1e-5, f"step {t} o"
    assert rel_err(to_np(S), Sy) <= 1e-5


@pytest.mark.timeout(900)
def test_decode_full_batch_512_steps():
    """The long-context decode workload as specified: 256 sequences x 16 heads
    of 128 x 128 fp32 states ~ N(0, 0.01), bf16 tokens, GDN gating, 512
    consecutive dr_decode_step calls on the same states.  The oracle runs the
    same 512 tokens per state as one sequence (a decode step is the forward of
    one token, started from the state); every step's o and the final states of
    all 4096 states are compared."""
    import delta_rule_linear_amd as drl
    from gpu_common import to_dev
    dp = inputs.make_decode_problem(256, 16, 128, 128, 512)
    announce("decode chain", dp.N, dp.H, dp.steps)
    S = to_dev(dp.S, "f32")
    q, k, v = to_dev(dp.q, "bf16"), to_dev(dp.k, "bf16"), to_dev(dp.v, "bf16")
    la, be = to_dev(dp.log_alpha, "f32"), to_dev(dp.beta, "f32")
    o = torch.empty((dp.steps, dp.N, dp.H, dp.Dv), dtype=torch.float32, device="cuda")
    for t in range(dp.steps):
        drl.dr_decode_step(S, q[t], k[t], v[t], la[t], be[t], gate="scalar", beta_mode="scalar", o=o[t])
    torch.cuda.synchronize()
    og, Sg = to_np(o), to_np(S)
    del q, k, v, la, be, o, S
    # tokens of each state in step order: [N, H, steps, D]
    seq = lambda a: np.ascontiguousarray(np.moveaxis(a, 0, 2))
    oy, Sy = oracle.forward(seq(dp.q), seq(dp.k), seq(dp.v), seq(dp.log_alpha), seq(dp.beta), dp.S,
                            gate="scalar", beta_mode="scalar")
    oy = np.moveaxis(oy, 2, 0)   # [steps, N, H, Dv]
    step_err = np.array([rel_err(og[t], oy[t]) for t in range(dp.steps)])
    es = rel_err(Sg, Sy)
    worst = int(np.argmax(step_err))
    print(f"decode 512 steps: worst step o {step_err.max():.2e} (step {worst}), "
          f"last step o {step_err[-1]:.2e}, final states {es:.2e}")
    assert step_err.max() <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("beta_mode", ["channel", "scalar"])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_kv_steps(gate, dtype, beta_mode):
    import delta_rule_linear_amd as drl
    import oracle
    from gpu_common import to_dev
    rng = (-0.2, -0.0005) if gate == "channel" else (-0.1, -0.001)
    dv = 128 if beta_mode == "channel" else 48   # scalar strengths allow Dv != Dk
    dp = inputs.make_decode_problem(5, 3, 128, dv, 4, in_dtype=dtype, gate=gate, beta_mode=beta_mode,
                                    log_alpha_range=rng, seed=12, beta_v=True)
    announce("decode kv", gate, dtype, beta_mode)
    S = to_dev(dp.S, "f32")
    Sy = dp.S.astype(np.float64)
    for t in range(dp.steps):
        la = None if dp.log_alpha is None else dp.log_alpha[t]
        o = drl.dr_decode_step_kv(S, to_dev(dp.q[t], dtype), to_dev(dp.k[t], dtype),
                                  to_dev(dp.v[t], dtype), to_dev(la, "f32"), to_dev(dp.beta[t], "f32"),
                                  to_dev(dp.beta_v[t], "f32"), gate=gate, beta_mode=beta_mode)
        oy, Sy = oracle.decode_step(Sy, dp.q[t], dp.k[t], dp.v[t], la, dp.beta[t], gate=gate,
                                    beta_mode=beta_mode, beta_v=dp.beta_v[t])
        assert rel_err(to_np(o), oy) <= 1e-5, f"step {t} o"
    assert rel_err(to_np(S), Sy) <= 1e-5


@pytest.mark.parametrize("gate,beta_mode", MODES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_input_prep(gate, beta_mode, dtype):
    import delta_rule_linear_amd as drl
    import oracle
    from gpu_common import to_dev
    rng = (-0.2, -0.0005) if gate == "channel" else (-0.1, -0.001)
    sepv = beta_mode == "channel"
    dp = inputs.make_decode_problem(5, 3, 128, 128, 4, in_dtype=dtype, gate=gate, beta_mode=beta_mode,
                                    log_alpha_range=rng, seed=15, beta_v=sepv, raw_inputs=True)
    announce("decode prep", gate, beta_mode, dtype)
    S = to_dev(dp.S, "f32")
    Sy = dp.S.astype(np.float64)
    for t in range(dp.steps):
        la = None if dp.log_alpha is None else dp.log_alpha[t]
        args = (S, to_dev(dp.q[t], dtype), to_dev(dp.k[t], dtype), to_dev(dp.v[t], dtype),
                to_dev(la, "f32"), to_dev(dp.beta[t], "f32"))
        if sepv:
            o = drl.dr_decode_step_kv(*args, to_dev(dp.beta_v[t], "f32"), gate=gate, qk_l2norm=True,
                                      beta_logit=True)
        else:
            o = drl.dr_decode_step(*args, gate=gate, beta_mode=beta_mode, qk_l2norm=True,
                                   beta_logit=True)
        oy, Sy = oracle.decode_step(Sy, dp.q[t], dp.k[t], dp.v[t], la, dp.beta[t], gate=gate,
                                    beta_mode=beta_mode, beta_v=None if not sepv else dp.beta_v[t],
                                    qk_l2norm=True, beta_logit=True)
        assert rel_err(to_np(o), oy) <= 1e-5, f"step {t} o"
    assert rel_err(to_np(S), Sy) <= 1e-5


# ---------------------------------------------------------------- invariants

def test_split_invariance_and_inplace_state():
    import delta_rule_linear_amd as drl
    from gpu_common import problem_to_dev
    p = inputs.make_chunk_problem(2, 3, 320, 128, 128, gate="channel", beta_mode="channel",
                                  log_alpha_range=(-0.2, -0.0005), s0_var=0.01, seed=11, name="split")
    t = problem_to_dev(p)
    announce("split invariance")
    o_full, S_full = drl.dr_chunk_fwd(**t, gate=p.gate, beta_mode=p.beta_mode)
    # split at a non-multiple of 64, carrying the state in place (S_final == S0)
    cut = 150
    sl = lambda x, s: None if x is None else x[:, :, s].contiguous()
    S = t["S0"].clone()
    o1, _ = drl.dr_chunk_fwd(sl(t["q"], slice(0, cut)), sl(t["k"], slice(0, cut)), sl(t["v"], slice(0, cut)),
                             sl(t["log_alpha"], slice(0, cut)), sl(t["beta"], slice(0, cut)), S,
                             S_final=S, gate=p.gate, beta_mode=p.beta_mode)
    o2, _ = drl.dr_chunk_fwd(sl(t["q"], slice(cut, None)), sl(t["k"], slice(cut, None)),
                             sl(t["v"], slice(cut, None)), sl(t["log_alpha"], slice(cut, None)),
                             sl(t["beta"], slice(cut, None)), S, S_final=S, gate=p.gate,
                             beta_mode=p.beta_mode)
    o_split = torch.cat([o1, o2], dim=2)
    assert rel_err(to_np(o_split), to_np(o_full)) <= 2e-3
    assert rel_err(to_np(S), to_np(S_full)) <= 2e-3


def test_prefill_then_decode_matches_longer_prefill():
    import delta_rule_linear_amd as drl
    from gpu_common import problem_to_dev
    p = inputs.make_chunk_problem(2, 4, 200, 128, 128, gate="scalar", s0_var=0.01, seed=12,
                                  name="prefill+decode")
    t = problem_to_dev(p)
    announce("prefill then decode")
    o_full, S_full = drl.dr_chunk_fwd(**t, gate="scalar", beta_mode="scalar")
    n = 5
    sl = lambda x, s: x[:, :, s].contiguous()
    _, S = drl.dr_chunk_fwd(sl(t["q"], slice(0, 200 - n)), sl(t["k"], slice(0, 200 - n)),
                            sl(t["v"], slice(0, 200 - n)), sl(t["log_alpha"], slice(0, 200 - n)),
                            sl(t["beta"], slice(0, 200 - n)), t["S0"], gate="scalar", beta_mode="scalar")
    for j in range(200 - n, 200):
        o = drl.dr_decode_step(S, t["q"][:, :, j].contiguous(), t["k"][:, :, j].contiguous(),
                               t["v"][:, :, j].contiguous(), t["log_alpha"][:, :, j].contiguous(),
                               t["beta"][:, :, j].contiguous(), gate="scalar", beta_mode="scalar")
        assert rel_err(to_np(o), to_np(o_full[:, :, j])) <= 3e-3
    assert rel_err(to_np(S), to_np(S_full)) <= 3e-3


def test_cross_mode_equivalence_on_gpu():
    import delta_rule_linear_amd as drl
    from gpu_common import problem_to_dev
    p = inputs.make_chunk_problem(1, 3, 130, 128, 128, gate="scalar", s0_var=0.01, seed=13, name="xmode")
    t = problem_to_dev(p)
    announce("cross-mode equivalence")
    o_s, S_s = drl.dr_chunk_fwd(**t, gate="scalar", beta_mode="scalar")
    lac = t["log_alpha"][..., None].expand(-1, -1, -1, 128).contiguous()
    bc = t["beta"][..., None].expand(-1, -1, -1, 128).contiguous()
    o_c, S_c = drl.dr_chunk_fwd(t["q"], t["k"], t["v"], lac, bc, t["S0"], gate="channel",
                                beta_mode="channel")
    assert rel_err(to_np(o_c), to_np(o_s)) <= 2e-3 and rel_err(to_np(S_c), to_np(S_s)) <= 2e-3
    o_n, S_n = drl.dr_chunk_fwd(t["q"], t["k"], t["v"], None, t["beta"], t["S0"], gate="none",
                                beta_mode="scalar")
    o_z, S_z = drl.dr_chunk_fwd(t["q"], t["k"], t["v"], torch.zeros_like(t["log_alpha"]), t["beta"],
                                t["S0"], gate="scalar", beta_mode="scalar")
    assert torch.equal(o_n, o_z) and torch.equal(S_n, S_z)


def test_beta_zero_is_pure_decay():
    import delta_rule_linear_amd as drl
    from gpu_common import problem_to_dev
    p = inputs.make_chunk_problem(1, 2, 100, 128, 128, gate="channel", log_alpha_range=(-0.2, -0.0005),
                                  s0_var=0.01, seed=14, name="beta0")
    t = problem_to_dev(p)
    t["beta"] = torch.zeros_like(t["beta"])
    announce("beta zero")
    o, S = drl.dr_chunk_fwd(**t, gate="channel", beta_mode="scalar")
    g = torch.cumsum(t["log_alpha"].double(), dim=2)               # [B,H,L,Dk]
    St = torch.exp(g)[..., None] * t["S0"].double()[:, :, None]    # [B,H,L,Dk,Dv]
    o_want = torch.einsum("bhlk,bhlkv->bhlv", t["q"].double(), St)
    assert rel_err(to_np(o), o_want.cpu().numpy()) <= 3e-3
    assert rel_err(to_np(S), St[:, :, -1].cpu().numpy()) <= 1e-5


def test_empty_sequence_returns_initial_state():
    import delta_rule_linear_amd as drl
    S0 = torch.randn(2, 3, 128, 64, device="cuda")
    z = lambda *s: torch.empty(*s, device="cuda", dtype=torch.bfloat16)
    o, S = drl.dr_chunk_fwd(z(2, 3, 0, 128), z(2, 3, 0, 128), z(2, 3, 0, 64),
                            torch.empty(2, 3, 0, device="cuda"), torch.empty(2, 3, 0, device="cuda"),
                            S0, gate="scalar", beta_mode="scalar")
    assert o.shape == (2, 3, 0, 64) and torch.equal(S, S0)
    o, S = drl.dr_chunk_fwd(z(2, 3, 0, 128), z(2, 3, 0, 128), z(2, 3, 0, 64),
                            torch.empty(2, 3, 0, device="cuda"), torch.empty(2, 3, 0, device="cuda"),
                            None, gate="scalar", beta_mode="scalar")
    assert torch.equal(S, torch.zeros_like(S0))


def test_deterministic_bits():
    p = inputs.make_chunk_problem(2, 4, 257, 128, 128, gate="channel", beta_mode="channel",
                                  log_alpha_range=(-0.2, -0.0005), seed=15, name="determinism")
    announce("determinism")
    o1, S1 = run_hip(p)
    o2, S2 = run_hip(p)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
