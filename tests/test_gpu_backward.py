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
from gpu_common import TOL, announce, problem_to_dev, rel_err, to_dev, to_np

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


def test_backward_channel_gate_full_size_sampled_sequences():
    # the KDA shape (B=2, H=32, L=16384, d=128, bf16, channel gate) in one call
    p = inputs.workload("kda_b2h32_16k")
    announce("backward full size", p.name)
    dO, dSf = inputs.backward_cotangents(p, 0)
    g = run_bwd(p, dO, dSf)
    for b, h in [(0, 0), (1, 31)]:
        s = p.head(b, h)
        ref = oracle_bwd(s, dO[b:b + 1, h:h + 1], dSf[b:b + 1, h:h + 1])
        for n in GRADS:
            x = to_np(g[n][b:b + 1, h:h + 1])
            e = rel_err(x, ref[n])
            assert e <= TOL["bf16"], f"sequence ({b},{h}) {n}: {e:.2e}"
    del g
    torch.cuda.empty_cache()


def _check_kv(p, seed=0, tol=None):
    import delta_rule_linear_amd as drl
    announce("backward kv", p.name, p.B, p.H, p.L, p.Dk, p.Dv, p.in_dtype, p.gate)
    dO, dSf = inputs.backward_cotangents(p, seed)
    t = problem_to_dev(p)
    g = drl.dr_chunk_bwd_kv(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["beta_v"], t["S0"],
                            to_dev(dO, "f32"), to_dev(dSf, "f32"), gate=p.gate)
    torch.cuda.synchronize()
    ref = oracle.backward(p.q, p.k, p.v, p.log_alpha, p.beta, p.S0, dO, dSf, gate=p.gate, beta_mode="channel",
                          beta_v=p.beta_v)
    tol = TOL[p.in_dtype] if tol is None else tol
    errs = {n: rel_err(to_np(g[n]), ref[n]) for n in GRADS + ("dbeta_v",) if ref.get(n) is not None}
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{p.name}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()) + f" (tol {tol:.0e})"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("L", [1, 65, 200])
@pytest.mark.parametrize("D", [64, 128])
def test_backward_kv_sweep(dtype, gate, L, D):
    # FG2-GDN+: separate channel-wise erase and write strengths
    rng = inputs.KDA_GATE if gate == "channel" else inputs.GDN_GATE
    p = inputs.make_chunk_problem(2, 2, L, D, D, in_dtype=dtype, gate=gate, beta_mode="channel", s0_var=0.01,
                                  seed=L + D + 11, log_alpha_range=rng, beta_v=True, name=f"bwd_kv_{gate}_{dtype}")
    _check_kv(p, seed=L + 2)


def test_backward_kv_full_size_sampled_sequences():
    import delta_rule_linear_amd as drl
    p = inputs.workload("fg2plus_b2h16_16k")
    announce("backward kv full size", p.name)
    dO, dSf = inputs.backward_cotangents(p, 0)
    t = problem_to_dev(p)
    g = drl.dr_chunk_bwd_kv(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["beta_v"], t["S0"],
                            to_dev(dO, "f32"), to_dev(dSf, "f32"), gate=p.gate)
    torch.cuda.synchronize()
    for b, h in [(0, 5), (1, 9)]:
        s = p.head(b, h)
        ref = oracle.backward(s.q, s.k, s.v, s.log_alpha, s.beta, s.S0, dO[b:b + 1, h:h + 1], dSf[b:b + 1, h:h + 1],
                              gate=s.gate, beta_mode="channel", beta_v=s.beta_v)
        for n in GRADS + ("dbeta_v",):
            if ref.get(n) is None:
                continue
            e = rel_err(to_np(g[n][b:b + 1, h:h + 1]), ref[n])
            assert e <= TOL["bf16"], f"sequence ({b},{h}) {n}: {e:.2e}"
    del g
    torch.cuda.empty_cache()


def test_backward_channel_beta_full_size_sampled_sequences():
    # the FG2-GDN shape (B=2, H=16, L=16384, d=128, bf16, channel gate and beta) in one call
    p = inputs.workload("fg2_b2h16_16k")
    announce("backward full size", p.name)
    dO, dSf = inputs.backward_cotangents(p, 0)
    g = run_bwd(p, dO, dSf)
    for b, h in [(0, 3), (1, 12)]:
        s = p.head(b, h)
        ref = oracle_bwd(s, dO[b:b + 1, h:h + 1], dSf[b:b + 1, h:h + 1])
        for n in GRADS:
            x = to_np(g[n][b:b + 1, h:h + 1])
            e = rel_err(x, ref[n])
            assert e <= TOL["bf16"], f"sequence ({b},{h}) {n}: {e:.2e}"
    del g
    torch.cuda.empty_cache()


def test_backward_full_size_sampled_sequences():
    # the benchmark's GDN shape (B=2, H=16, L=16384, d=128, bf16) in one call;
    # two sequences checked whole against the oracle run on that sequence
    p = inputs.workload("gdn_b2h16_16k")
    announce("backward full size", p.name)
    dO, dSf = inputs.backward_cotangents(p, 0)
    g = run_bwd(p, dO, dSf)
    for b, h in [(0, 0), (1, 15)]:
        s = p.head(b, h)
        ref = oracle_bwd(s, dO[b:b + 1, h:h + 1], dSf[b:b + 1, h:h + 1])
        for n in GRADS:
            x = to_np(g[n][b:b + 1, h:h + 1])
            e = rel_err(x, ref[n])
            assert e <= TOL["bf16"], f"sequence ({b},{h}) {n}: {e:.2e}"
