"""dr_chunk_fwd_noalloc (the library's per-GPU scratch array in place of a
workspace) against dr_chunk_fwd with a caller-owned workspace: the same
kernels on the same operands, so the results must agree bit for bit; the
oracle checks them too.  Two calls in a row, the second smaller and in other
modes, so that it runs on what the first left in the scratch array."""
import numpy as np
import pytest

from delta_rule_linear_amd import inputs
from gpu_common import TOL, announce, problem_to_dev, rel_err, run_oracle, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import delta_rule_linear_amd as drl
    drl.lib()


def _pair(p):
    import delta_rule_linear_amd as drl
    t = problem_to_dev(p)
    args = (t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["S0"])
    o_ref, S_ref = drl.dr_chunk_fwd(*args, gate=p.gate, beta_mode=p.beta_mode)
    o = torch.full_like(o_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    drl.dr_chunk_fwd_noalloc(*args, gate=p.gate, beta_mode=p.beta_mode, o=o, S_final=S)
    torch.cuda.synchronize()
    return o, S, o_ref, S_ref


def test_noalloc_matches_workspace_entry_point_twice():
    import delta_rule_linear_amd as drl
    cases = [
        inputs.make_chunk_problem(2, 16, 4096, 128, 128, gate="scalar", beta_mode="scalar",
                                  log_alpha_range=inputs.GDN_GATE, s0_var=0.01, seed=21, name="noalloc-gdn"),
        inputs.make_chunk_problem(1, 3, 300, 128, 128, gate="channel", beta_mode="channel",
                                  log_alpha_range=inputs.KDA_GATE, s0_var=0.01, seed=22, name="noalloc-fg2"),
    ]
    for p in cases:
        desc = drl.chunk_desc(p.B, p.H, p.L, p.Dk, p.Dv, drl.DR_BF16, drl.DR_F32, p.gate, p.beta_mode)
        assert drl.dr_chunk_fwd_workspace_bytes(desc) <= drl.DR_NOALLOC_SCRATCH_BYTES
        announce("noalloc", p.name, p.B, p.H, p.L, p.gate, p.beta_mode)
        o, S, o_ref, S_ref = _pair(p)
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), p.name
        heads = [(0, 0), (p.B - 1, p.H - 1)]
        for b, h in heads:
            oy, Sy = run_oracle(p.head(b, h))
            assert rel_err(to_np(o[b, h]), oy[0, 0]) <= TOL["bf16"]
            assert rel_err(to_np(S[b, h]), Sy[0, 0]) <= TOL["bf16"]


def test_noalloc_rejects_calls_beyond_the_scratch_array():
    import ctypes
    import delta_rule_linear_amd as drl
    desc = drl.chunk_desc(4, 16, 16384, 128, 128, drl.DR_BF16, drl.DR_F32, "scalar", "scalar")
    assert drl.dr_chunk_fwd_workspace_bytes(desc) > drl.DR_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(16, device="cuda")
    rc = drl.lib().dr_chunk_fwd_noalloc(ctypes.byref(desc), q.data_ptr(), q.data_ptr(), q.data_ptr(),
                                         q.data_ptr(), q.data_ptr(), None, q.data_ptr(), None, None)
    assert rc == drl.DR_ERR_WORKSPACE and "scratch array" in drl.dr_last_error()
