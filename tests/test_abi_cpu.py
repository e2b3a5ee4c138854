"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before any device work (so
these calls never touch the fake pointers they are given)."""
import ctypes
import os
import re

import pytest

import delta_rule_linear_amd as drl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "deltarule.h")

FAKE = 0x7f0000000000            # 16-byte aligned, never dereferenced
FAKE_MISALIGNED = FAKE + 8


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dr_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = drl.lib()
    declared = header_functions()
    assert set(declared) == set(drl.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_text():
    assert drl.dr_abi_version() == drl.DR_ABI_VERSION
    hdr = open(HEADER).read()
    assert re.search(r"#define DR_ABI_VERSION %d\b" % drl.DR_ABI_VERSION, hdr)
    for code in range(7):
        assert drl.dr_status_str(code).startswith("DR_")
    assert "unknown" in drl.dr_status_str(99)


def _desc(**kw):
    base = dict(B=2, H=3, L=100, Dk=128, Dv=128, in_dtype=drl.DR_BF16, out_dtype=drl.DR_F32,
                gate="scalar", beta_mode="scalar", flags=0)
    base.update(kw)
    return drl.chunk_desc(base["B"], base["H"], base["L"], base["Dk"], base["Dv"], base["in_dtype"],
                          base["out_dtype"], base["gate"], base["beta_mode"], base["flags"])


def _call(desc, q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, S0=None, o=FAKE, Sf=FAKE, ws=FAKE,
          wbytes=1 << 40):
    lib = drl.lib()
    return lib.dr_chunk_fwd(ctypes.byref(desc) if desc is not None else None, q, k, v, la, beta, S0,
                            o, Sf, ws, wbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Dk=96), drl.DR_ERR_UNSUPPORTED),
    (dict(Dk=256), drl.DR_ERR_UNSUPPORTED),
    (dict(Dv=8), drl.DR_ERR_UNSUPPORTED),
    (dict(Dv=100), drl.DR_ERR_UNSUPPORTED),
    (dict(Dv=272), drl.DR_ERR_UNSUPPORTED),
    (dict(Dv=64, beta_mode="channel"), drl.DR_ERR_UNSUPPORTED),
    (dict(L=-1), drl.DR_ERR_SHAPE),
    (dict(B=-2), drl.DR_ERR_SHAPE),
    (dict(B=70000), drl.DR_ERR_UNSUPPORTED),
])
def test_chunk_rejects_bad_descriptor(kw, code):
    assert _call(_desc(**kw)) == code
    assert drl.dr_last_error() != ""
    assert drl.dr_chunk_fwd_workspace_bytes(_desc(**kw)) == 0


def test_chunk_rejects_unknown_enums():
    d = _desc()
    d.gate = 7
    assert _call(d) == drl.DR_ERR_UNSUPPORTED
    d = _desc()
    d.in_dtype = 5
    assert _call(d) == drl.DR_ERR_UNSUPPORTED
    d = _desc()
    d.beta = 2
    assert _call(d) == drl.DR_ERR_UNSUPPORTED


def test_chunk_rejects_null_and_alignment():
    assert _call(None) == drl.DR_ERR_NULL
    assert _call(_desc(), q=None) == drl.DR_ERR_NULL
    assert _call(_desc(), o=None) == drl.DR_ERR_NULL
    assert _call(_desc(), la=None) == drl.DR_ERR_NULL              # scalar gate needs log alpha
    assert _call(_desc(gate="none")) == drl.DR_ERR_NULL             # gate none forbids it
    assert _call(_desc(), k=FAKE_MISALIGNED) == drl.DR_ERR_ALIGN
    assert _call(_desc(), S0=FAKE_MISALIGNED) == drl.DR_ERR_ALIGN
    assert "not 16-byte aligned" in drl.dr_last_error()


def test_chunk_workspace_checks():
    d = _desc()
    need = drl.dr_chunk_fwd_workspace_bytes(d)
    NC = (100 + 63) // 64
    # T^ and P (fp16 64x64 each) plus 128 floats of gate data per chunk slot
    assert need >= 2 * 3 * NC * (2 * 64 * 64 * 2 + 128 * 4)
    assert _call(d, ws=None) == drl.DR_ERR_WORKSPACE
    assert _call(d, wbytes=need - 1) == drl.DR_ERR_WORKSPACE
    # fp32 inputs carry two fp16 terms; channel modes add gated operands
    d32 = _desc(in_dtype=drl.DR_F32)
    assert drl.dr_chunk_fwd_workspace_bytes(d32) > need
    dch = _desc(gate="channel", beta_mode="channel")
    assert drl.dr_chunk_fwd_workspace_bytes(dch) > need
    assert drl.dr_chunk_fwd_workspace_bytes(_desc(L=0)) == 0
    assert drl.dr_chunk_fwd_workspace_bytes(_desc(B=0)) == 0


def test_input_flags_validation():
    d = _desc(flags=drl.DR_IN_QK_L2NORM | drl.DR_IN_BETA_LOGIT)
    assert _call(d, ws=None) == drl.DR_ERR_WORKSPACE     # known flags pass validation
    assert drl.dr_chunk_fwd_workspace_bytes(d) == drl.dr_chunk_fwd_workspace_bytes(_desc())
    d = _desc(flags=4)
    assert _call(d) == drl.DR_ERR_UNSUPPORTED
    assert "input_flags" in drl.dr_last_error()
    assert drl.dr_chunk_fwd_workspace_bytes(d) == 0
    D = drl.DecodeDesc
    ok = dict(N=4, H=2, Dk=128, Dv=128, in_dtype=drl.DR_BF16, out_dtype=drl.DR_F32, gate=1, beta=0)
    assert _dcall(D(**{**ok, "input_flags": 8})) == drl.DR_ERR_UNSUPPORTED
    assert _dcall(D(**{**ok, "input_flags": 3}), S=None) == drl.DR_ERR_NULL


def test_chunk_rejects_partial_state_overlap():
    d = _desc()
    nbytes = 2 * 3 * 128 * 128 * 4
    assert _call(d, S0=FAKE, Sf=FAKE + nbytes // 2) == drl.DR_ERR_UNSUPPORTED


def test_empty_work_needs_no_device():
    # B * H == 0: validated and done, nothing enqueued, nothing dereferenced
    assert _call(_desc(B=0), q=None, k=None, v=None, la=None, beta=None, o=None, Sf=None,
                 ws=None, wbytes=0) == drl.DR_OK


def _dcall(desc, q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, S=FAKE, o=FAKE):
    return drl.lib().dr_decode_step(ctypes.byref(desc) if desc is not None else None, q, k, v, la,
                                    beta, S, o, None)


def test_decode_validation():
    D = drl.DecodeDesc
    ok = dict(N=4, H=2, Dk=128, Dv=128, in_dtype=drl.DR_BF16, out_dtype=drl.DR_F32, gate=1, beta=0)
    assert _dcall(None) == drl.DR_ERR_NULL
    assert _dcall(D(**{**ok, "Dk": 32})) == drl.DR_ERR_UNSUPPORTED
    assert _dcall(D(**{**ok, "N": -1})) == drl.DR_ERR_SHAPE
    assert _dcall(D(**{**ok, "beta": 1, "Dv": 64})) == drl.DR_ERR_UNSUPPORTED
    assert _dcall(D(**ok), S=None) == drl.DR_ERR_NULL
    assert _dcall(D(**ok), la=None) == drl.DR_ERR_NULL
    assert _dcall(D(**ok), o=FAKE_MISALIGNED) == drl.DR_ERR_ALIGN
    assert _dcall(D(**{**ok, "N": 0})) == drl.DR_OK


def _kvcall(desc, q=FAKE, k=FAKE, v=FAKE, la=FAKE, bk=FAKE, bv=FAKE + 4096, S0=None, o=FAKE, Sf=FAKE,
            ws=FAKE, wbytes=1 << 40):
    return drl.lib().dr_chunk_fwd_kv(ctypes.byref(desc) if desc is not None else None, q, k, v, la, bk,
                                     bv, S0, o, Sf, ws, wbytes, None)


def test_chunk_kv_validation():
    ch = dict(gate="channel", beta_mode="channel")
    assert _kvcall(None) == drl.DR_ERR_NULL
    # separate strengths are channel-wise only
    assert _kvcall(_desc(gate="channel")) == drl.DR_ERR_UNSUPPORTED
    assert "DR_BETA_CHANNEL" in drl.dr_last_error()
    assert _kvcall(_desc(**ch), bv=None) == drl.DR_ERR_NULL
    assert _kvcall(_desc(**ch), bk=None) == drl.DR_ERR_NULL
    assert _kvcall(_desc(**ch), bv=FAKE_MISALIGNED) == drl.DR_ERR_ALIGN
    assert "beta_v" in drl.dr_last_error()
    assert _kvcall(_desc(**ch, Dv=64)) == drl.DR_ERR_UNSUPPORTED
    assert _kvcall(_desc(**ch), ws=None) == drl.DR_ERR_WORKSPACE
    assert _kvcall(_desc(**ch, B=0), q=None, k=None, v=None, la=None, bk=None, bv=None, o=None,
                   Sf=None, ws=None, wbytes=0) == drl.DR_OK


def test_decode_kv_validation():
    D = drl.DecodeDesc
    ok = dict(N=4, H=2, Dk=128, Dv=128, in_dtype=drl.DR_BF16, out_dtype=drl.DR_F32, gate=2, beta=1)

    def call(desc, bk=FAKE, bv=FAKE + 4096, S=FAKE):
        return drl.lib().dr_decode_step_kv(ctypes.byref(desc) if desc is not None else None, FAKE,
                                           FAKE, FAKE, FAKE, bk, bv, S, FAKE, None)

    assert call(None) == drl.DR_ERR_NULL
    assert call(D(**{**ok, "beta": 0})) == drl.DR_ERR_UNSUPPORTED
    assert call(D(**ok), bv=None) == drl.DR_ERR_NULL
    assert call(D(**ok), bv=FAKE_MISALIGNED) == drl.DR_ERR_ALIGN
    assert call(D(**{**ok, "N": 0})) == drl.DR_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(drl, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(drl, "_lib", None)
    with pytest.raises(ImportError):
        drl.lib()


def test_precond_validation_and_workspace():
    lib = drl.lib()

    def call(desc, ks=FAKE + 8192, ws=FAKE, wbytes=1 << 40):
        return lib.dr_chunk_fwd_precond(ctypes.byref(desc) if desc is not None else None, FAKE, FAKE,
                                        FAKE, FAKE, FAKE, ks, None, FAKE, FAKE, ws, wbytes, None)

    d = _desc()
    assert call(None) == drl.DR_ERR_NULL
    assert call(d, ks=None) == drl.DR_ERR_NULL
    assert "key_scale" in drl.dr_last_error()
    assert call(d, ks=FAKE_MISALIGNED) == drl.DR_ERR_ALIGN
    # the preconditioned forward runs the channel-gate kernels: more workspace
    # than the scalar-gate forward, the same as the channel-gate one
    need = drl.dr_chunk_fwd_precond_workspace_bytes(d)
    assert need > drl.dr_chunk_fwd_workspace_bytes(d)
    assert need == drl.dr_chunk_fwd_workspace_bytes(_desc(gate="channel"))
    assert call(d, wbytes=need - 1) == drl.DR_ERR_WORKSPACE
    assert drl.dr_chunk_fwd_precond_workspace_bytes(_desc(Dk=96)) == 0
    D = drl.DecodeDesc
    ok = dict(N=4, H=2, Dk=128, Dv=128, in_dtype=drl.DR_BF16, out_dtype=drl.DR_F32, gate=1, beta=0)
    dcall = lambda desc, ks=FAKE + 8192: lib.dr_decode_step_precond(
        ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, FAKE, ks, FAKE, FAKE, None)
    assert dcall(D(**ok), ks=None) == drl.DR_ERR_NULL
    assert dcall(D(**ok), ks=FAKE_MISALIGNED) == drl.DR_ERR_ALIGN
    assert dcall(D(**{**ok, "N": 0})) == drl.DR_OK


def test_backward_validation_and_workspace():
    lib = drl.lib()

    def call(desc, q=FAKE, la=FAKE, dO=FAKE, dq=FAKE, dla=FAKE, dS0=None, ws=FAKE, wbytes=1 << 40):
        return lib.dr_chunk_bwd(ctypes.byref(desc) if desc is not None else None, q, FAKE, FAKE, la, FAKE,
                                None, dO, None, dq, FAKE, FAKE, dla, FAKE, dS0, ws, wbytes, None)

    d = _desc()
    assert call(None) == drl.DR_ERR_NULL
    assert call(d, q=None) == drl.DR_ERR_NULL
    assert call(d, dO=None) == drl.DR_ERR_NULL
    assert call(d, dq=None) == drl.DR_ERR_NULL
    assert call(d, dla=None) == drl.DR_ERR_NULL                        # scalar gate: d log alpha needed
    assert call(_desc(gate="none"), la=None) == drl.DR_ERR_NULL        # no gate: none allowed
    assert call(d, dS0=FAKE_MISALIGNED) == drl.DR_ERR_ALIGN
    for bad in (dict(Dv=64, beta_mode="channel"), dict(flags=drl.DR_IN_QK_L2NORM),
                dict(out_dtype=drl.DR_BF16), dict(Dk=96)):
        assert call(_desc(**bad)) == drl.DR_ERR_UNSUPPORTED
        assert drl.dr_chunk_bwd_workspace_bytes(_desc(**bad)) == 0
    need = drl.dr_chunk_bwd_workspace_bytes(d)
    NCH = 2 * 3 * ((100 + 63) // 64)
    # per chunk: T, P, K K^T (64 x 64), 64 gate values, two states and three
    # 64 x Dv blocks, fp32
    assert need >= NCH * 4 * (3 * 64 * 64 + 64 + 2 * 128 * 128 + 3 * 64 * 128)
    assert call(d, ws=None) == drl.DR_ERR_WORKSPACE
    assert call(d, wbytes=need - 1) == drl.DR_ERR_WORKSPACE
    assert drl.dr_chunk_bwd_workspace_bytes(_desc(L=0)) == 0
    # a channel gate adds the per-channel decay and four gated operand planes
    assert drl.dr_chunk_bwd_workspace_bytes(_desc(gate="channel")) >= need + NCH * 4 * 5 * 64 * 128 - NCH * 4 * 64
    # a channel beta runs the unit-strength kernels on fp32 copies of q, sqrt(beta) k, sqrt(beta) v
    assert drl.dr_chunk_bwd_workspace_bytes(_desc(beta_mode="channel")) >= need + 3 * 2 * 3 * 100 * 128 * 4
    # no sequences: validated and done without touching memory
    assert lib.dr_chunk_bwd(ctypes.byref(_desc(B=0)), *([None] * 15), 0, None) == drl.DR_OK


def test_backward_kv_validation():
    lib = drl.lib()

    def call(desc, bv=FAKE + 4096, dbv=FAKE + 8192):
        return lib.dr_chunk_bwd_kv(ctypes.byref(desc) if desc is not None else None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   bv, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, dbv, None, FAKE, 1 << 40, None)

    assert call(_desc()) == drl.DR_ERR_UNSUPPORTED                  # separate strengths are channel-wise
    d = _desc(beta_mode="channel")
    assert call(d, bv=None) == drl.DR_ERR_NULL
    assert call(d, dbv=None) == drl.DR_ERR_NULL
    assert call(d, bv=FAKE_MISALIGNED) == drl.DR_ERR_ALIGN
    assert call(_desc(beta_mode="channel", B=0), bv=None, dbv=None) == drl.DR_OK
