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


def F(i):
    """The i-th fake tensor address: 16-byte aligned, 64 GiB apart, so that the
    host's overlap checks see distinct arrays."""
    return FAKE + (i << 36)


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


def _call(desc, q=F(0), k=F(1), v=F(2), la=F(3), beta=F(4), S0=None, o=F(5), Sf=F(6), ws=F(7),
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
    assert _call(d, S0=F(9), Sf=F(9) + nbytes // 2) == drl.DR_ERR_UNSUPPORTED
    # the same array exactly is the in-place state carry: validation goes on
    assert _call(d, S0=F(9), Sf=F(9), ws=None) == drl.DR_ERR_WORKSPACE


@pytest.mark.parametrize("arg", ["q", "k", "v", "la", "beta", "S0", "ws"])
def test_chunk_rejects_output_overlapping_an_input(arg):
    d = _desc()
    kw = {arg: F(5) + 4096}          # inside o's 2*3*100*128*4 bytes
    if arg == "S0":
        kw["S0"] = F(5)
    assert _call(d, **kw) == drl.DR_ERR_UNSUPPORTED
    assert "o overlaps" in drl.dr_last_error()
    # S_final overlapping an input other than S0
    assert _call(d, Sf=F(1) + 256) == drl.DR_ERR_UNSUPPORTED
    assert "S_final overlaps k" in drl.dr_last_error()
    # o and S_final overlapping each other
    assert _call(d, Sf=F(5) + 1024) == drl.DR_ERR_UNSUPPORTED


def test_empty_work_needs_no_device():
    # B * H == 0: validated and done, nothing enqueued, nothing dereferenced
    assert _call(_desc(B=0), q=None, k=None, v=None, la=None, beta=None, o=None, Sf=None,
                 ws=None, wbytes=0) == drl.DR_OK


def _dcall(desc, q=F(0), k=F(1), v=F(2), la=F(3), beta=F(4), S=F(5), o=F(6)):
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
    # o must not overlap the states or an input; the states must not overlap an input
    assert _dcall(D(**ok), o=F(5) + 1024) == drl.DR_ERR_UNSUPPORTED
    assert "o overlaps S" in drl.dr_last_error()
    assert _dcall(D(**ok), o=F(0)) == drl.DR_ERR_UNSUPPORTED
    assert _dcall(D(**ok), S=F(2) + 16) == drl.DR_ERR_UNSUPPORTED


def _kvcall(desc, q=F(0), k=F(1), v=F(2), la=F(3), bk=F(4), bv=F(8), S0=None, o=F(5), Sf=F(6),
            ws=F(7), wbytes=1 << 40):
    return drl.lib().dr_chunk_fwd_kv(ctypes.byref(desc) if desc is not None else None, q, k, v, la, bk,
                                     bv, S0, o, Sf, ws, wbytes, None)


def test_chunk_kv_validation():
    ch = dict(gate="channel", beta_mode="channel")
    assert _kvcall(None) == drl.DR_ERR_NULL
    # scalar separate strengths run on the channel-beta kernels: Dv == Dk
    assert _kvcall(_desc(gate="channel"), ws=None) == drl.DR_ERR_WORKSPACE
    assert _kvcall(_desc(gate="channel", Dv=64)) == drl.DR_ERR_UNSUPPORTED
    assert "Dv == Dk" in drl.dr_last_error()
    sc = _desc(gate="scalar")
    need_kv = drl.dr_chunk_fwd_kv_workspace_bytes(sc)
    assert need_kv == drl.dr_chunk_fwd_workspace_bytes(_desc(gate="scalar", beta_mode="channel"))
    assert need_kv > drl.dr_chunk_fwd_workspace_bytes(sc)
    assert _kvcall(sc, wbytes=need_kv - 1) == drl.DR_ERR_WORKSPACE
    assert drl.dr_chunk_fwd_kv_workspace_bytes(_desc(Dv=64)) == 0
    assert drl.dr_chunk_fwd_kv_workspace_bytes(_desc(**ch)) == drl.dr_chunk_fwd_workspace_bytes(_desc(**ch))
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

    def call(desc, bk=F(4), bv=F(8), S=F(5)):
        return drl.lib().dr_decode_step_kv(ctypes.byref(desc) if desc is not None else None, F(0),
                                           F(1), F(2), F(3), bk, bv, S, F(6), None)

    assert call(None) == drl.DR_ERR_NULL
    assert call(D(**{**ok, "beta": 0, "N": 0})) == drl.DR_OK        # scalar strengths are accepted
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

    def call(desc, ks=F(10), ws=F(7), wbytes=1 << 40):
        return lib.dr_chunk_fwd_precond(ctypes.byref(desc) if desc is not None else None, F(0), F(1),
                                        F(2), F(3), F(4), ks, None, F(5), F(6), ws, wbytes, None)

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
    dcall = lambda desc, ks=F(10): lib.dr_decode_step_precond(
        ctypes.byref(desc), F(0), F(1), F(2), F(3), F(4), ks, F(5), F(6), None)
    assert dcall(D(**ok), ks=None) == drl.DR_ERR_NULL
    assert dcall(D(**ok), ks=FAKE_MISALIGNED) == drl.DR_ERR_ALIGN
    assert dcall(D(**{**ok, "N": 0})) == drl.DR_OK


def test_backward_validation_and_workspace():
    lib = drl.lib()

    def call(desc, q=F(0), la=F(3), dO=F(11), dq=F(12), dla=F(13), dS0=None, ws=F(7), wbytes=1 << 40,
             dk=F(14)):
        return lib.dr_chunk_bwd(ctypes.byref(desc) if desc is not None else None, q, F(1), F(2), la, F(4),
                                None, dO, None, dq, dk, F(15), dla, F(16), dS0, ws, wbytes, None)

    d = _desc()
    assert call(None) == drl.DR_ERR_NULL
    assert call(d, q=None) == drl.DR_ERR_NULL
    assert call(d, dO=None) == drl.DR_ERR_NULL
    assert call(d, dq=None) == drl.DR_ERR_NULL
    assert call(d, dla=None) == drl.DR_ERR_NULL                        # scalar gate: d log alpha needed
    assert call(_desc(gate="none"), la=None) == drl.DR_ERR_NULL        # no gate: none allowed
    assert call(d, dS0=FAKE_MISALIGNED) == drl.DR_ERR_ALIGN
    for bad in (dict(Dv=64, beta_mode="channel"), dict(flags=4),
                dict(out_dtype=drl.DR_BF16), dict(Dk=96)):
        assert call(_desc(**bad)) == drl.DR_ERR_UNSUPPORTED
        assert drl.dr_chunk_bwd_workspace_bytes(_desc(**bad)) == 0
    need = drl.dr_chunk_bwd_workspace_bytes(d)
    NCH = 2 * 3 * ((100 + 63) // 64)
    # per chunk: T (64 x 64), 64 gate values, two states and the 64 x Dv block
    # dU, fp32 (with fp32 inputs also P, K K^T o E, U and R)
    assert need >= NCH * 4 * (64 * 64 + 64 + 2 * 128 * 128 + 64 * 128)
    assert call(d, ws=None) == drl.DR_ERR_WORKSPACE
    assert call(d, wbytes=need - 1) == drl.DR_ERR_WORKSPACE
    assert drl.dr_chunk_bwd_workspace_bytes(_desc(L=0)) == 0
    # bf16 inputs that the kernels see as they are, without a channel gate:
    # the matrix-core operands, 21504 bytes per chunk (T^ and P^T as bf16 hi
    # and lo packed triangles, gamma and lambda), in place of the fp32 P and
    # K K^T o E planes, and no U or R (the per-chunk kernel forms them again)
    base = drl.dr_chunk_bwd_workspace_bytes(_desc(in_dtype=drl.DR_F32))
    assert need == base + NCH * 21504 - 2 * NCH * 64 * 64 * 4 - 2 * NCH * 64 * 128 * 4
    # a channel gate adds the per-channel decay and four gated operand planes
    assert drl.dr_chunk_bwd_workspace_bytes(_desc(gate="channel")) >= base + NCH * 4 * 5 * 64 * 128 - NCH * 4 * 64
    # a channel beta runs the unit-strength kernels on fp32 copies of q, sqrt(beta) k, sqrt(beta) v
    assert drl.dr_chunk_bwd_workspace_bytes(_desc(beta_mode="channel")) >= base + 3 * 2 * 3 * 100 * 128 * 4
    # the normalisation runs the kernels on fp32 copies of q, k, v and keeps
    # 1/|q|, 1/|k| per token; logits alone need only the strengths' values
    ntok = 2 * 3 * 100
    lgt = drl.dr_chunk_bwd_workspace_bytes(_desc(flags=drl.DR_IN_BETA_LOGIT))
    l2 = drl.dr_chunk_bwd_workspace_bytes(_desc(flags=drl.DR_IN_QK_L2NORM))
    assert need + ntok * 4 <= lgt < need + ntok * 128
    assert l2 >= base + 3 * ntok * 128 * 4 + 3 * ntok * 4
    assert drl.dr_chunk_bwd_workspace_bytes(_desc(flags=3)) == l2
    assert call(_desc(flags=3), wbytes=l2 - 1) == drl.DR_ERR_WORKSPACE
    # no sequences: validated and done without touching memory
    assert lib.dr_chunk_bwd(ctypes.byref(_desc(B=0)), *([None] * 15), 0, None) == drl.DR_OK
    # gradients must not overlap each other or an input
    assert call(d, dk=F(12) + 1024) == drl.DR_ERR_UNSUPPORTED
    assert "dq overlaps dk" in drl.dr_last_error()
    assert call(d, dq=F(11)) == drl.DR_ERR_UNSUPPORTED
    assert "dq overlaps dO" in drl.dr_last_error()


def test_backward_kv_validation():
    lib = drl.lib()

    def call(desc, bv=F(8), dbv=F(17)):
        return lib.dr_chunk_bwd_kv(ctypes.byref(desc) if desc is not None else None, F(0), F(1), F(2), F(3), F(4),
                                   bv, None, F(11), None, F(12), F(14), F(15), F(13), F(16), dbv, None, F(7), 1 << 40,
                                   None)

    assert call(_desc(Dv=64)) == drl.DR_ERR_UNSUPPORTED            # scalar strengths: Dv == Dk
    assert drl.dr_chunk_bwd_kv_workspace_bytes(_desc()) == \
        drl.dr_chunk_bwd_workspace_bytes(_desc(beta_mode="channel"))
    assert drl.dr_chunk_bwd_kv_workspace_bytes(_desc(Dv=64)) == 0
    d = _desc(beta_mode="channel")
    assert call(d, bv=None) == drl.DR_ERR_NULL
    assert call(d, dbv=None) == drl.DR_ERR_NULL
    assert call(d, bv=FAKE_MISALIGNED) == drl.DR_ERR_ALIGN
    assert call(_desc(beta_mode="channel", B=0), bv=None, dbv=None) == drl.DR_OK


def test_backward_precond_validation():
    lib = drl.lib()

    def call(desc, ks=F(8), dks=F(17), wbytes=1 << 40):
        return lib.dr_chunk_bwd_precond(ctypes.byref(desc) if desc is not None else None, F(0), F(1), F(2), F(3),
                                        F(4), ks, None, F(11), None, F(12), F(14), F(15), F(13), F(16), dks, None,
                                        F(7), wbytes, None)

    d = _desc()
    assert call(None) == drl.DR_ERR_NULL
    assert call(d, ks=None) == drl.DR_ERR_NULL
    assert call(d, dks=None) == drl.DR_ERR_NULL
    assert call(d, ks=FAKE_MISALIGNED) == drl.DR_ERR_ALIGN
    assert call(d, dks=F(8)) == drl.DR_ERR_UNSUPPORTED               # the scales' gradient over the scales
    assert "dkey_scale overlaps key_scale" in drl.dr_last_error()
    assert call(_desc(flags=4)) == drl.DR_ERR_UNSUPPORTED
    # every gate mode runs the channel-gate kernels: their gated planes, and with
    # a scalar gate one more fp32 plane of per-channel d log alpha
    ntok = 2 * 3 * 100
    cg = drl.dr_chunk_bwd_workspace_bytes(_desc(gate="channel"))
    sc = drl.dr_chunk_bwd_precond_workspace_bytes(_desc())
    assert drl.dr_chunk_bwd_precond_workspace_bytes(_desc(gate="channel")) == cg
    assert drl.dr_chunk_bwd_precond_workspace_bytes(_desc(gate="none")) == cg
    assert sc >= cg + ntok * 128 * 4
    assert call(d, wbytes=sc - 1) == drl.DR_ERR_WORKSPACE
    assert drl.dr_chunk_bwd_precond_workspace_bytes(_desc(L=0)) == 0
    assert lib.dr_chunk_bwd_precond(ctypes.byref(_desc(B=0)), *([None] * 17), 0, None) == drl.DR_OK


def test_noalloc_validation():
    # host-side checks of the allocation-free forward: bad descriptors, and a
    # call whose workspace exceeds the scratch array, return before any device work
    lib = drl.lib()

    def call(desc, q=F(0), o=F(5)):
        return lib.dr_chunk_fwd_noalloc(ctypes.byref(desc) if desc is not None else None, q, F(1), F(2), F(3),
                                        F(4), None, o, F(6), None)

    assert call(None) == drl.DR_ERR_NULL
    assert call(_desc(Dk=96)) == drl.DR_ERR_UNSUPPORTED
    big = _desc(B=4, H=16, L=16384)
    assert drl.dr_chunk_fwd_workspace_bytes(big) > drl.DR_NOALLOC_SCRATCH_BYTES
    assert call(big) == drl.DR_ERR_WORKSPACE
    assert "scratch array" in drl.dr_last_error()
    hdr = open(HEADER).read()
    assert re.search(r"#define DR_NOALLOC_SCRATCH_BYTES \(\(size_t\)256 << 20\)", hdr)
    assert drl.DR_NOALLOC_SCRATCH_BYTES == 256 << 20


def test_backward_least_workspace():
    # bf16, scalar gate, 16384 tokens: segments of 32 chunks keep the
    # workspace far below the one that stores every chunk's states
    d = _desc(B=2, H=16, L=16384)
    full, least = drl.dr_chunk_bwd_workspace_bytes(d), drl.dr_chunk_bwd_workspace_bytes_min(d)
    assert least < 0.6e9 < full
    nseq, NC, st = 32, 256, 128 * 128 * 4
    # the states S_c and H_c of every chunk (the larger part of the full one)
    assert full - least > 2 * nseq * (NC - 32) * st
    # no segments: 32 chunks or fewer, fp32 inputs, a channel gate or beta, the input preparation
    for kw in (dict(L=32 * 64), dict(in_dtype=drl.DR_F32), dict(gate="channel"), dict(beta_mode="channel"),
               dict(flags=drl.DR_IN_QK_L2NORM)):
        dd = _desc(**{**dict(B=2, H=16, L=16384), **kw})
        assert drl.dr_chunk_bwd_workspace_bytes_min(dd) == drl.dr_chunk_bwd_workspace_bytes(dd), kw
    assert drl.dr_chunk_bwd_workspace_bytes_min(_desc(L=0)) == 0
    assert drl.dr_chunk_bwd_workspace_bytes_min(_desc(Dk=96)) == 0
    # below the least workspace the call is rejected before any launch
    lib = drl.lib()
    args = [F(i) for i in range(14)]
    for wbytes, code in ((least - 1, drl.DR_ERR_WORKSPACE), (0, drl.DR_ERR_WORKSPACE)):
        st_ = lib.dr_chunk_bwd(ctypes.byref(d), *args[:6], *args[6:8], *args[8:13], None, F(13), wbytes, None)
        assert st_ == code
        assert "at least" in drl.dr_last_error()
