"""The fp64 oracle against its pins (CPU only).  See oracle_pins.py for the
passage each pin follows."""
import numpy as np
import pytest

import oracle
import oracle_pins


def fwd(q, k, v, la, beta, S0, *, gate, beta_mode):
    return oracle.forward(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(fwd)


def test_thread_count_does_not_change_bits():
    q, k, v, la, beta, S0 = oracle_pins.random_case(7, B=3, H=5, L=20, Dk=8, Dv=8, gate="channel",
                                                    beta_mode="channel")
    a = oracle.forward(q, k, v, la, beta, S0, gate="channel", beta_mode="channel", nthreads=1)
    b = oracle.forward(q, k, v, la, beta, S0, gate="channel", beta_mode="channel", nthreads=8)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rejects_bad_arguments():
    q, k, v, la, beta, S0 = oracle_pins.random_case(8, gate="scalar", Dk=4, Dv=3)
    with pytest.raises(ValueError):       # channel beta needs d_v == d_k
        oracle.forward(q, k, v, la, np.repeat(beta[..., None], 4, -1), S0, gate="scalar",
                       beta_mode="channel")
    with pytest.raises(ValueError):       # gate none with a log alpha given
        oracle.forward(q, k, v, la, beta, S0, gate="none", beta_mode="scalar")


def test_decode_step_is_one_token_forward():
    q, k, v, la, beta, S0 = oracle_pins.random_case(9, B=3, H=2, L=1, Dk=6, Dv=5, gate="scalar")
    o1, S1 = oracle.decode_step(S0, q[:, :, 0], k[:, :, 0], v[:, :, 0], la[:, :, 0], beta[:, :, 0],
                                gate="scalar", beta_mode="scalar")
    o2, S2 = oracle.forward(q, k, v, la, beta, S0, gate="scalar", beta_mode="scalar")
    assert np.array_equal(o1, o2[:, :, 0]) and np.array_equal(S1, S2)



def fwd_kv(q, k, v, la, beta, beta_v, S0, *, gate, beta_mode):
    return oracle.forward(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode, beta_v=beta_v)


@pytest.mark.parametrize("pin", oracle_pins.KV_PINS, ids=lambda f: f.__name__)
def test_kv_pin(pin):
    pin(fwd_kv)


def test_kv_equal_strengths_is_the_single_strength_forward():
    for beta_mode in ("scalar", "channel"):
        q, k, v, la, beta, S0 = oracle_pins.random_case(33, L=10, Dk=5, Dv=5, gate="channel",
                                                        beta_mode=beta_mode)
        a = oracle.forward(q, k, v, la, beta, S0, gate="channel", beta_mode=beta_mode)
        b = oracle.forward(q, k, v, la, beta, S0, gate="channel", beta_mode=beta_mode, beta_v=beta)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_kv_decode_step_is_one_token_forward():
    q, k, v, la, beta, S0 = oracle_pins.random_case(37, B=3, H=2, L=1, Dk=6, Dv=6, gate="channel",
                                                    beta_mode="channel")
    bv = np.random.default_rng(38).uniform(0.05, 1.0, beta.shape)
    o1, S1 = oracle.decode_step(S0, q[:, :, 0], k[:, :, 0], v[:, :, 0], la[:, :, 0], beta[:, :, 0],
                                gate="channel", beta_mode="channel", beta_v=bv[:, :, 0])
    o2, S2 = oracle.forward(q, k, v, la, beta, S0, gate="channel", beta_mode="channel", beta_v=bv)
    assert np.array_equal(o1, o2[:, :, 0]) and np.array_equal(S1, S2)


def fwd_ex(q, k, v, la, beta, beta_v, S0, *, gate, beta_mode, qk_l2norm, beta_logit):
    return oracle.forward(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode, beta_v=beta_v,
                          qk_l2norm=qk_l2norm, beta_logit=beta_logit)


@pytest.mark.parametrize("pin", oracle_pins.PREP_PINS, ids=lambda f: f.__name__)
def test_input_preparation_pin(pin):
    pin(fwd_ex)


def test_input_preparation_off_is_the_plain_forward():
    q, k, v, la, beta, S0 = oracle_pins.random_case(130, L=10, Dk=5, Dv=5, gate="channel",
                                                    beta_mode="channel")
    a = oracle.forward(q, k, v, la, beta, S0, gate="channel", beta_mode="channel")
    lib = oracle._get()
    import ctypes
    dp = lambda x: np.ascontiguousarray(x, np.float64).ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    o = np.empty_like(a[0])
    Sf = np.empty_like(a[1])
    arrs = [np.ascontiguousarray(x, np.float64) for x in (q, k, v, la, beta, S0)]
    rc = lib.dro_forward_ex(1, 2, 10, 5, 5, dp(arrs[0]), dp(arrs[1]), dp(arrs[2]), dp(arrs[3]), 2,
                            dp(arrs[4]), dp(arrs[4]), 1, None, 0, dp(arrs[5]), dp(o), dp(Sf), 0)
    assert rc == 0
    assert np.array_equal(o, a[0]) and np.array_equal(Sf, a[1])


def test_input_preparation_decode_is_one_token_forward():
    q, k, v, la, beta, S0 = oracle_pins.random_case(131, B=3, H=2, L=1, Dk=6, Dv=6, gate="scalar",
                                                    beta_mode="scalar", unit_keys=False)
    kw = dict(gate="scalar", beta_mode="scalar", qk_l2norm=True, beta_logit=True)
    o1, S1 = oracle.decode_step(S0, q[:, :, 0], k[:, :, 0], v[:, :, 0], la[:, :, 0], beta[:, :, 0], **kw)
    o2, S2 = oracle.forward(q, k, v, la, beta, S0, **kw)
    assert np.array_equal(o1, o2[:, :, 0]) and np.array_equal(S1, S2)


def fwd_ks(q, k, v, la, beta, key_scale, S0, *, gate, beta_mode):
    return oracle.forward(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode, key_scale=key_scale)


@pytest.mark.parametrize("pin", oracle_pins.KS_PINS, ids=lambda f: f.__name__)
def test_key_scale_pin(pin):
    pin(fwd_ks)


def test_key_scale_decode_is_one_token_forward():
    q, k, v, la, beta, S0 = oracle_pins.random_case(140, B=3, H=2, L=1, Dk=6, Dv=6, gate="channel",
                                                    beta_mode="scalar")
    ks = np.random.default_rng(141).uniform(0.2, 2.0, q.shape)
    o1, S1 = oracle.decode_step(S0, q[:, :, 0], k[:, :, 0], v[:, :, 0], la[:, :, 0], beta[:, :, 0],
                                gate="channel", beta_mode="scalar", key_scale=ks[:, :, 0])
    o2, S2 = oracle.forward(q, k, v, la, beta, S0, gate="channel", beta_mode="scalar", key_scale=ks)
    assert np.array_equal(o1, o2[:, :, 0]) and np.array_equal(S1, S2)


def _fwd1(q, k, v, la, beta, S0, *, gate, beta_mode, lib=None):
    return oracle.forward(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode, lib=lib)


def _bwd1(q, k, v, la, beta, S0, dO, dS, *, gate, beta_mode, lib=None):
    return oracle.backward(q, k, v, la, beta, S0, dO, dS, gate=gate, beta_mode=beta_mode, lib=lib)


@pytest.mark.parametrize("pin", oracle_pins.BWD_PINS, ids=lambda f: f.__name__)
def test_backward_pin(pin):
    pin(_fwd1, _bwd1)


def _fwd_kv(q, k, v, la, beta, S0, *, gate, beta_mode, beta_v=None, lib=None):
    return oracle.forward(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode, beta_v=beta_v, lib=lib)


def _bwd_kv(q, k, v, la, beta, S0, dO, dS, *, gate, beta_mode, beta_v=None, lib=None):
    return oracle.backward(q, k, v, la, beta, S0, dO, dS, gate=gate, beta_mode=beta_mode, beta_v=beta_v, lib=lib)


@pytest.mark.parametrize("pin", oracle_pins.BWD_KV_PINS, ids=lambda f: f.__name__)
def test_backward_kv_pin(pin):
    pin(_fwd_kv, _bwd_kv)


def test_backward_without_final_state_gradient():
    q, k, v, la, beta, S0, Wo, WS = oracle_pins._bwd_case(310, "scalar", "scalar")
    a = oracle.backward(q, k, v, la, beta, S0, Wo, None, gate="scalar", beta_mode="scalar")
    b = oracle.backward(q, k, v, la, beta, S0, Wo, np.zeros_like(WS), gate="scalar", beta_mode="scalar")
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def _fwd_ex(q, k, v, la, beta, beta_v, ks, S0, *, gate, beta_mode, qk_l2norm, beta_logit, lib=None):
    return oracle.forward(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode, beta_v=beta_v, key_scale=ks,
                          qk_l2norm=qk_l2norm, beta_logit=beta_logit, lib=lib)


def _bwd_ex(q, k, v, la, beta, beta_v, ks, S0, dO, dS, *, gate, beta_mode, qk_l2norm, beta_logit, lib=None):
    return oracle.backward(q, k, v, la, beta, S0, dO, dS, gate=gate, beta_mode=beta_mode, beta_v=beta_v,
                           key_scale=ks, qk_l2norm=qk_l2norm, beta_logit=beta_logit, lib=lib)


@pytest.mark.parametrize("pin", oracle_pins.BWD_EX_PINS, ids=lambda f: f.__name__)
def test_backward_ex_pin(pin):
    pin(_fwd_ex, _bwd_ex)
