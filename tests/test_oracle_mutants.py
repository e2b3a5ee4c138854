"""Plant plausible mistakes in copies of the oracle's C source and check that
the pin suite catches every one of them (CPU only).  The mistakes are planted
in temporary copies; the committed oracle is never modified."""
import os

import numpy as np
import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "dr_oracle.c")

# (name, original text, planted text): each original must occur exactly once.
MUTANTS = [
    ("drop_decay", "row[j] *= a;", "row[j] *= 1.0;"),
    ("sign_of_error", "row[j] += w * (vt[j] - p[j]);", "row[j] += w * (vt[j] + p[j]);"),
    ("beta_not_sqrt", "kt[c] = sqrt(strength(b, logit)) * (kn * k_t[c]);",
     "kt[c] = strength(b, logit) * (kn * k_t[c]);"),
    ("value_unscaled", "vt[j] = sqrt(strength(b, logit)) * v_t[j];", "vt[j] = v_t[j];"),
    ("read_unscaled_key", "p[j] += row[j] * kt[c];", "p[j] += row[j] * k_t[c];"),
    ("output_from_query_free_state", "ot[j] += row[j] * (qn * qt[c]);", "ot[j] += row[j] * (qn * k_t[c]);"),
    ("gate_index_shift", "exp(la[(size_t)t * Dk + c])", "exp(la[(size_t)t * Dk + (c + 1) % Dk])"),
    ("channel_beta_wrong_channel", "betav[(size_t)t * Dk + j]", "betav[(size_t)t * Dk + (Dk - 1 - j)]"),
    ("error_drops_read", "(vt[j] - p[j])", "(vt[j] - 0.0 * p[j])"),
    ("state_not_carried", "if (S0) memcpy(S, S0", "if (0) memcpy(S, S0"),
    ("output_before_update",
     "/* S_t = S' + w (vt - p)^T, the write-side key w = s (.) kt */",
     "for (int j = 0; j < Dv; ++j) { double a_ = 0; for (int c = 0; c < Dk; ++c) a_ += S[(size_t)c * Dv + j] * qt[c]; o[(size_t)t * Dv + j] = a_; }\n        if (0)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "libmutant.so")))

    def fwd(q, k, v, la, beta, S0, *, gate, beta_mode):
        return oracle.forward(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode, lib=lib)

    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(fwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"


# Mistakes in the separate write strength, caught by the pins of that reading.
KV_MUTANTS = [
    ("value_uses_key_strength", "? betav[t] : betav[(size_t)t * Dk + j]", "? beta[t] : beta[(size_t)t * Dk + j]"),
    ("key_uses_value_strength", "? beta[t] : beta[(size_t)t * Dk + c]", "? betav[t] : betav[(size_t)t * Dk + c]"),
    ("value_strength_not_sqrt", "vt[j] = sqrt(strength(b, logit)) * v_t[j];",
     "vt[j] = strength(b, logit) * v_t[j];"),
]


@pytest.mark.parametrize("name,old,new", KV_MUTANTS, ids=[m[0] for m in KV_MUTANTS])
def test_kv_pins_catch_planted_mistake(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "libmutant.so")))

    def fwd_kv(q, k, v, la, beta, beta_v, S0, *, gate, beta_mode):
        return oracle.forward(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode, lib=lib,
                              beta_v=beta_v)

    caught = []
    for pin in oracle_pins.KV_PINS:
        try:
            pin(fwd_kv)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"


# Mistakes in the input preparation, caught by its pins.
PREP_MUTANTS = [
    ("query_not_normalised", "const double qn = l2 ? inv_l2(qt, Dk) : 1.0;", "const double qn = 1.0;"),
    ("key_by_squared_norm", "kt[c] = sqrt(strength(b, logit)) * (kn * k_t[c]);",
     "kt[c] = sqrt(strength(b, logit)) * (kn * kn * k_t[c]);"),
    ("zero_vector_not_kept", "return s > 0.0 ? 1.0 / sqrt(s) : 0.0;", "return 1.0 / sqrt(s);"),
    ("sigmoid_sign", "return logit ? 1.0 / (1.0 + exp(-x)) : x;", "return logit ? 1.0 / (1.0 + exp(x)) : x;"),
    ("value_strength_not_from_logit", "vt[j] = sqrt(strength(b, logit)) * v_t[j];", "vt[j] = sqrt(b) * v_t[j];"),
]


@pytest.mark.parametrize("name,old,new", PREP_MUTANTS, ids=[m[0] for m in PREP_MUTANTS])
def test_prep_pins_catch_planted_mistake(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "libmutant.so")))

    def fwd_ex(q, k, v, la, beta, beta_v, S0, *, gate, beta_mode, qk_l2norm, beta_logit):
        return oracle.forward(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode, lib=lib,
                              beta_v=beta_v, qk_l2norm=qk_l2norm, beta_logit=beta_logit)

    caught = []
    for pin in oracle_pins.PREP_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fwd_ex)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"


# Mistakes in the write-side key scaling, caught by its pins.
KS_MUTANTS = [
    ("write_key_unscaled", "const double w = ks ? ks[(size_t)t * Dk + c] * kt[c] : kt[c];",
     "const double w = kt[c];"),
    ("scale_squared", "const double w = ks ? ks[(size_t)t * Dk + c] * kt[c] : kt[c];",
     "const double w = ks ? ks[(size_t)t * Dk + c] * ks[(size_t)t * Dk + c] * kt[c] : kt[c];"),
    ("scale_on_the_read_side", "p[j] += row[j] * kt[c];",
     "p[j] += row[j] * (ks ? ks[(size_t)t * Dk + c] * kt[c] : kt[c]);"),
]


@pytest.mark.parametrize("name,old,new", KS_MUTANTS, ids=[m[0] for m in KS_MUTANTS])
def test_ks_pins_catch_planted_mistake(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "libmutant.so")))

    def fwd_ks(q, k, v, la, beta, key_scale, S0, *, gate, beta_mode):
        return oracle.forward(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode, lib=lib,
                              key_scale=key_scale)

    caught = []
    for pin in oracle_pins.KS_PINS:
        try:
            pin(fwd_ks)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"


# Mistakes in the backward, caught by its pins.
BWD_MUTANTS = [
    ("no_decay_on_state_gradient", "G[(size_t)c * Dv + j] = al[c] * g;", "G[(size_t)c * Dv + j] = g;"),
    ("read_term_sign", "dkt[c] = (st_ ? st_[c] : 1.0) * a - b;", "dkt[c] = (st_ ? st_[c] : 1.0) * a + b;"),
    ("output_gradient_dropped", "G[(size_t)c * Dv + j] += qh[c] * dot[j];", "G[(size_t)c * Dv + j] += 0.0 * dot[j];"),
    ("sqrt_factor_half_dropped", "double g = dkt[c] * kh[c] / (2.0 * sbk[c]);", "double g = dkt[c] * kh[c] / sbk[c];"),
    ("erase_term_dropped", "const double g = G[(size_t)c * Dv + j] - kt[c] * dvt[j];",
     "const double g = G[(size_t)c * Dv + j];"),
]


@pytest.mark.parametrize("name,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_bwd_pins_catch_planted_mistake(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "libmutant.so")))

    def fwd(q, k, v, la, beta, S0, *, gate, beta_mode):
        return oracle.forward(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode)

    def bwd(q, k, v, la, beta, S0, dO, dS, *, gate, beta_mode):
        return oracle.backward(q, k, v, la, beta, S0, dO, dS, gate=gate, beta_mode=beta_mode, lib=lib)

    caught = []
    for pin in oracle_pins.BWD_PINS:
        try:
            pin(fwd, bwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"


# The backward with a separate write strength: the value scaled by the erase
# strength, or the forward replayed with the erase strength on the value.
BWD_KV_MUTANTS = [
    ("bwd_value_scaled_by_erase_strength",
     "bvv[j] = strength(beta_mode == DRO_BETA_SCALAR ? bvs[t] : bvs[(size_t)t * Dk + j], logit);",
     "bvv[j] = strength(beta_mode == DRO_BETA_SCALAR ? bs[t] : bs[(size_t)t * Dk + j], logit);"),
    ("bwd_replay_without_write_strength",
     "bvs + (beta_mode == DRO_BETA_CHANNEL ? (size_t)t * Dk : (size_t)t), beta_mode,",
     "bs + (beta_mode == DRO_BETA_CHANNEL ? (size_t)t * Dk : (size_t)t), beta_mode,"),
    ("bwd_write_strength_gradient_halved",
     "double g = dvt[j] * v_t[j] / (2.0 * sbv[j]);",
     "double g = dvt[j] * v_t[j] / (4.0 * sbv[j]);"),
]


@pytest.mark.parametrize("name,old,new", BWD_KV_MUTANTS, ids=[m[0] for m in BWD_KV_MUTANTS])
def test_bwd_kv_pins_catch_planted_mistake(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "libmutant.so")))

    def fwd(q, k, v, la, beta, S0, *, gate, beta_mode, beta_v=None):
        return oracle.forward(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode, beta_v=beta_v)

    def bwd(q, k, v, la, beta, S0, dO, dS, *, gate, beta_mode, beta_v=None):
        return oracle.backward(q, k, v, la, beta, S0, dO, dS, gate=gate, beta_mode=beta_mode, beta_v=beta_v,
                               lib=lib)

    caught = []
    for pin in oracle_pins.BWD_KV_PINS:
        try:
            pin(fwd, bwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"


# Mistakes in the backward of the key scales and of the input preparation.
BWD_EX_MUTANTS = [
    ("bwd_query_projection_dropped", "l2 ? rq * (dqh[c] - qh[c] * pq) : dqh[c]", "l2 ? rq * dqh[c] : dqh[c]"),
    ("bwd_key_projection_dropped", "l2 ? rk * (dkh[c] - kh[c] * pk) : dkh[c]", "l2 ? rk * dkh[c] : dkh[c]"),
    ("bwd_logit_factor_dropped", "if (logit) g *= bkv[c] * (1.0 - bkv[c]);", "if (0) g *= bkv[c] * (1.0 - bkv[c]);"),
    ("bwd_write_logit_factor_dropped", "if (logit) g *= bvv[j] * (1.0 - bvv[j]);",
     "if (0) g *= bvv[j] * (1.0 - bvv[j]);"),
    ("bwd_write_scale_dropped", "dkt[c] = (st_ ? st_[c] : 1.0) * a - b;", "dkt[c] = a - b;"),
    ("bwd_scale_gradient_from_write_key", "dkey_scale[((size_t)s * L + t) * Dk + c] = kt[c] * a;",
     "dkey_scale[((size_t)s * L + t) * Dk + c] = w[c] * a;"),
    ("bwd_value_gradient_through_read_key", "for (int c = 0; c < Dk; ++c) a += G[(size_t)c * Dv + j] * w[c];",
     "for (int c = 0; c < Dk; ++c) a += G[(size_t)c * Dv + j] * kt[c];"),
]


@pytest.mark.parametrize("name,old,new", BWD_EX_MUTANTS, ids=[m[0] for m in BWD_EX_MUTANTS])
def test_bwd_ex_pins_catch_planted_mistake(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "libmutant.so")))

    def fwd_ex(q, k, v, la, beta, beta_v, ks, S0, *, gate, beta_mode, qk_l2norm, beta_logit):
        return oracle.forward(q, k, v, la, beta, S0, gate=gate, beta_mode=beta_mode, beta_v=beta_v, key_scale=ks,
                              qk_l2norm=qk_l2norm, beta_logit=beta_logit)

    def bwd_ex(q, k, v, la, beta, beta_v, ks, S0, dO, dS, *, gate, beta_mode, qk_l2norm, beta_logit):
        return oracle.backward(q, k, v, la, beta, S0, dO, dS, gate=gate, beta_mode=beta_mode, beta_v=beta_v,
                               key_scale=ks, qk_l2norm=qk_l2norm, beta_logit=beta_logit, lib=lib)

    caught = []
    for pin in oracle_pins.BWD_EX_PINS:
        try:
            pin(fwd_ex, bwd_ex)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
