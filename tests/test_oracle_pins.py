"""The float64 oracle against independent pins, and planted mistakes against the pins.

CPU only.  See tests/oracle_pins.py for what each pin states.
"""
import numpy as np
import pytest

import oracle.kla_f64 as O
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# Plausible mistakes, each planted in one step function of the oracle.  Every one
# must make at least one pin fail; otherwise the pins would not notice it.
MUTANTS = {
    "predict_drops_process_noise": ("predict_precision", lambda lam, a, pbar: lam / (a * a)),
    "predict_uses_a_not_a2": ("predict_precision", lambda lam, a, pbar: lam / (a + pbar * lam)),
    "predict_noise_wrong_side": ("predict_precision", lambda lam, a, pbar: lam / (a * a) + pbar),
    "update_drops_evidence": ("update_precision", lambda lam_pred, c: lam_pred),
    "update_subtracts_evidence": ("update_precision", lambda lam_pred, c: lam_pred - c),
    "forget_drops_decay": ("forget_gate", lambda a, lam_pred, lam: lam_pred / lam),
    "forget_inverted": ("forget_gate", lambda a, lam_pred, lam: a * lam / lam_pred),
    "forget_squared_decay": ("forget_gate", lambda a, lam_pred, lam: a * a * lam_pred / lam),
    "write_drops_value_precision": ("write_gate", lambda k, vp, lam: k / lam),
    "write_sign_flipped": ("write_gate", lambda k, vp, lam: -k * vp / lam),
    "write_uses_k_squared": ("write_gate", lambda k, vp, lam: k * k * vp / lam),
    "readout_transposed_state": ("readout",
                                 lambda q, M: np.einsum("...i,...ji->...j", q, M[..., : q.shape[-1], : q.shape[-1]])),
    "readout_sums_without_q": ("readout", lambda q, M: M.sum(axis=-2)),
    "readout_abs_q": ("readout", lambda q, M: np.einsum("...i,...ij->...j", np.abs(q), M)),
}


# Plausible mistakes in the OU discretisation (oracle/kla_ou_f64.py).
def _ou_no_factor_two(theta, sigma2, dt):
    th, s2, d = (np.asarray(x, np.float64) for x in (theta, sigma2, dt))
    return -th * d, s2 * (-np.expm1(-th * d)) / np.where(th == 0, 1.0, th)


def _ou_euler(theta, sigma2, dt):
    th, s2, d = (np.asarray(x, np.float64) for x in (theta, sigma2, dt))
    return -th * d, s2 * d


def _ou_variance_squared_decay(theta, sigma2, dt):
    th, s2, d = (np.asarray(x, np.float64) for x in (theta, sigma2, dt))
    return -th * d, s2 * (-np.expm1(-th * d)) / np.where(th == 0, 1.0, 2 * th)


OU_MUTANTS = {"ou_drops_factor_two": _ou_no_factor_two, "ou_euler_noise": _ou_euler,
              "ou_noise_uses_a_not_a2": _ou_variance_squared_decay}


@pytest.mark.parametrize("name", sorted(OU_MUTANTS))
def test_pins_catch_planted_ou_mistake(name, monkeypatch):
    import oracle.kla_ou_f64 as OU
    monkeypatch.setattr(OU, "ou_discretize_f64", OU_MUTANTS[name])
    failed = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"


# Plausible mistakes in the prologue (oracle/kla_prologue_f64.py): name of the
# module function and its replacement.
def _conv_reversed_taps(x, w, b=None):
    import oracle.kla_prologue_f64 as OP
    return OP.__dict__["_orig_conv"](x, np.asarray(w)[..., ::-1], b)


def _conv_centred(x, w, b=None):
    import oracle.kla_prologue_f64 as OP
    u = OP.__dict__["_orig_conv"](x, w, b)
    sh = (np.asarray(w).shape[-1] - 1) // 2
    return np.concatenate([u[:, :, sh:], np.zeros_like(u[:, :, :sh])], axis=2)


def _conv_no_bias(x, w, b=None):
    import oracle.kla_prologue_f64 as OP
    return OP.__dict__["_orig_conv"](x, w, None)


PROLOGUE_MUTANTS = {
    "conv_reversed_taps": ("causal_conv_f64", _conv_reversed_taps),
    "conv_not_causal": ("causal_conv_f64", _conv_centred),
    "conv_drops_bias": ("causal_conv_f64", _conv_no_bias),
    "silu_is_sigmoid": ("silu_f64", lambda u: 1.0 / (1.0 + np.exp(-np.asarray(u, np.float64)))),
    "silu_wrong_sign": ("silu_f64", lambda u: np.asarray(u, np.float64) / (1.0 + np.exp(np.asarray(u, np.float64)))),
    "softplus_is_exp": ("softplus_f64", lambda x: np.exp(np.asarray(x, np.float64))),
    "softplus_is_relu": ("softplus_f64", lambda x: np.maximum(np.asarray(x, np.float64), 0.0)),
}


@pytest.mark.parametrize("name", sorted(PROLOGUE_MUTANTS))
def test_pins_catch_planted_prologue_mistake(name, monkeypatch):
    import oracle.kla_prologue_f64 as OP
    attr, fn = PROLOGUE_MUTANTS[name]
    monkeypatch.setitem(OP.__dict__, "_orig_conv", OP.causal_conv_f64)
    monkeypatch.setattr(OP, attr, fn)
    failed = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:  # AssertionError or a shape/ValueError from the mutant
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
