"""Plants plausible mistakes in the NumPy oracle (CPU only) and checks that the
pins in test_oracle_pins.py catch every one of them.

Each mutant replaces ``oracle.kla_ref.step`` for the duration of one test;
``kla_ref.forward`` and ``kla_ref.decode_step`` pick it up through the module.
"""
import numpy as np
import pytest

from oracle import kla_ref
from tests import test_oracle_pins as pins

_real_step = kla_ref.step


def _mk(variant):
    def step(S, q_t, k_t, v_t, log_alpha_t, eta_t, eps, beta_mode="kaczmarz"):
        S = np.asarray(S, dtype=np.float64)
        q_t, k_t, v_t = (np.asarray(x, dtype=np.float64) for x in (q_t, k_t, v_t))
        alpha = np.exp(np.asarray(log_alpha_t, dtype=np.float64))
        nk = np.sum(k_t * k_t, axis=-1)
        eps32 = np.float64(np.float32(eps))
        eta = np.asarray(eta_t, dtype=np.float64)
        if beta_mode == "direct":
            if variant == "direct_still_normalised":
                beta = eta / np.where(nk + eps32 != 0, nk + eps32, 1.0)
            elif variant == "direct_ignores_eta":
                beta = np.ones_like(nk)
            else:
                beta = np.broadcast_to(eta, nk.shape).copy()
        elif variant == "beta_norm_not_squared":
            beta = eta / (np.sqrt(nk) + eps32)
        elif variant == "beta_ignores_eta":
            beta = 1.0 / (nk + eps32)
        elif variant == "beta_ignores_eps":
            beta = eta / np.where(nk != 0, nk, 1.0)
        else:
            beta = eta / np.where(nk + eps32 != 0, nk + eps32, 1.0)
        S_dec = alpha[..., None, None] * S
        if variant == "residual_undecayed":
            e = v_t - np.einsum("...kv,...k->...v", S, k_t)
        elif variant == "residual_sign":
            e = np.einsum("...kv,...k->...v", S_dec, k_t) - v_t
        elif variant == "residual_transposed":
            e = v_t - np.einsum("...kv,...v->...k", S_dec, k_t) if S.shape[-1] == S.shape[-2] else \
                v_t - np.einsum("...kv,...k->...v", S_dec, k_t) * 1.0001
        else:
            e = v_t - np.einsum("...kv,...k->...v", S_dec, k_t)
        if variant == "write_outer_transposed" and S.shape[-1] == S.shape[-2]:
            upd = e[..., :, None] * k_t[..., None, :]
        else:
            upd = k_t[..., :, None] * e[..., None, :]
        if variant == "decay_after_write":
            S_new = alpha[..., None, None] * (S + beta[..., None, None] * upd)
        elif variant == "no_decay":
            S_new = S + beta[..., None, None] * upd
        else:
            S_new = S_dec + beta[..., None, None] * upd
        if variant == "readout_before_write":
            o = np.einsum("...kv,...k->...v", S_dec, q_t)
        elif variant == "readout_with_key":
            o = np.einsum("...kv,...k->...v", S_new, k_t)
        else:
            o = np.einsum("...kv,...k->...v", S_new, q_t)
        return o, S_new
    return step


MUTANTS = ["beta_norm_not_squared", "beta_ignores_eta", "beta_ignores_eps", "residual_undecayed",
           "residual_sign", "residual_transposed", "write_outer_transposed", "decay_after_write",
           "no_decay", "readout_before_write", "readout_with_key", "direct_still_normalised",
           "direct_ignores_eta"]

PIN_CALLS = [
    lambda: pins.test_worked_example_exact(kla_ref.forward),
    pins.test_worked_example_exact_no_decay_rounding,
    lambda: pins.test_constraint_exact_projection(kla_ref.forward),
    pins.test_minimum_norm_change,
    pins.test_exact_line_search,
    pins.test_normalised_sgd_step,
    lambda: pins.test_orthogonal_keys_reduce_to_masked_form(kla_ref.forward),
    lambda: pins.test_repeated_key_overwrite(kla_ref.forward),
    lambda: pins.test_pure_decay(kla_ref.forward),
    lambda: pins.test_product_form_brute_force(kla_ref.forward),
    lambda: pins.test_direct_equals_kaczmarz_on_unit_keys("numpy"),
    lambda: pins.test_write_residual_law("numpy"),
]


def test_unmutated_oracle_passes_all_pins():
    for call in PIN_CALLS:
        call()


@pytest.mark.parametrize("variant", MUTANTS)
def test_mutant_is_caught(monkeypatch, variant):
    monkeypatch.setattr(kla_ref, "step", _mk(variant))
    caught = 0
    for call in PIN_CALLS:
        try:
            call()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin catches the planted mistake {variant!r}"
