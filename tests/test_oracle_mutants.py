"""The oracle pins must catch plausible mistakes.

Each mutant below is a copy of the oracle's covariance step with one planted
error (a sign, a transpose, a dropped centering, a wrong normalisation...).
With the mutant patched into the oracle, at least one forward pin must fail.
"""

import numpy as np
import pytest

from oracle import plx_oracle as orc
from tests import test_oracle_pins as pins


def _m_sign(w, K, V, rho):
    vbar, kbar = w @ V, w @ K
    sigma = ((V - vbar) * w[:, None]).T @ (K - kbar)
    return vbar + sigma @ rho, vbar, kbar, sigma


def _m_transpose(w, K, V, rho):
    vbar, kbar = w @ V, w @ K
    sigma = ((K - kbar) * w[:, None]).T @ (V - vbar)  # d_k x d_v
    o = vbar - (sigma @ rho[: sigma.shape[1]] if sigma.shape[0] == vbar.shape[0] else sigma.T @ rho)
    return o, vbar, kbar, sigma


def _m_no_centering(w, K, V, rho):
    # Centering only one factor is an exact identity (the weighted mean of
    # v_j - vbar is zero), so the planted error drops both centerings.
    vbar, kbar = w @ V, w @ K
    sigma = (V * w[:, None]).T @ K
    return vbar - sigma @ rho, vbar, kbar, sigma


def _m_unweighted(w, K, V, rho):
    vbar, kbar = w @ V, w @ K
    n = K.shape[0]
    sigma = (V - vbar).T @ (K - kbar) / n
    return vbar - sigma @ rho, vbar, kbar, sigma


def _m_sample_cov(w, K, V, rho):
    vbar, kbar = w @ V, w @ K
    n = K.shape[0]
    sigma = ((V - vbar) * w[:, None]).T @ (K - kbar)
    if n > 1:
        sigma = sigma * (n / (n - 1))
    return vbar - sigma @ rho, vbar, kbar, sigma


def _m_no_intercept(w, K, V, rho):
    vbar, kbar = w @ V, w @ K
    sigma = ((V - vbar) * w[:, None]).T @ (K - kbar)
    return -(sigma @ rho), vbar, kbar, sigma


def _m_squared_weights(w, K, V, rho):
    vbar, kbar = w @ V, w @ K
    sigma = ((V - vbar) * (w * w)[:, None]).T @ (K - kbar)
    return vbar - sigma @ rho, vbar, kbar, sigma


MUTANTS = [_m_sign, _m_transpose, _m_no_centering, _m_unweighted,
           _m_sample_cov, _m_no_intercept, _m_squared_weights]


def _forward_pins():
    yield pins.test_single_key_row_returns_its_value_for_any_probe, ()
    yield pins.test_zero_probe_is_causal_softmax_attention, (1, 1, 1, 17, 8)
    yield pins.test_uniform_weights_give_population_cross_covariance, ()
    yield pins.test_solved_probe_reproduces_weighted_local_linear_regression, (0,)
    yield pins.test_two_key_closed_form, ()
    for s in range(6):
        yield pins.test_streaming_identity_exact_rationals, (s,)
    yield pins.test_output_is_affine_in_probe, ()
    yield pins.test_constant_values_or_keys_kill_the_correction, ()


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_pins_catch_mutant(mutant, monkeypatch):
    monkeypatch.setattr(orc, "row_from_weights", mutant)
    caught = []
    for fn, args in _forward_pins():
        try:
            fn(*args)
        except Exception:  # assertion or a shape error both count as caught
            caught.append(fn.__name__)
    assert caught, f"no pin caught {mutant.__name__}"


def test_unmutated_oracle_passes_every_forward_pin():
    for fn, args in _forward_pins():
        fn(*args)
