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


# -- family corners and the correction-to-output ratio -------------------------

from tests import test_oracle_family_pins as fpins  # noqa: E402

_row_family = orc.row_family
_uniform_weights = orc.uniform_weights
_cor = orc.correction_to_output


def _fm_noint_centred(w, K, V, rho, intercept=True):
    if intercept:
        return _row_family(w, K, V, rho, True)
    vbar, kbar = w @ V, w @ K
    sigma = ((V - vbar) * w[:, None]).T @ (K - kbar)
    return -(sigma @ rho), sigma @ rho


def _fm_noint_sign(w, K, V, rho, intercept=True):
    if intercept:
        return _row_family(w, K, V, rho, True)
    sigma = (V * w[:, None]).T @ K
    return sigma @ rho, sigma @ rho


def _fm_noint_transposed(w, K, V, rho, intercept=True):
    if intercept:
        return _row_family(w, K, V, rho, True)
    sigma = (K * w[:, None]).T @ V  # d_k x d_v: sum_j w_j k_j (v_j . rho)
    return -(sigma @ rho), sigma @ rho


def _fm_noint_keeps_vbar(w, K, V, rho, intercept=True):
    if intercept:
        return _row_family(w, K, V, rho, True)
    sigma = (V * w[:, None]).T @ K
    return w @ V - sigma @ rho, sigma @ rho


def _fm_corr_is_output(w, K, V, rho, intercept=True):
    o, _ = _row_family(w, K, V, rho, intercept)
    return o, o


def _fm_uniform_n_minus_1(n):
    m = max(n - 1, 1)
    return np.full(n, 1.0 / m), np.log(m)


def _fm_uniform_lse_zero(n):
    return np.full(n, 1.0 / n), 0.0


def _fm_cor_squared(corr, o):
    return np.float64(np.dot(corr, corr)) / np.float64(np.dot(o, o))


def _fm_cor_inverted(corr, o):
    return np.float64(np.linalg.norm(o)) / np.float64(np.linalg.norm(corr))


FAMILY_MUTANTS = [
    ("row_family", _fm_noint_centred), ("row_family", _fm_noint_sign),
    ("row_family", _fm_noint_transposed), ("row_family", _fm_noint_keeps_vbar),
    ("row_family", _fm_corr_is_output), ("uniform_weights", _fm_uniform_n_minus_1),
    ("uniform_weights", _fm_uniform_lse_zero), ("correction_to_output", _fm_cor_squared),
    ("correction_to_output", _fm_cor_inverted),
]


def _family_pins():
    for name in dir(fpins):
        if name.startswith("test_"):
            fn = getattr(fpins, name)
            marks = getattr(fn, "pytestmark", [])
            params = [m for m in marks if m.name == "parametrize"]
            if params:
                for args in params[0].args[1]:
                    yield fn, tuple(args)
            else:
                yield fn, ()


@pytest.mark.parametrize("target,mutant", FAMILY_MUTANTS, ids=lambda x: x if isinstance(x, str) else x.__name__)
def test_family_pins_catch_mutant(target, mutant, monkeypatch):
    monkeypatch.setattr(orc, target, mutant)
    caught = []
    with np.errstate(all="ignore"):
        for fn, args in _family_pins():
            try:
                fn(*args)
            except Exception:
                caught.append(fn.__name__)
    assert caught, f"no pin caught {mutant.__name__}"


def test_unmutated_oracle_passes_every_family_pin():
    n = 0
    for fn, args in _family_pins():
        fn(*args)
        n += 1
    assert n >= 12


_project = orc.project_qkvr


def _pm_kv_swapped(x, W, Hq, Hkv, d):
    q, k, v, rho = _project(x, W, Hq, Hkv, d)
    return q, v, k, rho


def _pm_dim_major(x, W, Hq, Hkv, d):
    B, T, _ = x.shape
    y = x @ W.T
    outs, off = [], 0
    for H in (Hq, Hkv, Hkv, Hq):
        blk = y[:, :, off: off + H * d].reshape(B, T, d, H).transpose(0, 3, 1, 2)
        outs.append(np.ascontiguousarray(blk))
        off += H * d
    return tuple(outs)


def _pm_dim_reversed(x, W, Hq, Hkv, d):
    return tuple(np.ascontiguousarray(t[..., ::-1]) for t in _project(x, W, Hq, Hkv, d))


def _pm_heads_of_block_swapped(x, W, Hq, Hkv, d):
    q, k, v, rho = _project(x, W, Hq, Hkv, d)
    return q[:, ::-1].copy(), k, v, rho


@pytest.mark.parametrize("mutant", [_pm_kv_swapped, _pm_dim_major, _pm_dim_reversed, _pm_heads_of_block_swapped],
                         ids=lambda f: f.__name__)
def test_projection_pins_catch_mutant(mutant, monkeypatch):
    monkeypatch.setattr(orc, "project_qkvr", mutant)
    caught = []
    for fn in (fpins.test_projection_exact_integers_brute_force,
               fpins.test_projection_one_hot_tokens_place_weight_columns):
        try:
            fn()
        except Exception:
            caught.append(fn.__name__)
    assert caught, f"no pin caught {mutant.__name__}"
