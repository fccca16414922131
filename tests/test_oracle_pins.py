"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a library routine (torch SDPA,
numpy covariance, least squares), a closed form, exact rational arithmetic,
an invariant of the definition, or finite differences.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import plx_oracle as orc

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa_causal(q, k, v, scale):
    """torch fp64 CPU softmax attention, causal, GQA by repeating KV heads."""
    group = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(np.repeat(k, group, axis=1))
    vt = torch.from_numpy(np.repeat(v, group, axis=1))
    qt = torch.from_numpy(q)
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, is_causal=True, scale=scale).numpy()


# -- single key ---------------------------------------------------------------

def test_single_key_row_returns_its_value_for_any_probe():
    """A query with one key has zero covariance, so o = v_0 exactly."""
    g = _rng(10)
    for _ in range(5):
        K = g.standard_normal((1, 7))
        V = g.standard_normal((1, 5))
        q, rho = g.standard_normal(7), 100 * g.standard_normal(7)
        o, o_sa, lse, sigma = orc.row_forward(q, K, V, rho, 0.3)
        assert np.array_equal(sigma, np.zeros((5, 7)))
        assert np.array_equal(o, V[0])
        assert np.array_equal(o_sa, V[0])
    # prefill row 0 has exactly one key
    q = g.standard_normal((1, 1, 6, 4))
    k = g.standard_normal((1, 1, 6, 4))
    v = g.standard_normal((1, 1, 6, 4))
    rho = g.standard_normal((1, 1, 6, 4))
    out = orc.prefill_forward(q, k, v, rho, 0.5)
    assert np.array_equal(out["o"][0, 0, 0], v[0, 0, 0])


# -- rho = 0 is softmax attention (W_R = 0 recovers the Transformer) ----------

@pytest.mark.parametrize("B,Hq,Hkv,T,d", [(1, 1, 1, 17, 8), (2, 4, 2, 23, 16), (1, 6, 3, 9, 5)])
def test_zero_probe_is_causal_softmax_attention(B, Hq, Hkv, T, d):
    g = _rng(11)
    q = g.standard_normal((B, Hq, T, d))
    k = g.standard_normal((B, Hkv, T, d))
    v = g.standard_normal((B, Hkv, T, d))
    rho = np.zeros((B, Hq, T, d))
    scale = 1.0 / np.sqrt(d)
    out = orc.prefill_forward(q, k, v, rho, scale)
    ref = _sdpa_causal(q, k, v, scale)
    np.testing.assert_allclose(out["o"], ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(out["o_sa"], ref, rtol=0, atol=1e-13)
    # LSE: natural log-sum-exp of the scaled causal scores
    group = Hq // Hkv
    kr = torch.from_numpy(np.repeat(k, group, axis=1))
    s = torch.from_numpy(q) @ kr.transpose(-1, -2) * scale
    mask = torch.triu(torch.ones(T, T, dtype=torch.bool), diagonal=1)
    lse_ref = torch.logsumexp(s.masked_fill(mask, float("-inf")), dim=-1).numpy()
    np.testing.assert_allclose(out["lse"], lse_ref, rtol=0, atol=1e-12)


# -- uniform weights: the unweighted covariance (bandwidth -> infinity) --------

def test_uniform_weights_give_population_cross_covariance():
    """q = 0 makes every weight 1/n; Sigma must then equal numpy's biased
    cross-covariance of (v, k), with v on the rows and k on the columns."""
    g = _rng(12)
    n, dk, dv = 13, 4, 3  # d_v != d_k catches a transposed Sigma
    K = g.standard_normal((n, dk))
    V = g.standard_normal((n, dv))
    rho = g.standard_normal(dk)
    o, o_sa, _, sigma = orc.row_forward(np.zeros(dk), K, V, rho, 1.0)
    cov = np.cov(np.hstack([V, K]).T, bias=True)[:dv, dv:]
    np.testing.assert_allclose(sigma, cov, rtol=0, atol=1e-14)
    np.testing.assert_allclose(o_sa, V.mean(axis=0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o, V.mean(axis=0) - cov @ rho, rtol=0, atol=1e-14)


# -- local linear regression: the probe the exact method would solve for ------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_solved_probe_reproduces_weighted_local_linear_regression(seed):
    """With rho = Sigma_KK^{-1}(kbar - x0) the output must equal the intercept of
    the weighted least-squares fit v ~ b + W (k - x0) evaluated at x0.  This is
    the local-linear estimator that Parallax parameterises; numpy's lstsq and
    weighted covariance fix the expected value."""
    g = _rng(100 + seed)
    n, dk, dv = 11, 3, 2
    K = g.standard_normal((n, dk))
    V = g.standard_normal((n, dv))
    q = g.standard_normal(dk)
    scale = 0.7
    s = scale * K @ q
    w = np.exp(s - s.max())
    w /= w.sum()
    kbar = np.average(K, axis=0, weights=w)
    sigma_kk = np.cov(K.T, aweights=w, bias=True)
    x0 = q
    rho_star = np.linalg.solve(sigma_kk, kbar - x0)
    o, _, _, _ = orc.row_forward(q, K, V, rho_star, scale)
    X = np.hstack([np.ones((n, 1)), K - x0])
    sw = np.sqrt(w)[:, None]
    coef, *_ = np.linalg.lstsq(sw * X, sw * V, rcond=None)
    np.testing.assert_allclose(o, coef[0], rtol=0, atol=1e-10)


# -- two keys: closed form -----------------------------------------------------

def test_two_key_closed_form():
    """With two keys, Sigma = w1 w2 (v1 - v2)(k1 - k2)^T, so
    o = vbar - w1 w2 (v1 - v2) ((k1 - k2) . rho)."""
    g = _rng(13)
    for _ in range(10):
        K = g.standard_normal((2, 6))
        V = g.standard_normal((2, 4))
        q, rho = g.standard_normal(6), g.standard_normal(6)
        scale = 0.4
        a = scale * K[0] @ q
        b = scale * K[1] @ q
        w1 = 1.0 / (1.0 + np.exp(b - a))
        w2 = 1.0 - w1
        vbar = w1 * V[0] + w2 * V[1]
        expect = vbar - w1 * w2 * (V[0] - V[1]) * ((K[0] - K[1]) @ rho)
        o, o_sa, _, _ = orc.row_forward(q, K, V, rho, scale)
        np.testing.assert_allclose(o, expect, rtol=0, atol=1e-14)
        np.testing.assert_allclose(o_sa, vbar, rtol=0, atol=1e-14)


# -- the streaming identity, exactly ------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_streaming_identity_exact_rationals(seed):
    """Exact arithmetic: Sigma rho = sum_j w_j (k_j . rho) v_j - vbar (kbar . rho)
    equals the oracle's explicit covariance form, for rational weights."""
    g = _rng(200 + seed)
    n = int(g.integers(1, 7))
    dk, dv = int(g.integers(1, 4)), int(g.integers(1, 4))
    K = np.array([[Fraction(int(x)) for x in row] for row in g.integers(-5, 6, (n, dk))], dtype=object)
    V = np.array([[Fraction(int(x)) for x in row] for row in g.integers(-5, 6, (n, dv))], dtype=object)
    rho = np.array([Fraction(int(x), int(y)) for x, y in zip(g.integers(-5, 6, dk), g.integers(1, 4, dk))],
                   dtype=object)
    raw = [Fraction(int(x)) for x in g.integers(1, 9, n)]
    total = sum(raw)
    w = np.array([x / total for x in raw], dtype=object)
    o, vbar, kbar, sigma = orc.row_from_weights(w, K, V, rho)
    # identity side, written independently in exact arithmetic
    r = [sum(K[j, t] * rho[t] for t in range(dk)) for j in range(n)]
    c = sum(w[j] * r[j] for j in range(n))
    vb = [sum(w[j] * V[j, t] for j in range(n)) for t in range(dv)]
    u = [sum(w[j] * r[j] * V[j, t] for j in range(n)) for t in range(dv)]
    o_identity = [vb[t] * (1 + c) - u[t] for t in range(dv)]
    assert list(o) == o_identity
    assert list(vbar) == vb


# -- structure of the correction ---------------------------------------------

def test_output_is_affine_in_probe():
    g = _rng(14)
    n, d = 9, 5
    K, V = g.standard_normal((n, d)), g.standard_normal((n, d))
    q = g.standard_normal(d)
    r1, r2 = g.standard_normal(d), g.standard_normal(d)
    o1, sa, _, _ = orc.row_forward(q, K, V, r1, 0.5)
    o2, _, _, _ = orc.row_forward(q, K, V, r2, 0.5)
    o12, _, _, _ = orc.row_forward(q, K, V, r1 + 2.5 * r2, 0.5)
    np.testing.assert_allclose(o12 - sa, (o1 - sa) + 2.5 * (o2 - sa), rtol=0, atol=1e-13)


def test_constant_values_or_keys_kill_the_correction():
    g = _rng(15)
    n, d = 8, 4
    K = g.standard_normal((n, d))
    V = np.tile(g.standard_normal(d), (n, 1))
    q, rho = g.standard_normal(d), g.standard_normal(d)
    o, sa, _, _ = orc.row_forward(q, K, V, rho, 1.0)
    np.testing.assert_allclose(o, V[0], rtol=0, atol=1e-14)
    K2 = np.tile(g.standard_normal(d), (n, 1))
    V2 = g.standard_normal((n, d))
    o, sa, _, _ = orc.row_forward(q, K2, V2, rho, 1.0)
    np.testing.assert_allclose(o, V2.mean(axis=0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o, sa, rtol=0, atol=1e-14)


def test_zero_query_lse_counts_keys():
    """q = 0: every score is 0, so LSE_i = ln(i + 1) exactly (the key count)."""
    T, d = 40, 4
    g = _rng(16)
    q = np.zeros((1, 1, T, d))
    k = g.standard_normal((1, 1, T, d))
    v = g.standard_normal((1, 1, T, d))
    out = orc.prefill_forward(q, k, v, np.zeros_like(q), 1.0)
    np.testing.assert_allclose(out["lse"][0, 0], np.log(np.arange(1, T + 1)), rtol=0, atol=1e-13)


# -- decode and GQA ----------------------------------------------------------

def test_decode_equals_last_prefill_row_and_ignores_cache_order():
    g = _rng(17)
    B, Hq, Hkv, T, d = 2, 4, 2, 19, 8
    q = g.standard_normal((B, Hq, T, d))
    k = g.standard_normal((B, Hkv, T, d))
    v = g.standard_normal((B, Hkv, T, d))
    rho = g.standard_normal((B, Hq, T, d))
    pre = orc.prefill_forward(q, k, v, rho, 0.35)
    ctx = np.array([T, 11])
    qd = np.stack([q[0, :, T - 1], q[1, :, 10]])
    rd = np.stack([rho[0, :, T - 1], rho[1, :, 10]])
    dec = orc.decode_forward(qd, rd, k, v, ctx, 0.35)
    o = dec["o"].reshape(B, Hq, d)
    np.testing.assert_allclose(o[0], pre["o"][0, :, T - 1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(o[1], pre["o"][1, :, 10], rtol=0, atol=1e-13)
    perm = g.permutation(T)
    dec_p = orc.decode_forward(qd[:1], rd[:1], k[:1, :, perm], v[:1, :, perm], ctx[:1], 0.35)
    np.testing.assert_allclose(dec_p["o"], dec["o"][:Hq], rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    g = _rng(18)
    B, Hq, Hkv, T, d = 1, 6, 2, 10, 4
    q = g.standard_normal((B, Hq, T, d))
    k = g.standard_normal((B, Hkv, T, d))
    v = g.standard_normal((B, Hkv, T, d))
    rho = g.standard_normal((B, Hq, T, d))
    a = orc.prefill_forward(q, k, v, rho, 0.5)
    b = orc.prefill_forward(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), rho, 0.5)
    np.testing.assert_array_equal(a["o"], b["o"])


# -- backward ----------------------------------------------------------------

def _loss(q, k, v, rho, g, scale):
    return float(np.sum(orc.prefill_forward(q, k, v, rho, scale)["o"] * g))


def test_backward_matches_central_finite_differences_T32():
    rng = _rng(19)
    B, Hq, Hkv, T, d = 1, 2, 1, 32, 6
    scale = 1.0 / np.sqrt(d)
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    rho = 0.5 * rng.standard_normal((B, Hq, T, d))
    g = rng.standard_normal((B, Hq, T, d))
    grads = orc.prefill_backward(q, k, v, rho, g, scale)
    inputs = {"q": q, "k": k, "v": v, "rho": rho}
    names = {"q": "dq", "k": "dk", "v": "dv", "rho": "drho"}
    h = 1e-5
    for name, x in inputs.items():
        flat = x.reshape(-1)
        idx = rng.choice(flat.size, size=24, replace=False)
        for t in idx:
            old = flat[t]
            flat[t] = old + h
            lp = _loss(q, k, v, rho, g, scale)
            flat[t] = old - h
            lm = _loss(q, k, v, rho, g, scale)
            flat[t] = old
            fd = (lp - lm) / (2 * h)
            an = grads[names[name]].reshape(-1)[t]
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (name, t, fd, an)


def test_backward_zero_probe_matches_torch_autograd_of_sdpa():
    rng = _rng(20)
    B, Hq, Hkv, T, d = 1, 4, 2, 12, 8
    scale = 1.0 / np.sqrt(d)
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    g = rng.standard_normal((B, Hq, T, d))
    grads = orc.prefill_backward(q, k, v, np.zeros_like(q), g, scale)
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(2, dim=1), vt.repeat_interleave(2, dim=1), is_causal=True, scale=scale)
    out.backward(torch.from_numpy(g))
    np.testing.assert_allclose(grads["dq"], qt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(grads["dk"], kt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(grads["dv"], vt.grad.numpy(), rtol=0, atol=1e-12)


def test_probe_gradient_is_minus_covariance_transpose_times_upstream():
    """o is affine in rho with slope -Sigma, so d<g,o>/d rho = -Sigma^T g; the
    slope is measured here by differencing the output, not read from Sigma."""
    rng = _rng(21)
    n, d = 14, 5
    K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    q, rho, g = rng.standard_normal(d), rng.standard_normal(d), rng.standard_normal(d)
    _, _, _, drho = orc.row_backward(q, K, V, rho, g, 0.6)
    o0, _, _, _ = orc.row_forward(q, K, V, rho, 0.6)
    slope = np.empty((d, d))
    for t in range(d):
        e = np.zeros(d)
        e[t] = 1.0
        o1, _, _, _ = orc.row_forward(q, K, V, rho + e, 0.6)
        slope[:, t] = o1 - o0  # exact: o is affine in rho
    np.testing.assert_allclose(drho, slope.T @ g, rtol=0, atol=1e-12)


def test_kv_row_gradients_match_full_backward():
    rng = _rng(22)
    B, Hq, Hkv, T, d = 1, 4, 2, 10, 4
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    rho = rng.standard_normal((B, Hq, T, d))
    g = rng.standard_normal((B, Hq, T, d))
    full = orc.prefill_backward(q, k, v, rho, g, 0.5)

    def get_row(b, h, hk, i):
        return q[b, h, i], k[b, hk, :i + 1], v[b, hk, :i + 1], rho[b, h, i], g[b, h, i]

    keys = [(0, 0, 0), (0, 1, 7), (0, 1, 9)]
    dk, dv = orc.prefill_backward_kv_rows(get_row, keys, T, Hq, Hkv, 0.5)
    for n, (b, hk, j) in enumerate(keys):
        np.testing.assert_allclose(dk[n], full["dk"][b, hk, j], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv[n], full["dv"][b, hk, j], rtol=0, atol=1e-13)


def test_probe_mean_c_is_softmax_weighted_probe_score():
    """c_i = kbar_i . rho_i equals sum_j w_ij (rho_i . k_j), with w from torch's
    causal softmax (fp64)."""
    g = _rng(23)
    B, Hq, Hkv, T, d = 1, 4, 2, 21, 6
    q = g.standard_normal((B, Hq, T, d))
    k = g.standard_normal((B, Hkv, T, d))
    v = g.standard_normal((B, Hkv, T, d))
    rho = g.standard_normal((B, Hq, T, d))
    out = orc.prefill_forward(q, k, v, rho, 0.4)
    kk = torch.from_numpy(np.repeat(k, 2, axis=1))
    s = 0.4 * torch.from_numpy(q) @ kk.transpose(-1, -2)
    s = s.masked_fill(~torch.ones(T, T, dtype=torch.bool).tril(), float("-inf"))
    w = torch.softmax(s, dim=-1)
    r = torch.from_numpy(rho) @ kk.transpose(-1, -2)
    np.testing.assert_allclose(out["c"], (w * r).sum(-1).numpy(), rtol=0, atol=1e-12)
