"""Pins of the oracle's family corners, correction-to-output ratio and stacked
projection against facts that do not come from the oracle's own code: numpy's
covariance, the recurrent (state-space) form of causal linear attention,
torch's softmax and SDPA, exact rational and integer arithmetic, one-hot
placement probes, and invariants of the definitions.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import plx_oracle as orc


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(seed, B=1, Hq=2, Hkv=1, T=11, d=6, dv=None):
    g = _rng(seed)
    dv = dv or d
    q = g.standard_normal((B, Hq, T, d))
    k = g.standard_normal((B, Hkv, T, d))
    v = g.standard_normal((B, Hkv, T, dv))
    rho = 0.5 * g.standard_normal((B, Hq, T, d))
    return q, k, v, rho


def _torch_causal_weights(q, k, scale):
    """Causal softmax weights [B, Hq, T, T] from torch (GQA by repeating K)."""
    group = q.shape[1] // k.shape[1]
    kr = torch.from_numpy(np.repeat(k, group, axis=1))
    s = torch.from_numpy(q) @ kr.transpose(-1, -2) * scale
    T = q.shape[2]
    mask = torch.triu(torch.ones(T, T, dtype=torch.bool), diagonal=1)
    return torch.softmax(s.masked_fill(mask, float("-inf")), dim=-1).numpy()


def _sdpa(q, k, v, scale):
    group = q.shape[1] // k.shape[1]
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(np.repeat(k, group, axis=1)),
        torch.from_numpy(np.repeat(v, group, axis=1)), is_causal=True, scale=scale).numpy()


# -- uniform weights, intercept: the unweighted cross-covariance ---------------

def test_uniform_intercept_is_population_cross_covariance_for_any_query():
    """With the uniform flag the query plays no part: Sigma is numpy's biased
    cross-covariance of (v, k) over the causal prefix, o = mean(v) - Sigma rho,
    and the LSE is ln n."""
    q, k, v, rho = _inputs(1, d=4, dv=3)
    out = orc.prefill_forward_family(q, k, v, rho, 0.3, uniform=True, intercept=True)
    for h in range(2):
        for i in range(k.shape[2]):
            K, V = k[0, 0, : i + 1], v[0, 0, : i + 1]
            cov = np.cov(np.hstack([V, K]).T, bias=True)[:3, 3:] if i else np.zeros((3, 4))
            np.testing.assert_allclose(out["o"][0, h, i], V.mean(0) - cov @ rho[0, h, i], rtol=0, atol=1e-13)
            assert abs(out["lse"][0, h, i] - np.log(i + 1)) < 1e-15


def test_uniform_flag_equals_softmax_oracle_at_zero_query():
    """q = 0 makes the softmax weights uniform, so the already pinned softmax
    oracle at q = 0 must agree with the uniform flag at any q."""
    q, k, v, rho = _inputs(2, B=2, Hq=4, Hkv=2, T=9, d=5)
    ref = orc.prefill_forward(np.zeros_like(q), k, v, rho, 0.7)
    out = orc.prefill_forward_family(q, k, v, rho, 0.7, uniform=True, intercept=True)
    np.testing.assert_allclose(out["o"], ref["o"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(out["lse"], ref["lse"], rtol=0, atol=1e-13)


# -- uniform weights, no intercept: causal linear attention --------------------

def test_uniform_no_intercept_is_recurrent_linear_attention():
    """The linear-attention corner written as a recurrence over a d_v x d_k
    state: S_t = S_{t-1} + v_t k_t^T, o_t = -S_t rho_t / t."""
    q, k, v, rho = _inputs(3, B=1, Hq=2, Hkv=2, T=14, d=5, dv=3)
    out = orc.prefill_forward_family(q, k, v, rho, 0.5, uniform=True, intercept=False)
    for h in range(2):
        S = np.zeros((3, 5))
        for t in range(14):
            S = S + np.outer(v[0, h, t], k[0, h, t])
            np.testing.assert_allclose(out["o"][0, h, t], -(S @ rho[0, h, t]) / (t + 1), rtol=0, atol=1e-13)


def test_uniform_no_intercept_exact_rationals():
    """Exact arithmetic on small integers: o = -(1/n) sum_j (k_j . rho) v_j."""
    g = _rng(4)
    for _ in range(6):
        n, dk, dv = int(g.integers(1, 7)), int(g.integers(1, 4)), int(g.integers(1, 4))
        K = np.array([[Fraction(int(x)) for x in r] for r in g.integers(-5, 6, (n, dk))], dtype=object)
        V = np.array([[Fraction(int(x)) for x in r] for r in g.integers(-5, 6, (n, dv))], dtype=object)
        rho = np.array([Fraction(int(x), 3) for x in g.integers(-5, 6, dk)], dtype=object)
        w = np.array([Fraction(1, n)] * n, dtype=object)
        o, corr = orc.row_family(w, K, V, rho, intercept=False)
        expect = [-sum(sum(K[j, t] * rho[t] for t in range(dk)) * V[j, e] for j in range(n)) / n
                  for e in range(dv)]
        assert list(o) == expect
        assert list(corr) == [-x for x in expect]


# -- softmax weights, no intercept ---------------------------------------------

def test_softmax_no_intercept_is_minus_weighted_probe_scores_times_values():
    """Matrix form from torch's causal softmax: o = -(W . (rho K^T)) V."""
    q, k, v, rho = _inputs(5, B=1, Hq=4, Hkv=2, T=10, d=6)
    scale = 0.4
    out = orc.prefill_forward_family(q, k, v, rho, scale, uniform=False, intercept=False)
    W = _torch_causal_weights(q, k, scale)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    R = rho @ kr.transpose(0, 1, 3, 2)
    np.testing.assert_allclose(out["o"], -((W * R) @ vr), rtol=0, atol=1e-13)


def test_intercept_minus_no_intercept_is_vbar_times_one_plus_c():
    """o_int - o_noint = vbar (1 + kbar . rho), with vbar = SDPA(q, k, v) and
    kbar = SDPA(q, k, k) from torch, and o_int the pinned Parallax oracle."""
    q, k, v, rho = _inputs(6, B=2, Hq=2, Hkv=1, T=12, d=4)
    scale = 0.6
    o_int = orc.prefill_forward(q, k, v, rho, scale)["o"]
    o_no = orc.prefill_forward_family(q, k, v, rho, scale, intercept=False)["o"]
    vbar = _sdpa(q, k, v, scale)
    kbar = _sdpa(q, k, k, scale)
    c = np.sum(kbar * rho, axis=-1, keepdims=True)
    np.testing.assert_allclose(o_int - o_no, vbar * (1 + c), rtol=0, atol=1e-12)


def test_default_corner_is_the_parallax_oracle():
    q, k, v, rho = _inputs(7, B=1, Hq=2, Hkv=1, T=8, d=4)
    a = orc.prefill_forward(q, k, v, rho, 0.5)
    b = orc.prefill_forward_family(q, k, v, rho, 0.5)
    np.testing.assert_array_equal(a["o"], b["o"])
    np.testing.assert_array_equal(a["lse"], b["lse"])


# -- correction-to-output ratio ------------------------------------------------

def test_cor_against_sdpa_and_its_invariants():
    """COR = ||vbar - o|| / ||o|| with vbar from torch SDPA; zero at rho = 0;
    exactly one at the no-intercept corners (the whole output is the
    correction); the correction doubles with rho."""
    q, k, v, rho = _inputs(8, B=1, Hq=2, Hkv=1, T=9, d=5)
    scale = 0.45
    out = orc.prefill_forward_family(q, k, v, rho, scale)
    vbar = _sdpa(q, k, v, scale)
    expect = np.linalg.norm(vbar - out["o"], axis=-1) / np.linalg.norm(out["o"], axis=-1)
    np.testing.assert_allclose(out["cor"], expect, rtol=1e-11, atol=0)
    zero = orc.prefill_forward_family(q, k, v, np.zeros_like(rho), scale)
    assert np.all(zero["cor"] == 0.0)
    for uniform in (False, True):
        no = orc.prefill_forward_family(q, k, v, rho, scale, uniform=uniform, intercept=False)
        np.testing.assert_allclose(no["cor"], 1.0, rtol=1e-15, atol=0)
    # corr(2 rho) = 2 corr(rho): ||vbar - o(2 rho)|| = 2 ||vbar - o(rho)||
    two = orc.prefill_forward_family(q, k, v, 2 * rho, scale)
    np.testing.assert_allclose(two["cor"] * np.linalg.norm(two["o"], axis=-1),
                               2 * out["cor"] * np.linalg.norm(out["o"], axis=-1), rtol=1e-11)


def test_single_key_has_zero_cor_with_intercept():
    q, k, v, rho = _inputs(9, T=1)
    out = orc.prefill_forward_family(q, k, v, rho, 0.3)
    assert np.all(out["cor"] == 0.0)
    np.testing.assert_array_equal(out["o"][0, :, 0], np.repeat(v[0, :, 0], 2, axis=0))


@pytest.mark.parametrize("uniform,intercept", [(False, True), (True, True), (False, False), (True, False)])
def test_decode_family_equals_last_prefill_row(uniform, intercept):
    """Decode with ctx = t on the prefill's K/V and the query at row t-1 equals
    prefill row t-1 at every corner; GQA head mapping included."""
    q, k, v, rho = _inputs(10, B=2, Hq=4, Hkv=2, T=7, d=4)
    pre = orc.prefill_forward_family(q, k, v, rho, 0.5, uniform, intercept)
    ctx = np.array([7, 4])
    qd = np.stack([q[0, :, 6], q[1, :, 3]])
    rd = np.stack([rho[0, :, 6], rho[1, :, 3]])
    dec = orc.decode_forward_family(qd, rd, k, v, ctx, 0.5, uniform, intercept)
    for b, i in ((0, 6), (1, 3)):
        np.testing.assert_allclose(dec["o"][b], pre["o"][b, :, i], rtol=0, atol=1e-14)
        np.testing.assert_allclose(dec["lse"][b], pre["lse"][b, :, i], rtol=0, atol=1e-14)
        np.testing.assert_allclose(dec["cor"][b], pre["cor"][b, :, i], rtol=1e-14, atol=0)


# -- the stacked projection [W_Q; W_K; W_V; W_R] x ------------------------------

def test_projection_exact_integers_brute_force():
    """Small integers: every output element equals the integer dot product of
    its weight row and token, computed with Python ints."""
    g = _rng(20)
    B, T, D, Hq, Hkv, d = 2, 3, 5, 2, 1, 3
    x = g.integers(-4, 5, (B, T, D))
    W = g.integers(-4, 5, ((2 * Hq + 2 * Hkv) * d, D))
    q, k, v, rho = orc.project_qkvr(x.astype(np.float64), W.astype(np.float64), Hq, Hkv, d)
    blocks = [(q, Hq, 0), (k, Hkv, Hq * d), (v, Hkv, (Hq + Hkv) * d), (rho, Hq, (Hq + 2 * Hkv) * d)]
    for out, H, base in blocks:
        assert out.shape == (B, H, T, d)
        for b in range(B):
            for h in range(H):
                for t in range(T):
                    for j in range(d):
                        row = W[base + h * d + j]
                        assert out[b, h, t, j] == sum(int(row[c]) * int(x[b, t, c]) for c in range(D))


def test_projection_one_hot_tokens_place_weight_columns():
    """x_t = e_c(t) picks weight column c(t), so out[b,h,t,:] is the slice of
    that column belonging to (block, head): a placement probe for the layout."""
    B, T, Hq, Hkv, d = 2, 5, 4, 2, 4
    N = (2 * Hq + 2 * Hkv) * d
    D = B * T
    W = np.arange(N * D, dtype=np.float64).reshape(N, D)
    x = np.zeros((B, T, D))
    for b in range(B):
        for t in range(T):
            x[b, t, b * T + t] = 1.0
    q, k, v, rho = orc.project_qkvr(x, W, Hq, Hkv, d)
    for b in range(B):
        for t in range(T):
            col = W[:, b * T + t]
            np.testing.assert_array_equal(q[b, :, t].reshape(-1), col[: Hq * d])
            np.testing.assert_array_equal(k[b, :, t].reshape(-1), col[Hq * d: (Hq + Hkv) * d])
            np.testing.assert_array_equal(v[b, :, t].reshape(-1), col[(Hq + Hkv) * d: (Hq + 2 * Hkv) * d])
            np.testing.assert_array_equal(rho[b, :, t].reshape(-1), col[(Hq + 2 * Hkv) * d:])
