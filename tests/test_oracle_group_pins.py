"""Pins of ``prefill_backward_group``, the closed-form dense backward the
full-size GPU checks use.

It must equal ``prefill_backward`` (reverse mode through the explicit
covariance, itself pinned to fp64 central differences and to torch autograd)
on inputs with GQA groups, a ragged number of rows per step and several
probe scales.  Mutants plant plausible slips in its source (a sign, a dropped
term, an off-by-one causal mask, c in place of r) and must fail that pin.
The backward is not given by the pages; both forms differentiate the
operator o = o^SA - Sigma_KV rho ("当注意力学会追问", section 1.3).
"""

import inspect
import textwrap

import numpy as np
import pytest

from oracle import plx_oracle as orc


def _case(seed, G=3, T=29, d=6, rho_std=0.8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((G, T, d))
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    rho = rho_std * rng.standard_normal((G, T, d))
    g = rng.standard_normal((G, T, d))
    return q, k, v, rho, g


def _reference(q, k, v, rho, g, scale):
    G = q.shape[0]
    # one batch, G query heads on a single KV head
    full = orc.prefill_backward(q[None], k[None, None], v[None, None], rho[None], g[None], scale)
    return {"dq": full["dq"][0], "drho": full["drho"][0], "dk": full["dk"][0, 0], "dv": full["dv"][0, 0]}


def _pin(fn):
    for seed, rps, rho_std in ((1, 7, 0.8), (2, 256, 0.1), (3, 1, 2.0)):
        q, k, v, rho, g = _case(seed, rho_std=rho_std)
        ref = _reference(q, k, v, rho, g, 0.45)
        got = fn(q, k, v, rho, g, 0.45, rows_per_step=rps)
        for n in ref:
            np.testing.assert_allclose(got[n], ref[n], rtol=0, atol=1e-11, err_msg=n)


def test_group_backward_equals_reverse_mode():
    _pin(orc.prefill_backward_group)


def test_group_magnitudes_bound_the_gradients():
    """Each gradient element is a sum of products whose absolute values sum
    to at most the reported magnitude."""
    q, k, v, rho, g = _case(4)
    out = orc.prefill_backward_group(q, k, v, rho, g, 0.45, magnitudes=True, rows_per_step=5)
    for n in ("dq", "drho", "dk", "dv"):
        assert np.all(np.abs(out[n]) <= out["m_" + n] * (1 + 1e-12)), n


MUTATIONS = [
    ("dR sign", "dr = -w * (a - dl[:, None])", "dr = w * (a - dl[:, None])"),
    ("dropped delta term", "+ dl[:, None] * (r - c[:, None])", "+ 0.0 * (r - c[:, None])"),
    ("mask excludes the diagonal", "np.arange(i1)[None, :] <= np.arange(i0, i1)[:, None]",
     "np.arange(i1)[None, :] < np.arange(i0, i1)[:, None] + (np.arange(i0, i1)[:, None] == 0)"),
    ("c in place of r in f", "f = 1.0 + c[:, None] - r", "f = 1.0 + c[:, None] - c[:, None]"),
    ("G from vbar", "Gi = np.sum(gh * o, axis=1)", "Gi = np.sum(gh * vbar, axis=1)"),
    ("dk without the probe part", "scale * (ds.T @ qh) + dr.T @ rh", "scale * (ds.T @ qh)"),
    ("dq unscaled", 'out["dq"][h, i0:i1] = scale * (ds @ K)', 'out["dq"][h, i0:i1] = ds @ K'),
]


def _mutant(old, new):
    src = textwrap.dedent(inspect.getsource(orc.prefill_backward_group))
    assert src.count(old) == 1, old
    ns = {"np": np}
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["prefill_backward_group"]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_group_pin_catches_mutant(name, old, new):
    fn = _mutant(old, new)
    with pytest.raises((AssertionError, FloatingPointError, ValueError)):
        with np.errstate(all="ignore"):
            _pin(fn)
