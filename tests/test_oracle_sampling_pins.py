"""Pins of the oracle's sampled forms, which every full-size GPU check uses.

``prefill_rows``, ``decode_forward`` with a callable cache and a ``heads``
list, ``prefill_backward_rows`` and ``prefill_backward_kv_rows`` are checked
here against the whole-array forms (themselves pinned in
``test_oracle_pins.py``), through the same fetch helpers (``tests/_fetch.py``)
the GPU tests call, on generated workloads with B > 1 and GQA groups G > 1.
The operator every path computes is o = o^SA - Sigma_KV rho ("当注意力学会追问",
section 1.3; "Riepilogo Tecnico: Parallax", section "Meccanismo Principale").

Each mutant plants a plausible mistake in those paths (the interleaved KV-head
mapping h % Hkv, a key prefix one row short, a ``heads`` list returned in
sorted order instead of the order asked for) and must make a pin fail.
"""

import numpy as np
import pytest

from oracle import plx_oracle as orc
from parallax_local_linear_plx_amd import inputs
from tests import _fetch


def _prefill_wl(dtype="bf16"):
    return inputs.make_prefill(2, 6, 2, 23, 8, dtype=dtype, seed=901, rho_std=0.7, with_grad=True)


def _rows(wl):
    g = np.random.default_rng(3)
    rows = [(0, 0, 0), (1, 5, wl.T - 1), (1, 3, 11), (0, 2, 1)]
    rows += [(int(g.integers(wl.B)), int(g.integers(wl.Hq)), int(g.integers(wl.T))) for _ in range(12)]
    return rows


def _expanded(wl):
    """The workload's arrays with K and V repeated per query head (MHA form),
    so the whole-array reference needs no head mapping at all."""
    f = {n: x.f64() for n, x in wl.tensors.items()}
    G = wl.Hq // wl.Hkv
    f["k"] = np.repeat(f["k"], G, axis=1)
    f["v"] = np.repeat(f["v"], G, axis=1)
    return f, G


def _full_forward(wl):
    f, _ = _expanded(wl)
    return orc.prefill_forward(f["q"], f["k"], f["v"], f["rho"], wl.scale)


def _full_backward(wl):
    f, G = _expanded(wl)
    out = orc.prefill_backward(f["q"], f["k"], f["v"], f["rho"], f["d_o"], wl.scale)
    for n in ("dk", "dv"):
        x = out[n]
        out[n] = x.reshape(x.shape[0], wl.Hkv, G, *x.shape[2:]).sum(axis=2)
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_rows_equal_full_prefill(dtype):
    wl = _prefill_wl(dtype)
    full = _full_forward(wl)
    rows = _rows(wl)
    o, lse = _fetch.prefill_oracle_rows(wl, rows)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_array_equal(o[n], full["o"][b, h, i])
        np.testing.assert_array_equal(lse[n], full["lse"][b, h, i])


def test_training_rows_equal_full_backward():
    wl = _prefill_wl()
    full = _full_backward(wl)
    rows = _rows(wl)
    dq, dr = _fetch.training_oracle_rows(wl, rows)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(dq[n], full["dq"][b, h, i], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dr[n], full["drho"][b, h, i], rtol=0, atol=1e-12)
    keys = [(0, 0, 0), (1, 1, wl.T - 1), (1, 0, 9), (0, 1, 17)]
    dk, dv = _fetch.training_oracle_keys(wl, keys)
    for n, (b, hk, j) in enumerate(keys):
        np.testing.assert_allclose(dk[n], full["dk"][b, hk, j], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv[n], full["dv"][b, hk, j], rtol=0, atol=1e-12)


def _decode_wl():
    return inputs.make_decode(3, 8, 2, 8, 0, S_max=40, dtype="bf16", seed=902, rho_std=0.7,
                              ctx_list=[40, 1, 17])


def test_decode_callable_heads_equal_array_form():
    """The callable-cache form on an unsorted ``heads`` list returns the heads
    in the order asked for, each equal to the array form's value."""
    wl = _decode_wl()
    q = wl.tensors["q"].f64().reshape(wl.B, wl.Hq, wl.d)
    rho = wl.tensors["rho"].f64().reshape(wl.B, wl.Hq, wl.d)
    # the array form on the cache repeated per query head (no head mapping),
    # its NaN padding rows past each sequence's length never read
    G = wl.Hq // wl.Hkv
    k = np.repeat(wl.tensors["k"].f64(), G, axis=1)
    v = np.repeat(wl.tensors["v"].f64(), G, axis=1)
    full = orc.decode_forward(q, rho, k, v, wl.ctx_len, wl.scale)
    o_full = full["o"].reshape(wl.B, wl.Hq, wl.d)
    lse_full = full["lse"].reshape(wl.B, wl.Hq)
    heads = [(2, 7), (0, 3), (1, 0), (2, 0), (0, 4), (1, 6), (0, 0)]
    part = _fetch.decode_oracle(wl, heads)
    assert part["heads"] == heads
    for n, (b, h) in enumerate(heads):
        np.testing.assert_array_equal(part["o"][n], o_full[b, h])
        np.testing.assert_array_equal(part["lse"][n], lse_full[b, h])
    # and every head of the callable form, in the default order
    every = _fetch.decode_oracle(wl)
    np.testing.assert_array_equal(every["o"].reshape(wl.B, wl.Hq, wl.d), o_full)


def test_decode_callable_matches_last_prefill_row():
    """Decode through the fetch helper on a prefill workload's keys equals that
    prefill's row ctx - 1, for each sequence's own ctx."""
    wl = _prefill_wl()
    full = _full_forward(wl)
    ctx = np.array([wl.T, 9], np.int32)
    dec = inputs.Workload("decode-of-prefill", wl.dtype, wl.B, wl.Hq, wl.Hkv, wl.d, wl.scale,
                          S_max=wl.T)
    dec.ctx_len = ctx
    dec.tensors["k"], dec.tensors["v"] = wl.tensors["k"], wl.tensors["v"]
    qb = wl.tensors["q"].data[np.arange(wl.B), :, ctx - 1]
    rb = wl.tensors["rho"].data[np.arange(wl.B), :, ctx - 1]
    dec.tensors["q"] = inputs.Tensor(wl.dtype, qb[:, :, None, :])
    dec.tensors["rho"] = inputs.Tensor(wl.dtype, rb[:, :, None, :])
    got = _fetch.decode_oracle(dec)["o"].reshape(wl.B, wl.Hq, wl.d)
    for b in range(wl.B):
        np.testing.assert_allclose(got[b], full["o"][b, :, ctx[b] - 1], rtol=0, atol=1e-13)


# -- mutants ------------------------------------------------------------------

def _mut_interleaved_heads(h, Hq, Hkv):
    return h % Hkv


def _mut_short_prefix(wl):
    ten = wl.tensors

    def get_row(b, h, hk, i):
        n = max(i, 1)
        return (ten["q"].f64_slice((b, h, i)), ten["k"].f64_slice((b, hk, slice(0, n))),
                ten["v"].f64_slice((b, hk, slice(0, n))), ten["rho"].f64_slice((b, h, i)))

    return get_row


def _mut_short_cache(wl):
    ten = wl.tensors

    def fetch(b, hk, n):
        m = max(n - 1, 1)
        return ten["k"].f64_slice((b, hk, slice(0, m))), ten["v"].f64_slice((b, hk, slice(0, m)))

    return fetch


_real_decode_forward = orc.decode_forward


def _mut_sorted_heads(q, rho, k_cache, v_cache, ctx_len, scale, heads=None):
    return _real_decode_forward(q, rho, k_cache, v_cache, ctx_len, scale,
                                heads=None if heads is None else sorted(heads))


SAMPLING_PINS = [
    lambda: test_prefill_rows_equal_full_prefill("bf16"),
    test_training_rows_equal_full_backward,
    test_decode_callable_heads_equal_array_form,
    test_decode_callable_matches_last_prefill_row,
]

MUTANTS = [
    ("interleaved_kv_heads", lambda mp: mp.setattr(orc, "_kv_head", _mut_interleaved_heads)),
    ("short_key_prefix", lambda mp: mp.setattr(_fetch, "prefill_row_fetch", _mut_short_prefix)),
    ("short_cache", lambda mp: mp.setattr(_fetch, "decode_kv_fetch", _mut_short_cache)),
    ("sorted_heads", lambda mp: mp.setattr(orc, "decode_forward", _mut_sorted_heads)),
]


@pytest.mark.parametrize("name,plant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_sampling_pins_catch_mutant(name, plant, monkeypatch):
    plant(monkeypatch)
    failed = 0
    for pin in SAMPLING_PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            failed += 1
    assert failed >= 1, f"mutant {name} passed every sampling pin"


def test_unmutated_sampling_paths_pass_every_pin():
    for pin in SAMPLING_PINS:
        pin()
