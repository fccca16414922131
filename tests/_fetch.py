"""Row and cache fetchers that feed the oracle's sampled forms.

The full-size GPU checks cannot afford the whole oracle, so they call
``prefill_rows``, ``decode_forward`` with a callable cache and
``prefill_backward_kv_rows`` / ``row_backward`` on sampled rows.  The slicing
those calls depend on (which KV head, which key prefix, which query row) lives
here, in one place, so that the CPU pins in ``test_oracle_sampling_pins.py``
check exactly the code the GPU tests run.  Nothing here does arithmetic: each
function only slices a generated workload and upcasts to float64.
"""

from __future__ import annotations

from oracle import plx_oracle as orc


def prefill_row_fetch(wl):
    """get_row(b, h, hk, i) -> (q_i, K[:i+1], V[:i+1], rho_i) of a prefill workload."""
    ten = wl.tensors

    def get_row(b, h, hk, i):
        return (ten["q"].f64_slice((b, h, i)), ten["k"].f64_slice((b, hk, slice(0, i + 1))),
                ten["v"].f64_slice((b, hk, slice(0, i + 1))), ten["rho"].f64_slice((b, h, i)))

    return get_row


def training_row_fetch(wl):
    """get_row(b, h, hk, i) -> (q_i, K[:i+1], V[:i+1], rho_i, dO_i) of a training workload."""
    ten = wl.tensors
    base = prefill_row_fetch(wl)

    def get_row(b, h, hk, i):
        return base(b, h, hk, i) + (ten["d_o"].f64_slice((b, h, i)),)

    return get_row


def prefill_oracle_rows(wl, rows):
    """Oracle (o, lse) of the prefill workload on the sampled rows (b, h, i)."""
    return orc.prefill_rows(prefill_row_fetch(wl), rows, wl.Hq, wl.Hkv, wl.scale)


def decode_kv_fetch(wl):
    """fetch(b, hk, n) -> (K[:n], V[:n]) of a decode workload's cache."""
    ten = wl.tensors

    def fetch(b, hk, n):
        return ten["k"].f64_slice((b, hk, slice(0, n))), ten["v"].f64_slice((b, hk, slice(0, n)))

    return fetch


def decode_oracle(wl, heads=None):
    """Oracle decode of a workload (q and rho stored [B, Hq, 1, d]) on the
    listed (b, h) heads, in the order given, through the callable cache form."""
    q = wl.tensors["q"].f64().reshape(wl.B, wl.Hq, wl.d)
    rho = wl.tensors["rho"].f64().reshape(wl.B, wl.Hq, wl.d)
    return orc.decode_forward(q, rho, decode_kv_fetch(wl), wl.Hkv, wl.ctx_len, wl.scale, heads=heads)


def training_oracle_rows(wl, rows):
    """Oracle dQ and drho rows of a training workload at the sampled (b, h, i)."""
    return orc.prefill_backward_rows(training_row_fetch(wl), rows, wl.Hq, wl.Hkv, wl.scale)


def training_oracle_keys(wl, keys):
    """Oracle dK and dV rows of a training workload at the sampled (b, hk, j)."""
    return orc.prefill_backward_kv_rows(training_row_fetch(wl), keys, wl.T, wl.Hq, wl.Hkv, wl.scale)
