"""GPU parity of plx_qkvr_proj (the stacked [W_Q; W_K; W_V; W_R] projection in
front of the operator) against the fp64 oracle, through the C ABI.

Bar: every output is the bf16 rounding (to nearest, ties to even) of an fp32
accumulation, so |got - ref| <= 2^-8 |ref| + 4 D 2^-24 sum_c |x_c w_c| per
element (half a bf16 ulp of the result plus a worst-case fp32 summation
bound over D terms); the mean error must also stay under 2^-9 mean |ref|.
Integer inputs whose results are exact in bf16, and one-hot tokens, must come
out bit-exact.
"""

import numpy as np
import pytest

from oracle import plx_oracle as orc
from parallax_local_linear_plx_amd import inputs
from tests._util import say, to_device

pytestmark = pytest.mark.gpu


def _run(x_bits, w_bits, Hq, Hkv, d):
    import torch

    from parallax_local_linear_plx_amd import plx_qkvr_proj

    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()
    w = torch.from_numpy(np.ascontiguousarray(w_bits).view(np.int16)).view(torch.bfloat16).cuda()
    out = plx_qkvr_proj(x, w, Hq, Hkv, d)
    torch.cuda.synchronize()
    return {n: t.float().cpu().numpy().astype(np.float64) for n, t in out.items()}


def _check(got, ref, bound, what):
    err = np.abs(got - ref)
    tol = 2.0 ** -8 * np.abs(ref) + bound
    worst = float(np.max(err / tol)) if err.size else 0.0
    say(f"  {what}: max |d| {err.max():.3e}, max |d|/bound {worst:.3f}, mean |d| {err.mean():.3e}")
    assert np.all(err <= tol), f"{what}: {int(np.sum(err > tol))} elements outside the bound"
    assert err.mean() <= 2.0 ** -9 * np.abs(ref).mean() + 1e-30, f"{what}: mean error too large"


def _bounds(x, w, Hq, Hkv, d):
    """4 D 2^-24 sum_c |x_c w_c| per output element, in the output layout."""
    D = x.shape[-1]
    return tuple(4 * D * 2.0 ** -24 * a for a in orc.project_qkvr(np.abs(x), np.abs(w), Hq, Hkv, d))


@pytest.mark.parametrize("B,T,D,Hq,Hkv,d", [
    (2, 37, 128, 4, 2, 64),     # ragged token count, N = 768 (three feature tiles)
    (1, 300, 256, 2, 1, 64),    # N = 384: a half-filled feature tile
    (3, 100, 64, 2, 2, 128),    # one 64-deep reduction tile
    (1, 513, 1024, 4, 1, 128),  # the layer width of the projected-probe workload
    (1, 100, 128, 2, 1, 256),   # d = 256: a head spans both feature halves of a tile
])
def test_projection_against_oracle(gpu_lib, B, T, D, Hq, Hkv, d):
    say(f"case proj B{B} T{T} D{D} Hq{Hq} Hkv{Hkv} d{d}")
    wl = inputs.make_projection(B, T, D, Hq, Hkv, d, seed=100 + T)
    x, w = wl.tensors["x"], wl.tensors["w"]
    got = _run(x.data, w.data, Hq, Hkv, d)
    ref = orc.project_qkvr(x.f64(), w.f64(), Hq, Hkv, d)
    bnd = _bounds(x.f64(), w.f64(), Hq, Hkv, d)
    for n, r, bd in zip(("q", "k", "v", "rho"), ref, bnd):
        assert got[n].shape == r.shape
        _check(got[n], r, bd, n)


def test_projection_integer_inputs_are_exact(gpu_lib):
    """|x|, |w| <= 2 and D = 64: every dot product is an integer of magnitude
    <= 256, exact in fp32 and in bf16, so the outputs must match exactly."""
    B, T, D, Hq, Hkv, d = 2, 41, 64, 2, 1, 128
    g = np.random.default_rng(7)
    x = g.integers(-2, 3, (B, T, D)).astype(np.float32)
    w = g.integers(-2, 3, ((2 * Hq + 2 * Hkv) * d, D)).astype(np.float32)
    got = _run(inputs.bf16_round_bits(x), inputs.bf16_round_bits(w), Hq, Hkv, d)
    ref = orc.project_qkvr(x.astype(np.float64), w.astype(np.float64), Hq, Hkv, d)
    for n, r in zip(("q", "k", "v", "rho"), ref):
        assert np.array_equal(got[n], r), n


def test_projection_one_hot_tokens_place_weight_columns(gpu_lib):
    """Token (b, t) = e_c selects weight column c: a bit-exact placement probe
    of the [B, H, T, d] layout of all four outputs."""
    B, T, Hq, Hkv, d = 2, 96, 4, 2, 64
    D = B * T
    D = (D + 63) // 64 * 64
    N = (2 * Hq + 2 * Hkv) * d
    w = inputs.bf16_round_bits(np.random.default_rng(8).standard_normal((N, D)).astype(np.float32))
    x = np.zeros((B, T, D), np.float32)
    for b in range(B):
        for t in range(T):
            x[b, t, b * T + t] = 1.0
    got = _run(inputs.bf16_round_bits(x), w, Hq, Hkv, d)
    ref = orc.project_qkvr(x.astype(np.float64), inputs.bf16_bits_to_f32(w).astype(np.float64), Hq, Hkv, d)
    for n, r in zip(("q", "k", "v", "rho"), ref):
        assert np.array_equal(got[n], r), n


def test_projection_full_size_sampled_tokens(gpu_lib):
    """B=4, T=4096, D=1024, Hq=16, Hkv=8, d=128 (the projected-probe prefill's
    layer), the launch the benchmark times; sampled tokens against the oracle."""
    say("case proj B4 T4096 D1024 Hq16 Hkv8 d128 (sampled tokens)")
    B, T, D, Hq, Hkv, d = 4, 4096, 1024, 16, 8, 128
    wl = inputs.make_projection(B, T, D, Hq, Hkv, d, seed=6)
    x, w = wl.tensors["x"], wl.tensors["w"]
    got = _run(x.data, w.data, Hq, Hkv, d)
    for n in got:
        assert np.all(np.isfinite(got[n])), n
    g = np.random.default_rng(9)
    toks = [(0, 0), (3, 4095), (1, 255), (1, 256), (2, 2047)]
    toks += [(int(g.integers(B)), int(g.integers(T))) for _ in range(27)]
    wf = w.f64()
    for b, t in toks:
        xs = x.f64_slice((b, slice(t, t + 1)))[None]
        ref = orc.project_qkvr(xs, wf, Hq, Hkv, d)
        bnd = _bounds(xs, wf, Hq, Hkv, d)
        for n, r, bd in zip(("q", "k", "v", "rho"), ref, bnd):
            gv = got[n][b:b + 1, :, t:t + 1]
            err = np.abs(gv - r)
            assert np.all(err <= 2.0 ** -8 * np.abs(r) + bd), (n, b, t, float(err.max()))
