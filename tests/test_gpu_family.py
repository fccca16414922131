"""GPU parity of the family corners and the correction-to-output ratio
(plx_fwd_prefill_ex, plx_decode_ex) against the fp64 oracle, through the C ABI.

o and the softmax-attention mean vbar are held to the usual bars.  COR is a
ratio of norms, so its bar is propagated from the errors the same call makes
on o and vbar: the kernel's correction is vbar - o up to fp32 rounding (-o
without an intercept), hence
  |COR - COR_ref| <= (||d corr|| + COR_ref ||d o||) / (||o_ref|| - ||d o||) + slack
with ||d corr|| <= ||d vbar|| + ||d o|| and slack a few hundred fp32 ulps of
the terms the kernel combines.  Rows whose ||o_ref|| is within 2 ||d o|| of
zero (COR ill-conditioned) only need a finite, non-negative value.
"""

import numpy as np
import pytest

from oracle import plx_oracle as orc
from parallax_local_linear_plx_amd import inputs
from tests._util import LSE_ABS, check_bf16, check_fp32, say, to_device

pytestmark = pytest.mark.gpu

UNIFORM, NO_ICPT = 1, 2
FLAGS = [0, UNIFORM, NO_ICPT, UNIFORM | NO_ICPT]


def check_cor(cor, cor_ref, o, o_ref, vb, vb_ref, intercept, what):
    cor = np.asarray(cor, np.float64).reshape(-1)
    cor_ref = np.asarray(cor_ref, np.float64).reshape(-1)
    d = o_ref.shape[-1]
    o = o.reshape(-1, d).astype(np.float64)
    o_ref = o_ref.reshape(-1, d)
    vb = vb.reshape(-1, d).astype(np.float64)
    vb_ref = vb_ref.reshape(-1, d)
    e_o = np.linalg.norm(o - o_ref, axis=1)
    e_v = np.linalg.norm(vb - vb_ref, axis=1)
    n_o = np.linalg.norm(o_ref, axis=1)
    n_v = np.linalg.norm(vb_ref, axis=1)
    e_c = e_o + e_v if intercept else e_o
    ok_rows = n_o > 2 * e_o + 1e-30
    assert np.all(np.isfinite(cor[ok_rows])) and np.all(cor[ok_rows] >= 0), f"{what}: bad COR values"
    slack = 1e-5 * np.maximum(cor_ref, 1.0) * (n_v + n_o) / np.where(ok_rows, n_o, 1.0)
    tol = (e_c + cor_ref * e_o) / np.where(ok_rows, n_o - e_o, 1.0) + slack
    err = np.abs(cor - cor_ref)
    bad = ok_rows & ~(err <= tol)
    say(f"  {what}: max |dCOR| {err[ok_rows].max():.3e}, max |dCOR|/bound "
        f"{(err[ok_rows] / tol[ok_rows]).max():.3f}, COR range [{cor_ref.min():.3g}, {cor_ref.max():.3g}]")
    assert not bad.any(), f"{what}: {bad.sum()} rows outside the propagated bound"
    if not intercept:
        np.testing.assert_allclose(cor[ok_rows], 1.0, rtol=0, atol=tol[ok_rows].max())


def _check_out(got, ref, what, dtype):
    if dtype == "f32":
        check_fp32(got, ref, what)
    else:
        check_bf16(got, ref, what)


# -- prefill -------------------------------------------------------------------

def _prefill(wl, flags, t=None):
    import torch

    from parallax_local_linear_plx_amd import plx_fwd_prefill_ex

    if t is None:
        t = {n: to_device(x) for n, x in wl.tensors.items()}
    out = plx_fwd_prefill_ex(t["q"], t["k"], t["v"], t["rho"], wl.scale, flags=flags, aux=True)
    torch.cuda.synchronize()
    return {n: x.cpu().numpy() for n, x in out.items()}, t


@pytest.mark.parametrize("dtype,B,Hq,Hkv,T,d", [
    ("f32", 1, 2, 1, 130, 64),
    ("f32", 1, 2, 2, 67, 128),
    ("bf16", 1, 4, 2, 300, 128),
    ("bf16", 2, 2, 1, 161, 64),
    ("bf16", 1, 2, 1, 150, 256),
])
@pytest.mark.parametrize("flags", FLAGS)
def test_prefill_family_against_oracle(gpu_lib, dtype, B, Hq, Hkv, T, d, flags):
    uniform, intercept = bool(flags & UNIFORM), not (flags & NO_ICPT)
    say(f"case prefill {dtype} B{B} Hq{Hq} Hkv{Hkv} T{T} d{d} flags={flags}")
    wl = inputs.make_prefill(B, Hq, Hkv, T, d, dtype=dtype, seed=70 + T + flags, rho_std=0.5)
    got, _ = _prefill(wl, flags)
    f = {n: x.f64() for n, x in wl.tensors.items()}
    ref = orc.prefill_forward_family(f["q"], f["k"], f["v"], f["rho"], wl.scale, uniform, intercept)
    # vbar: the weighted mean the kernel used, against the oracle's mean at the
    # same corner (the intercept corner's output with rho = 0)
    vb_ref = orc.prefill_forward_family(f["q"], f["k"], f["v"], np.zeros_like(f["rho"]), wl.scale,
                                        uniform, True)["o"]
    _check_out(got["o"], ref["o"], "o", dtype)
    _check_out(got["vbar"], vb_ref, "vbar", dtype)
    assert np.max(np.abs(got["lse"] - ref["lse"])) <= LSE_ABS
    check_cor(got["cor"], ref["cor"], got["o"], ref["o"], got["vbar"], vb_ref, intercept, "cor")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_ex_default_corner_is_plx_fwd_prefill_bitwise(gpu_lib, dtype):
    import torch

    from parallax_local_linear_plx_amd import plx_fwd_prefill

    wl = inputs.make_prefill(1, 4, 2, 257, 128, dtype=dtype, seed=81)
    got, t = _prefill(wl, 0)
    base = plx_fwd_prefill(t["q"], t["k"], t["v"], t["rho"], wl.scale, aux=True)
    torch.cuda.synchronize()
    for n in ("o", "lse", "c", "vbar"):
        assert np.array_equal(base[n].cpu().numpy(), got[n]), n


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_uniform_weights_key_count_is_exact(gpu_lib, dtype):
    """With uniform weights exp(LSE_i) is the key count i + 1 exactly, for any q."""
    wl = inputs.make_prefill(1, 2, 1, 700, 64, dtype=dtype, seed=82)
    got, _ = _prefill(wl, UNIFORM)
    n = np.rint(np.exp(got["lse"].astype(np.float64))).astype(np.int64)
    assert np.array_equal(n, np.broadcast_to(np.arange(1, 701), n.shape))


def test_zero_probe_has_zero_cor_and_single_key_row(gpu_lib):
    wl = inputs.make_prefill(1, 2, 1, 40, 128, dtype="bf16", seed=83)
    wl.tensors["rho"].data[...] = 0
    got, _ = _prefill(wl, 0)
    assert np.all(got["cor"] == 0.0)
    got, _ = _prefill(inputs.make_prefill(1, 2, 1, 1, 64, dtype="f32", seed=84), 0)
    assert np.all(got["cor"] < 1e-6)


# -- decode --------------------------------------------------------------------

def _decode(wl, flags, num_splits, rho_zero=False):
    import torch

    from parallax_local_linear_plx_amd import plx_decode_ex

    t = {n: to_device(x) for n, x in wl.tensors.items()}
    q = t["q"].reshape(wl.B, wl.Hq, wl.d)
    rho = t["rho"].reshape(wl.B, wl.Hq, wl.d)
    if rho_zero:
        rho = torch.zeros_like(rho)
    ctx = torch.from_numpy(wl.ctx_len.astype(np.int32)).cuda()
    out = plx_decode_ex(q, rho, t["k"], t["v"], ctx, wl.scale, flags=flags, num_splits=num_splits)
    torch.cuda.synchronize()
    return {n: x.cpu().numpy() for n, x in out.items()}


@pytest.mark.parametrize("dtype,num_splits,G,d", [
    ("bf16", 0, 2, 128),
    ("bf16", 3, 16, 64),
    ("f32", 0, 4, 128),
    ("f32", 2, 1, 64),
])
@pytest.mark.parametrize("flags", FLAGS)
def test_decode_family_against_oracle(gpu_lib, dtype, num_splits, G, d, flags):
    uniform, intercept = bool(flags & UNIFORM), not (flags & NO_ICPT)
    say(f"case decode {dtype} splits={num_splits} G{G} d{d} flags={flags}")
    wl = inputs.make_decode(3, 2 * G, 2, d, 0, S_max=900, dtype=dtype, seed=90 + G + flags,
                            ctx_list=[900, 1, 417], rho_std=0.5)
    got = _decode(wl, flags, num_splits)
    # the kernel's own weighted mean: rho = 0 leaves the score columns, P and
    # the value products unchanged and makes o = O / l
    vb = _decode(wl, flags & UNIFORM, num_splits, rho_zero=True)["o"]
    q = wl.tensors["q"].f64().reshape(wl.B, wl.Hq, wl.d)
    rho = wl.tensors["rho"].f64().reshape(wl.B, wl.Hq, wl.d)
    k, v = wl.tensors["k"].f64(), wl.tensors["v"].f64()
    ref = orc.decode_forward_family(q, rho, k, v, wl.ctx_len, wl.scale, uniform, intercept)
    vb_ref = orc.decode_forward_family(q, np.zeros_like(rho), k, v, wl.ctx_len, wl.scale, uniform,
                                       True)["o"]
    _check_out(got["o"], ref["o"], "o", dtype)
    _check_out(vb, vb_ref, "vbar", dtype)
    assert np.max(np.abs(got["lse"] - ref["lse"])) <= LSE_ABS
    check_cor(got["cor"], ref["cor"], got["o"], ref["o"], vb, vb_ref, intercept, "cor")


def test_decode_invalid_length_gives_nan_cor(gpu_lib):
    wl = inputs.make_decode(2, 4, 2, 128, 0, S_max=256, dtype="bf16", seed=95, ctx_list=[256, 100])
    wl.ctx_len = np.array([256, 0], np.int32)
    got = _decode(wl, 0, 0)
    assert np.all(np.isnan(got["cor"][1])) and np.all(np.isfinite(got["cor"][0]))
    assert np.all(np.isnan(got["o"][1]))
