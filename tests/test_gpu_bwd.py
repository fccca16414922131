"""GPU parity of plx_bwd (dQ, dK, dV, drho) against the fp64 oracle."""

import numpy as np
import pytest

from oracle import plx_oracle as orc
from parallax_local_linear_plx_amd import inputs
from tests import _fetch
from tests._util import check_bf16, check_fp32_grad, say, to_device

pytestmark = pytest.mark.gpu


def _run(wl, do_scale=1.0):
    import torch

    from parallax_local_linear_plx_amd import plx_bwd, plx_fwd_prefill

    t = {n: to_device(x) for n, x in wl.tensors.items()}
    if do_scale != 1.0:
        t["d_o"] = t["d_o"] * do_scale  # a power of two: exact in the input dtype
    fwd = plx_fwd_prefill(t["q"], t["k"], t["v"], t["rho"], wl.scale, aux=True)
    nan = float("nan")
    grads = {
        "dq": torch.full(t["q"].shape, nan, dtype=torch.float32, device="cuda"),
        "dk": torch.full(t["k"].shape, nan, dtype=torch.float32, device="cuda"),
        "dv": torch.full(t["v"].shape, nan, dtype=torch.float32, device="cuda"),
        "drho": torch.full(t["rho"].shape, nan, dtype=torch.float32, device="cuda"),
    }
    plx_bwd(t["q"], t["k"], t["v"], t["rho"], t["d_o"], fwd["o"], fwd["lse"], fwd["c"], fwd["vbar"],
            wl.scale, grads=grads)
    torch.cuda.synchronize()
    return {n: x.cpu().numpy() for n, x in grads.items()}


def _oracle(wl):
    f = {n: x.f64() for n, x in wl.tensors.items()}
    return orc.prefill_backward(f["q"], f["k"], f["v"], f["rho"], f["d_o"], wl.scale)


def _magnitudes(wl, rho=None):
    """Per-element sums of the absolute products behind each gradient element
    (the scale of the fp32 summation bound), group by group."""
    f = {n: x.f64() for n, x in wl.tensors.items()}
    if rho is not None:
        f["rho"] = rho
    G = wl.Hq // wl.Hkv
    m = {n: np.empty(f[src].shape) for n, src in (("dq", "q"), ("drho", "rho"), ("dk", "k"), ("dv", "v"))}
    for b in range(wl.B):
        for hk in range(wl.Hkv):
            hs = slice(hk * G, (hk + 1) * G)
            out = orc.prefill_backward_group(f["q"][b, hs], f["k"][b, hk], f["v"][b, hk], f["rho"][b, hs],
                                             f["d_o"][b, hs], wl.scale, magnitudes=True)
            m["dq"][b, hs], m["drho"][b, hs] = out["m_dq"], out["m_drho"]
            m["dk"][b, hk], m["dv"][b, hk] = out["m_dk"], out["m_dv"]
    return m


def _n_terms(wl):
    # products per gradient element: one per (query head, row) or per key,
    # each made of d-long fp32 dot products
    return (wl.Hq // wl.Hkv) * wl.T + 2 * wl.d


@pytest.mark.parametrize("B,Hq,Hkv,T,d", [(1, 1, 1, 128, 64), (2, 4, 2, 150, 128), (1, 2, 1, 1, 64),
                                          (1, 3, 1, 97, 64)])
def test_fp32_gradients(gpu_lib, B, Hq, Hkv, T, d):
    say(f"case bwd fp32 B{B} Hq{Hq} Hkv{Hkv} T{T} d{d}")
    wl = inputs.make_prefill(B, Hq, Hkv, T, d, dtype="f32", seed=100 + T, rho_std=0.1, with_grad=True)
    got = _run(wl)
    ref = _oracle(wl)
    mag = _magnitudes(wl)
    for n in ("dq", "dk", "dv", "drho"):
        check_fp32_grad(got[n], ref[n], mag[n], _n_terms(wl), n)


@pytest.mark.parametrize("B,Hq,Hkv,T,d", [
    (1, 4, 2, 300, 128), (1, 2, 2, 129, 64), (2, 2, 1, 77, 128),
    (1, 1, 1, 1, 128),     # a single row
    (1, 8, 2, 513, 64),    # G = 4; several 128-key blocks and 64-row query tiles, ragged tail
    (1, 16, 1, 200, 128),  # G = 16: one KV head shared by sixteen query heads
    (1, 6, 2, 150, 64),    # G = 3
    (1, 2, 1, 17, 64),     # d = 64 waves hold two 16-row blocks: the second holds one row
    (1, 4, 2, 257, 64),    # one row past the 256 rows (and keys) of a d = 64 workgroup
])
def test_bf16_gradients(gpu_lib, B, Hq, Hkv, T, d):
    """Training-workload probe scale, rho ~ N(0, 0.1^2): the bf16 bars."""
    say(f"case bwd bf16 B{B} Hq{Hq} Hkv{Hkv} T{T} d{d}")
    wl = inputs.make_prefill(B, Hq, Hkv, T, d, dtype="bf16", seed=200 + T, with_grad=True)
    got = _run(wl)
    ref = _oracle(wl)
    for n in ("dq", "dk", "dv", "drho"):
        check_bf16(got[n], ref[n], n)


@pytest.mark.parametrize("T", [200, 513])
def test_bf16_gradients_projected_probe_scale(gpu_lib, T):
    """The prefill workload's probe rho = W_R x (~N(0,1) per component, ten
    times the training scale, |r| up to ~40): the same bf16 bars."""
    say(f"case bwd bf16 B1 Hq2 Hkv1 T{T} d128 projected rho")
    wl = inputs.make_prefill(1, 2, 1, T, 128, dtype="bf16", seed=400 + T - 200, rho_projected=True,
                             with_grad=True)
    got = _run(wl)
    ref = _oracle(wl)
    for n in ("dq", "dk", "dv", "drho"):
        check_bf16(got[n], ref[n], n)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_bf16_gradients_follow_the_scale_of_do(gpu_lib, d):
    """Every gradient is linear in dO.  dO x 2^-20 (the size of a loss averaged
    over about a million tokens, far below fp16's normal range) and dO x 2^12
    give exactly the unscaled run's gradients times 2^-20 and 2^12, and, back at
    unit scale, they meet the bf16 bars against the oracle."""
    B, Hq, Hkv, T = (1, 4, 2, 300) if d < 256 else (1, 4, 1, 129)
    say(f"case bwd bf16 dO scale B{B} Hq{Hq} Hkv{Hkv} T{T} d{d}")
    wl = inputs.make_prefill(B, Hq, Hkv, T, d, dtype="bf16", seed=700 + d, with_grad=True)
    base = _run(wl)
    ref = _oracle(wl)
    for e in (-20, 12):
        got = _run(wl, do_scale=2.0 ** e)
        for n in ("dq", "dk", "dv", "drho"):
            np.testing.assert_array_equal(got[n], base[n] * np.float32(2.0 ** e), err_msg=f"{n} at 2^{e}")
            check_bf16(got[n] * np.float32(2.0 ** -e), ref[n], f"{n} at 2^{e}")


def test_zero_probe_gradients_are_attention_gradients(gpu_lib):
    """rho = 0: dQ, dK, dV equal torch autograd of causal SDPA (fp64, CPU)."""
    import torch

    B, Hq, Hkv, T, d = 1, 2, 1, 70, 64
    wl = inputs.make_prefill(B, Hq, Hkv, T, d, dtype="f32", seed=300, with_grad=True)
    wl.tensors["rho"].data[...] = 0
    got = _run(wl)
    f = {n: torch.tensor(x.f64(), requires_grad=n in ("q", "k", "v")) for n, x in wl.tensors.items()}
    out = torch.nn.functional.scaled_dot_product_attention(
        f["q"], f["k"].repeat_interleave(Hq // Hkv, 1), f["v"].repeat_interleave(Hq // Hkv, 1),
        is_causal=True, scale=wl.scale)
    out.backward(f["d_o"])
    mag = _magnitudes(wl)
    for n, ref in (("dq", f["q"].grad.numpy()), ("dk", f["k"].grad.numpy()), ("dv", f["v"].grad.numpy())):
        check_fp32_grad(got[n], ref, mag[n], _n_terms(wl), n)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_upstream_gradient_gives_zero_gradients(gpu_lib, dtype):
    """dO = 0: every gradient is exactly zero (the bf16 path keeps its dO
    scale at 1 when max|dO| = 0, so nothing is divided by zero)."""
    wl = inputs.make_prefill(1, 4, 2, 150, 64, dtype=dtype, seed=302, with_grad=True)
    wl.tensors["d_o"].data[...] = 0
    got = _run(wl)
    for n in got:
        assert np.all(got[n] == 0), n


def test_repeat_runs_are_bitwise_identical(gpu_lib):
    wl = inputs.make_prefill(1, 2, 1, 260, 128, dtype="bf16", seed=301, with_grad=True)
    a = _run(wl)
    b = _run(wl)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def _group_oracle(wl, b, hk):
    """Dense closed-form oracle of one (b, kv head) group: every row of dQ /
    drho of its G query heads and every key of dK / dV."""
    G = wl.Hq // wl.Hkv
    ten = wl.tensors
    hs = slice(hk * G, (hk + 1) * G)
    return orc.prefill_backward_group(ten["q"].f64_slice((b, hs)), ten["k"].f64_slice((b, hk)),
                                      ten["v"].f64_slice((b, hk)), ten["rho"].f64_slice((b, hs)),
                                      ten["d_o"].f64_slice((b, hs)), wl.scale)


def _check_group(got, wl, b, hk):
    G = wl.Hq // wl.Hkv
    hs = slice(hk * G, (hk + 1) * G)
    ref = _group_oracle(wl, b, hk)
    # keys near the start are attended by thousands of rows: their gradients
    # are far above the bar, so a wrong or missing dK / dV cannot pass
    for n in ("dk", "dv"):
        assert np.abs(ref[n]).max() >= 10 * 2e-2, (n, float(np.abs(ref[n]).max()))
        check_bf16(got[n][b, hk], ref[n], f"{n} (b={b}, kv head {hk}, every key)")
    for n in ("dq", "drho"):
        check_bf16(got[n][b, hs], ref[n], f"{n} (b={b}, kv head {hk}, every row)")


def test_bf16_gradients_one_group_every_key_T1024(gpu_lib):
    """Every key and every row of one (b, kv head) group at T = 1024, G = 2."""
    say("case bwd bf16 B1 Hq2 Hkv1 T1024 d128 (every element)")
    wl = inputs.make_prefill(1, 2, 1, 1024, 128, dtype="bf16", seed=250, with_grad=True)
    got = _run(wl)
    _check_group(got, wl, 0, 0)


def test_bf16_training_full_size(gpu_lib):
    """Training step at full size (B=8, Hq=16, Hkv=8, T=4096, d=128), in the
    launch configuration the benchmark times: two whole (b, kv head) groups
    compared element by element (every key of dK / dV, every row of dQ /
    drho), sampled rows of the other groups, and two invariants over every
    key: shifting all keys by one vector leaves o unchanged
    (sum_j dK_j = 0); shifting all values by u shifts o by u
    (sum_j dV_j = sum over the group's rows of dO)."""
    say("case bwd bf16 B8 Hq16 Hkv8 T4096 d128")
    wl = inputs.bf16_training()
    got = _run(wl)
    for n in got:
        assert np.all(np.isfinite(got[n])), n
    T, Hq, Hkv = wl.T, wl.Hq, wl.Hkv
    for b, hk in ((0, 0), (7, 7)):
        _check_group(got, wl, b, hk)
    g = np.random.default_rng(5)
    rows = [(3, 4, 2000), (5, 9, 4095), (2, 13, 1)] + [
        (int(g.integers(8)), int(g.integers(16)), int(g.integers(4096))) for _ in range(9)]
    rdq, rdr = _fetch.training_oracle_rows(wl, rows)
    check_bf16(np.array([got["dq"][b, h, i] for b, h, i in rows]), rdq, "dq (sampled rows)")
    check_bf16(np.array([got["drho"][b, h, i] for b, h, i in rows]), rdr, "drho (sampled rows)")
    keys = [(5, 3, T - 1), (2, 6, T - 300)]
    dk, dv = _fetch.training_oracle_keys(wl, keys)
    check_bf16(np.array([got["dk"][b, hk, j] for b, hk, j in keys]), dk, "dk (sampled keys)")
    check_bf16(np.array([got["dv"][b, hk, j] for b, hk, j in keys]), dv, "dv (sampled keys)")
    # invariants over all keys
    sum_dk = got["dk"].astype(np.float64).sum(axis=2)
    scale_dk = np.abs(got["dk"]).astype(np.float64).sum(axis=2)
    assert np.all(np.abs(sum_dk) <= 2e-3 * scale_dk + 1e-2), float(np.max(np.abs(sum_dk)))
    sum_dv = got["dv"].astype(np.float64).sum(axis=2)
    d_o = wl.tensors["d_o"].f64().reshape(wl.B, Hkv, Hq // Hkv, T, wl.d).sum(axis=(2, 3))
    scale_dv = np.abs(got["dv"]).astype(np.float64).sum(axis=2)
    assert np.all(np.abs(sum_dv - d_o) <= 2e-3 * scale_dv + 1e-2), float(np.max(np.abs(sum_dv - d_o)))


@pytest.mark.parametrize("B,Hq,Hkv,T", [(1, 1, 1, 1), (1, 4, 1, 129), (1, 16, 1, 300), (2, 2, 2, 300)])
def test_bf16_gradients_head_dim_256(gpu_lib, B, Hq, Hkv, T):
    """d = 256: four waves (one per SIMD) on 32-row / 32-key tiles; G = 1, 4
    and 16, several tiles and a ragged tail, and the single-row case; every
    element of every group against the oracle."""
    say(f"case bwd bf16 d256 B{B} Hq{Hq} Hkv{Hkv} T{T}")
    wl = inputs.make_prefill(B, Hq, Hkv, T, 256, dtype="bf16", seed=260 + T + Hq, with_grad=True)
    got = _run(wl)
    G = Hq // Hkv
    for b in range(B):
        for hk in range(Hkv):
            ref = _group_oracle(wl, b, hk)
            hs = slice(hk * G, (hk + 1) * G)
            for n in ("dk", "dv"):
                check_bf16(got[n][b, hk], ref[n], f"{n} (b={b}, kv head {hk})")
            for n in ("dq", "drho"):
                check_bf16(got[n][b, hs], ref[n], f"{n} (b={b}, kv head {hk})")
