"""GPU parity of plx_fwd_prefill against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest

from oracle import plx_oracle as orc
from parallax_local_linear_plx_amd import inputs
from tests import _fetch
from tests._util import LSE_ABS, check_bf16, check_fp32, say, to_device

pytestmark = pytest.mark.gpu


def _run(wl, aux=False):
    import torch

    from parallax_local_linear_plx_amd import plx_fwd_prefill

    t = {n: to_device(x) for n, x in wl.tensors.items()}
    o = torch.full((wl.B, wl.Hq, wl.T, wl.d), float("nan"), dtype=torch.float32, device="cuda")
    out = plx_fwd_prefill(t["q"], t["k"], t["v"], t["rho"], wl.scale, o=o, aux=aux)
    torch.cuda.synchronize()
    return {n: x.cpu().numpy() for n, x in out.items()}


def _oracle(wl):
    f = {n: x.f64() for n, x in wl.tensors.items()}
    return orc.prefill_forward(f["q"], f["k"], f["v"], f["rho"], wl.scale)


def test_fp32_single_head_T128_d64(gpu_lib):
    wl = inputs.fp32_single_head()
    say("case fp32 B1 H1 T128 d64")
    got = _run(wl)
    ref = _oracle(wl)
    e = check_fp32(got["o"], ref["o"], "o")
    check_fp32(got["lse"], ref["lse"], "lse")
    say(f"  max |d| {e:.2e}")


@pytest.mark.parametrize("B,Hq,Hkv,T,d", [(2, 4, 2, 200, 128), (1, 2, 1, 1, 64), (1, 3, 3, 129, 64)])
def test_fp32_gqa_ragged(gpu_lib, B, Hq, Hkv, T, d):
    say(f"case fp32 B{B} Hq{Hq} Hkv{Hkv} T{T} d{d}")
    wl = inputs.make_prefill(B, Hq, Hkv, T, d, dtype="f32", seed=31 + T, rho_std=0.5)
    got = _run(wl, aux=True)
    ref = _oracle(wl)
    check_fp32(got["o"], ref["o"], "o")
    check_fp32(got["lse"], ref["lse"], "lse")
    check_fp32(got["vbar"], ref["o_sa"], "vbar")
    check_fp32(got["c"], ref["c"], "c")


@pytest.mark.parametrize("B,Hq,Hkv,T,d,proj", [
    (1, 4, 2, 333, 128, True),
    (1, 2, 2, 129, 64, True),
    (2, 2, 1, 64, 128, False),
    (1, 1, 1, 1, 128, True),
    (1, 6, 2, 150, 128, False),  # three query heads per KV head
    (1, 1, 1, 1, 64, False),     # d = 64 waves hold two 16-row blocks: a single row
    (1, 2, 1, 17, 64, True),     # the second block of a wave holds one row
    (1, 4, 2, 257, 64, False),   # one row past the 256 rows of a d = 64 workgroup
])
def test_bf16_against_oracle(gpu_lib, B, Hq, Hkv, T, d, proj):
    say(f"case bf16 B{B} Hq{Hq} Hkv{Hkv} T{T} d{d} projected-rho={proj}")
    wl = inputs.make_prefill(B, Hq, Hkv, T, d, dtype="bf16", seed=41 + T, rho_projected=proj)
    got = _run(wl, aux=True)
    ref = _oracle(wl)
    check_bf16(got["o"], ref["o"], "o")
    check_bf16(got["vbar"], ref["o_sa"], "vbar")
    assert np.max(np.abs(got["lse"] - ref["lse"])) <= LSE_ABS
    # the auxiliary c = kbar . rho the backward consumes: from unrounded sums,
    # so it is accurate to fp32 rounding of sum p r / sum p, |r| up to ~50
    err_c = np.abs(got["c"] - ref["c"])
    say(f"  c: max-abs {err_c.max():.3e}  max|ref| {np.abs(ref['c']).max():.3e}")
    assert np.all(err_c <= 1e-4 * np.maximum(np.abs(ref["c"]), 1.0)), float(err_c.max())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_key_count_probe_is_exact(gpu_lib, dtype):
    """q = 0 gives p = 1 for every visible key, so exp(LSE_i) must round to
    i + 1 exactly: the causal key set of every row, the ragged tail included."""
    B, Hq, Hkv, T, d = 1, 2, 1, 1000, 128
    wl = inputs.make_prefill(B, Hq, Hkv, T, d, dtype=dtype, seed=5)
    wl.tensors["q"].data[...] = 0
    got = _run(wl)
    n = np.rint(np.exp(got["lse"].astype(np.float64))).astype(np.int64)
    want = np.broadcast_to(np.arange(1, T + 1), n.shape)
    assert np.array_equal(n, want)


def test_head_and_batch_mapping_probe(gpu_lib):
    """V constant per (b, kv head) with an integer code: o must round to the
    code of KV head h // (Hq / Hkv) of the same batch, for every row."""
    B, Hq, Hkv, T, d = 3, 8, 2, 77, 64
    wl = inputs.make_prefill(B, Hq, Hkv, T, d, dtype="bf16", seed=6)
    codes = np.arange(B * Hkv).reshape(B, Hkv) + 1
    v = np.zeros((B, Hkv, T, d), np.float32)
    v[...] = codes[:, :, None, None]
    wl.tensors["v"].data[...] = inputs.bf16_round_bits(v)
    got = _run(wl)
    want = np.repeat(codes, Hq // Hkv, axis=1)[:, :, None, None]
    assert np.array_equal(np.rint(got["o"]), np.broadcast_to(want, got["o"].shape))


def test_repeat_runs_are_bitwise_identical(gpu_lib):
    wl = inputs.make_prefill(1, 2, 1, 300, 128, dtype="bf16", seed=8, rho_projected=True)
    a = _run(wl)
    b = _run(wl)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])


def test_bf16_prefill_full_size_sampled_rows(gpu_lib):
    """The GQA prefill at its full size (B=4, Hq=16, Hkv=8, T=4096, d=128,
    rho = W_R x) in the launch configuration the benchmark times; sampled rows
    are checked against the oracle row by row."""
    say("case bf16 prefill B4 Hq16 Hkv8 T4096 d128 (sampled rows)")
    wl = inputs.bf16_prefill()
    got = _run(wl)
    assert np.all(np.isfinite(got["o"])), "unwritten or non-finite output"
    g = np.random.default_rng(99)
    rows = [(0, 0, 0), (0, 0, 1), (3, 15, 4095), (1, 7, 4094), (2, 8, 2048), (0, 1, 127), (0, 1, 128)]
    rows += [(int(g.integers(4)), int(g.integers(16)), int(g.integers(4096))) for _ in range(40)]
    T = wl.T
    ref_o, ref_lse = _fetch.prefill_oracle_rows(wl, rows)
    got_o = np.array([got["o"][b, h, i] for b, h, i in rows])
    got_lse = np.array([got["lse"][b, h, i] for b, h, i in rows])
    check_bf16(got_o, ref_o, "o (sampled rows)")
    assert np.max(np.abs(got_lse - ref_lse)) <= LSE_ABS
    assert T == 4096


@pytest.mark.parametrize("B,Hq,Hkv,T", [(1, 2, 1, 200), (1, 4, 2, 129), (2, 1, 1, 64), (1, 1, 1, 1)])
def test_bf16_head_dim_256_against_oracle(gpu_lib, B, Hq, Hkv, T):
    """d = 256: four waves of 16 rows, 64-key tiles; several tiles and a
    ragged tail, GQA, and the single-key row."""
    say(f"case bf16 d256 B{B} Hq{Hq} Hkv{Hkv} T{T}")
    wl = inputs.make_prefill(B, Hq, Hkv, T, 256, dtype="bf16", seed=61 + T, rho_std=0.1)
    got = _run(wl, aux=True)
    ref = _oracle(wl)
    check_bf16(got["o"], ref["o"], "o")
    check_bf16(got["vbar"], ref["o_sa"], "vbar")
    assert np.max(np.abs(got["lse"] - ref["lse"])) <= LSE_ABS


def test_key_count_probe_head_dim_256(gpu_lib):
    wl = inputs.make_prefill(1, 2, 1, 333, 256, dtype="bf16", seed=7)
    wl.tensors["q"].data[...] = 0
    got = _run(wl)
    n = np.rint(np.exp(got["lse"].astype(np.float64))).astype(np.int64)
    assert np.array_equal(n, np.broadcast_to(np.arange(1, 334), n.shape))
