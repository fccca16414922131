"""GPU parity of plx_decode (split-K partials + merge) against the fp64 oracle."""

import numpy as np
import pytest

from oracle import plx_oracle as orc
from parallax_local_linear_plx_amd import inputs
from tests import _fetch
from tests._util import LSE_ABS, check_bf16, check_fp32, say, to_device

pytestmark = pytest.mark.gpu


def _dev(wl):
    import torch

    t = {n: to_device(x) for n, x in wl.tensors.items()}
    t["q"] = t["q"].reshape(wl.B, wl.Hq, wl.d)
    t["rho"] = t["rho"].reshape(wl.B, wl.Hq, wl.d)
    t["ctx"] = torch.from_numpy(wl.ctx_len.astype(np.int32)).cuda()
    return t


def _run(wl, num_splits=0, t=None):
    import torch

    from parallax_local_linear_plx_amd import plx_decode

    if t is None:
        t = _dev(wl)
    o = torch.full((wl.B, wl.Hq, wl.d), float("nan"), dtype=torch.float32, device="cuda")
    out = plx_decode(t["q"], t["rho"], t["k"], t["v"], t["ctx"], wl.scale, num_splits=num_splits, o=o)
    torch.cuda.synchronize()
    return {n: x.cpu().numpy() for n, x in out.items()}


def _oracle(wl, heads=None):
    return _fetch.decode_oracle(wl, heads)


@pytest.mark.parametrize("num_splits", [0, 1, 3, 7])
def test_bf16_ragged_small(gpu_lib, num_splits):
    say(f"case decode bf16 B3 Hq4 Hkv2 S700 ragged splits={num_splits}")
    wl = inputs.make_decode(3, 4, 2, 128, 0, S_max=700, dtype="bf16", seed=50, ctx_list=[700, 1, 333])
    got = _run(wl, num_splits)
    ref = _oracle(wl)
    check_bf16(got["o"].reshape(-1, wl.d), ref["o"], "o")
    assert np.max(np.abs(got["lse"].reshape(-1) - ref["lse"])) <= LSE_ABS


@pytest.mark.parametrize("G,d", [(1, 64), (8, 128), (16, 64), (2, 128)])
def test_fp32_group_sizes(gpu_lib, G, d):
    say(f"case decode fp32 G{G} d{d}")
    wl = inputs.make_decode(2, 2 * G, 2, d, 0, S_max=300, dtype="f32", seed=60 + G, ctx_range=(1, 300),
                            rho_std=0.5)
    got = _run(wl, 2)
    ref = _oracle(wl)
    check_fp32(got["o"].reshape(-1, d), ref["o"], "o")
    check_fp32(got["lse"].reshape(-1), ref["lse"], "lse")


@pytest.mark.parametrize("dtype,G,num_splits", [
    ("bf16", 3, 0), ("bf16", 5, 2), ("bf16", 7, 0), ("bf16", 12, 0), ("bf16", 24, 0), ("bf16", 32, 3),
    ("f32", 3, 2), ("f32", 24, 2),
])
def test_group_sizes_of_any_count(gpu_lib, dtype, G, num_splits):
    """Any Hq / Hkv, not only powers of two: a group of more than 16 query
    heads is covered 16 heads at a time, the remainder by the kernel whose
    column capacity holds it.  Every head matches the oracle, and nothing is
    written past the workspace (a guard region after it keeps its fill)."""
    import torch

    from parallax_local_linear_plx_amd import decode_workspace_size, plx_decode

    B, Hkv, S = 2, 2, 300
    d = 64 if dtype == "f32" else 128
    say(f"case decode {dtype} G{G} Hq{G * Hkv} Hkv{Hkv} d{d} splits={num_splits}")
    wl = inputs.make_decode(B, G * Hkv, Hkv, d, 0, S_max=S, dtype=dtype, seed=90 + G, ctx_list=[S, 137],
                            rho_std=0.5)
    t = _dev(wl)
    need = decode_workspace_size(B, wl.Hq, Hkv, S, d, num_splits)
    ws = torch.full((need + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    o = torch.full((B, wl.Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    out = plx_decode(t["q"], t["rho"], t["k"], t["v"], t["ctx"], wl.scale, num_splits=num_splits,
                     workspace=ws, o=o)
    torch.cuda.synchronize()
    ref = _oracle(wl)
    check = check_bf16 if dtype == "bf16" else check_fp32
    check(out["o"].cpu().numpy().reshape(-1, d), ref["o"], "o")
    assert np.max(np.abs(out["lse"].cpu().numpy().reshape(-1) - ref["lse"])) <= LSE_ABS
    assert bool((ws[need:] == 0x5A).all()), "write past the workspace"


@pytest.mark.parametrize("num_splits", [0, 1, 5, 64])
def test_key_count_probe_is_exact(gpu_lib, num_splits):
    """q = 0: exp(LSE) must round to ctx_len[b] exactly for every split count."""
    ctx = np.array([5000, 1, 129, 4097], np.int32)
    wl = inputs.make_decode(4, 4, 2, 128, 0, S_max=5000, dtype="bf16", seed=70, ctx_list=ctx)
    wl.tensors["q"].data[...] = 0
    got = _run(wl, num_splits)
    n = np.rint(np.exp(got["lse"].astype(np.float64))).astype(np.int64)
    assert np.array_equal(n, np.repeat(ctx[:, None], wl.Hq, axis=1))


def test_mapping_probe_and_invalid_lengths(gpu_lib):
    """V constant per (b, kv head): o rounds to that code; ctx_len outside
    [1, S_max] gives NaN for that sequence only."""
    import torch

    B, Hq, Hkv, S, d = 4, 8, 2, 600, 128
    wl = inputs.make_decode(B, Hq, Hkv, d, S, dtype="bf16", seed=80)
    codes = (np.arange(B * Hkv).reshape(B, Hkv) + 1).astype(np.float32)
    v = np.broadcast_to(codes[:, :, None, None], (B, Hkv, S, d)).astype(np.float32)
    wl.tensors["v"].data[...] = inputs.bf16_round_bits(v)
    t = _dev(wl)
    ctx = np.array([600, 0, 601, 17], np.int32)
    t["ctx"] = torch.from_numpy(ctx).cuda()
    got = _run(wl, 0, t)
    o = got["o"]
    want = np.repeat(codes, Hq // Hkv, axis=1)
    for b in (0, 3):
        assert np.array_equal(np.rint(o[b]), np.broadcast_to(want[b][:, None], o[b].shape))
    for b in (1, 2):
        assert np.all(np.isnan(o[b])) and np.all(np.isnan(got["lse"][b]))


@pytest.mark.parametrize("Hq,Hkv", [(16, 8), (32, 2)])
def test_bf16_balanced_schedule_many_short_sequences(gpu_lib, Hq, Hkv):
    """Automatic schedule over many short ragged sequences: workgroup ranges
    span several (b, kv head) segments.  Valid sequences match the oracle and
    the explicit-split path; lengths outside [1, S_max] give NaN rows."""
    import torch

    B, d, S = 40, 128, 300
    say(f"case decode bf16 balanced B{B} Hq{Hq} Hkv{Hkv} ctx U{{1..{S}}} + invalid lengths")
    wl = inputs.make_decode(B, Hq, Hkv, d, 0, S_max=S, dtype="bf16", seed=85, ctx_range=(1, S))
    t = _dev(wl)
    ctx = wl.ctx_len.copy()
    ctx[[3, 17]] = [0, S + 1]  # invalid: those rows must be NaN
    t["ctx"] = torch.from_numpy(ctx).cuda()
    got = _run(wl, 0, t)
    split = _run(wl, 3, t)
    valid = [b for b in range(B) if 1 <= ctx[b] <= S]
    for b in (3, 17):
        assert np.all(np.isnan(got["o"][b])) and np.all(np.isnan(got["lse"][b]))
    heads = [(b, h) for b in valid for h in range(Hq)]
    ref = _oracle(wl, heads)
    o = np.array([got["o"][b, h] for b, h in heads])
    check_bf16(o, ref["o"], "o")
    assert np.max(np.abs(np.array([got["lse"][b, h] for b, h in heads]) - ref["lse"])) <= LSE_ABS
    o_split = np.array([split["o"][b, h] for b, h in heads])
    assert np.max(np.abs(o - o_split)) < 1e-3


@pytest.mark.parametrize("Hq,Hkv,S,ctx_list,bad", [
    (4, 2, 4096, [3, 9, 5, 1, 7, 2], {1: 0, 4: 4097}),   # fewer keys than workgroups
    (16, 1, 8192, [7, 2, 11], {1: -5}),                 # two 8-head passes, sparse
])
def test_bf16_balanced_schedule_fewer_keys_than_workgroups(gpu_lib, Hq, Hkv, S, ctx_list, bad):
    """Automatic schedule when the valid keys number fewer than the workgroups:
    ranges hold at most one key, some are empty, and the workgroup that
    completes a segment's count merges it."""
    import torch

    B, d = len(ctx_list), 128
    say(f"case decode bf16 balanced sparse B{B} Hq{Hq} Hkv{Hkv} S{S} ctx {ctx_list} invalid {bad}")
    wl = inputs.make_decode(B, Hq, Hkv, d, 0, S_max=S, dtype="bf16", seed=86, ctx_list=ctx_list)
    t = _dev(wl)
    ctx = wl.ctx_len.copy()
    for b, c in bad.items():
        ctx[b] = c
    t["ctx"] = torch.from_numpy(ctx).cuda()
    got = _run(wl, 0, t)
    for b in bad:
        assert np.all(np.isnan(got["o"][b])) and np.all(np.isnan(got["lse"][b]))
    heads = [(b, h) for b in range(B) if b not in bad for h in range(Hq)]
    ref = _oracle(wl, heads)
    check_bf16(np.array([got["o"][b, h] for b, h in heads]), ref["o"], "o")
    assert np.max(np.abs(np.array([got["lse"][b, h] for b, h in heads]) - ref["lse"])) <= LSE_ABS


@pytest.mark.parametrize("Hq,Hkv,S", [(16, 1, 65536), (2, 1, 200000)])
def test_bf16_balanced_schedule_one_long_segment(gpu_lib, Hq, Hkv, S):
    """One sequence spread over every workgroup: a segment merges 64 and more
    records (the merge's multi-batch path), with one or two head passes."""
    B, d = 1, 128
    say(f"case decode bf16 balanced one segment B{B} Hq{Hq} Hkv{Hkv} ctx{S}")
    wl = inputs.make_decode(B, Hq, Hkv, d, S, dtype="bf16", seed=87)
    got = _run(wl)
    heads = [(0, h) for h in range(Hq)]
    ref = _oracle(wl, heads)
    check_bf16(np.array([got["o"][b, h] for b, h in heads]), ref["o"], "o")
    assert np.max(np.abs(np.array([got["lse"][b, h] for b, h in heads]) - ref["lse"])) <= LSE_ABS
    split = _run(wl, 5)
    assert np.max(np.abs(got["o"] - split["o"])) < 1e-3


def test_decode_matches_prefill_last_row(gpu_lib):
    """Decode over the first t cache rows equals the prefill output at row t-1
    (both on the GPU, both checked against the oracle)."""
    import torch

    from parallax_local_linear_plx_amd import plx_decode, plx_fwd_prefill

    B, Hq, Hkv, T, d = 2, 4, 2, 257, 128
    wl = inputs.make_prefill(B, Hq, Hkv, T, d, dtype="bf16", seed=90)
    t = {n: to_device(x) for n, x in wl.tensors.items()}
    pre = plx_fwd_prefill(t["q"], t["k"], t["v"], t["rho"], wl.scale)
    ctx = torch.tensor([T, 100], dtype=torch.int32, device="cuda")
    qd = torch.stack([t["q"][0, :, T - 1], t["q"][1, :, 99]]).contiguous()
    rd = torch.stack([t["rho"][0, :, T - 1], t["rho"][1, :, 99]]).contiguous()
    dec = plx_decode(qd, rd, t["k"], t["v"], ctx, wl.scale, num_splits=2)
    torch.cuda.synchronize()
    o_pre = torch.stack([pre["o"][0, :, T - 1], pre["o"][1, :, 99]]).cpu().numpy()
    assert np.max(np.abs(dec["o"].cpu().numpy() - o_pre)) < 5e-3


def test_bf16_decode_full_size_sampled_heads(gpu_lib):
    """Batched decode at full size: B=64, Hq=16, Hkv=8, ctx=8192, d=128."""
    say("case decode bf16 B64 Hq16 Hkv8 ctx8192 d128 (sampled heads)")
    wl = inputs.bf16_decode()
    got = _run(wl)
    assert np.all(np.isfinite(got["o"]))
    g = np.random.default_rng(7)
    heads = [(0, 0), (63, 15), (31, 8)] + [(int(g.integers(64)), int(g.integers(16))) for _ in range(21)]
    ref = _oracle(wl, heads)
    check_bf16(np.array([got["o"][b, h] for b, h in heads]), ref["o"], "o (sampled heads)")
    assert np.max(np.abs(np.array([got["lse"][b, h] for b, h in heads]) - ref["lse"])) <= LSE_ABS


def test_bf16_long_decode_full_size_sampled_heads(gpu_lib):
    """Long-context ragged decode at full size: B=8, ctx ~ U{16384..131072}."""
    say("case long decode bf16 B8 Hq16 Hkv8 ctx 16384-131072 d128 (sampled heads)")
    wl = inputs.bf16_long_decode()
    say(f"  ctx_len = {wl.ctx_len.tolist()}")
    got = _run(wl)
    assert np.all(np.isfinite(got["o"]))
    heads = [(b, (5 * b) % 16) for b in range(8)] + [(int(np.argmax(wl.ctx_len)), 15)]
    ref = _oracle(wl, heads)
    check_bf16(np.array([got["o"][b, h] for b, h in heads]), ref["o"], "o (sampled heads)")
    assert np.max(np.abs(np.array([got["lse"][b, h] for b, h in heads]) - ref["lse"])) <= LSE_ABS


@pytest.mark.parametrize("G,num_splits", [(1, 0), (2, 3), (4, 0), (8, 1), (16, 0), (16, 5)])
def test_bf16_head_dim_256(gpu_lib, G, num_splits):
    """d = 256 on both schedules and every group size, ragged contexts
    including a single key."""
    say(f"case decode bf16 d256 G{G} splits={num_splits}")
    wl = inputs.make_decode(3, 2 * G, 2, 256, 0, S_max=900, dtype="bf16", seed=90 + G,
                            ctx_list=[900, 1, 513])
    got = _run(wl, num_splits)
    ref = _oracle(wl)
    check_bf16(got["o"].reshape(-1, 256), ref["o"], "o")
    assert np.max(np.abs(got["lse"].reshape(-1) - ref["lse"])) <= LSE_ABS


def test_bf16_head_dim_256_key_count_probe(gpu_lib):
    ctx = np.array([3000, 1, 257], np.int32)
    wl = inputs.make_decode(3, 4, 2, 256, 0, S_max=3000, dtype="bf16", seed=71, ctx_list=ctx)
    wl.tensors["q"].data[...] = 0
    for ns in (0, 3):
        got = _run(wl, ns)
        n = np.rint(np.exp(got["lse"].astype(np.float64))).astype(np.int64)
        assert np.array_equal(n, np.repeat(ctx[:, None], wl.Hq, axis=1)), ns


@pytest.mark.parametrize("num_splits,dtype", [(0, "bf16"), (3, "bf16"), (2, "f32")])
def test_repeat_runs_are_bitwise_identical(gpu_lib, num_splits, dtype):
    """The four waves of a workgroup combine their states in a fixed order and
    the merge sums records in slot order: repeated calls agree bit for bit."""
    wl = inputs.make_decode(5, 8, 2, 128, 0, S_max=3000, dtype=dtype, seed=130,
                            ctx_list=[3000, 1, 777, 2048, 129])
    t = _dev(wl)
    a = _run(wl, num_splits, t)
    for _ in range(3):
        b = _run(wl, num_splits, t)
        assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])
