"""plx_decode_noalloc (records in the library's static per-GPU array) against
plx_decode (caller-owned workspace) through the C ABI: two calls in a row,
the second smaller, and each against the oracle."""

import numpy as np
import pytest

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


def _both(wl, num_splits):
    import torch

    from parallax_local_linear_plx_amd import plx_decode, plx_decode_noalloc

    t = _dev(wl)
    nan = float("nan")
    o_a = torch.full((wl.B, wl.Hq, wl.d), nan, dtype=torch.float32, device="cuda")
    o_b = torch.full((wl.B, wl.Hq, wl.d), nan, dtype=torch.float32, device="cuda")
    a = plx_decode(t["q"], t["rho"], t["k"], t["v"], t["ctx"], wl.scale, num_splits=num_splits, o=o_a)
    b = plx_decode_noalloc(t["q"], t["rho"], t["k"], t["v"], t["ctx"], wl.scale,
                           num_splits=num_splits, o=o_b)
    torch.cuda.synchronize()
    return ({n: x.cpu().numpy() for n, x in a.items()}, {n: x.cpu().numpy() for n, x in b.items()})


@pytest.mark.parametrize("dtype,num_splits", [("bf16", 0), ("bf16", 3), ("f32", 0)])
def test_noalloc_matches_workspace_decode_twice(gpu_lib, dtype, num_splits):
    cases = [
        inputs.make_decode(6, 16, 8, 128, 0, S_max=4000, dtype=dtype, seed=140,
                           ctx_list=[4000, 1, 2500, 777, 3999, 129]),
        inputs.make_decode(2, 4, 2, 128, 0, S_max=300, dtype=dtype, seed=141, ctx_list=[300, 57]),
    ]
    for wl in cases:
        say(f"case decode_noalloc {dtype} splits={num_splits} B{wl.B} Hq{wl.Hq} Hkv{wl.Hkv} S{wl.S_max}")
        a, b = _both(wl, num_splits)
        # same kernels and schedule: bitwise the same as the workspace entry point
        assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])
        ref = _fetch.decode_oracle(wl)
        if dtype == "bf16":
            check_bf16(b["o"].reshape(-1, wl.d), ref["o"], "o")
            assert np.max(np.abs(b["lse"].reshape(-1) - ref["lse"])) <= LSE_ABS
        else:
            check_fp32(b["o"].reshape(-1, wl.d), ref["o"], "o")
            check_fp32(b["lse"].reshape(-1), ref["lse"], "lse")
