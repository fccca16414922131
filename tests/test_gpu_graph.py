"""The entry points captured in a HIP graph (through torch.cuda.CUDAGraph) and
replayed: every replay, with new inputs copied in between and eager work and
synchronisations around it, must reproduce the eager call bit for bit.  The
library launches kernels only (no memset or copy nodes), so a captured call
is the same kernel sequence as an eager one."""

import numpy as np
import pytest

from parallax_local_linear_plx_amd import inputs
from tests._util import say, to_device

pytestmark = pytest.mark.gpu


def _capture(fn):
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the graph (loads the library, allocates nothing new)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("num_splits", [0, 3])
def test_decode_graph_replays_match_eager(gpu_lib, num_splits):
    import torch

    from parallax_local_linear_plx_amd import decode_workspace_size, plx_decode

    B, Hq, Hkv, d, S = 3, 8, 2, 128, 700
    say(f"case decode graph replay splits={num_splits}")
    wl = inputs.make_decode(B, Hq, Hkv, d, 0, S_max=S, dtype="bf16", seed=120, ctx_list=[700, 1, 333])
    t = {n: to_device(x) for n, x in wl.tensors.items()}
    q = t["q"].reshape(B, Hq, d).clone()
    rho = t["rho"].reshape(B, Hq, d).clone()
    ctx = torch.from_numpy(wl.ctx_len).cuda()
    ws = torch.empty(decode_workspace_size(B, Hq, Hkv, S, d, num_splits), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")

    def call():
        out = plx_decode(q, rho, t["k"], t["v"], ctx, wl.scale, num_splits=num_splits, workspace=ws, o=o,
                         lse=True)
        lse.copy_(out["lse"])

    g = _capture(call)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    for rep in range(4):
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda").bfloat16())
        rho.copy_((0.1 * torch.randn(rho.shape, generator=gen, device="cuda")).bfloat16())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = o.clone(), lse.clone()
        ws.fill_(0xFF)  # eager work between replays, and a dirty workspace
        call()
        torch.cuda.synchronize()
        assert torch.equal(got_o, o) and torch.equal(got_l, lse), f"replay {rep} differs from eager"
    del g


def test_prefill_graph_replays_match_eager(gpu_lib):
    import torch

    from parallax_local_linear_plx_amd import plx_fwd_prefill

    wl = inputs.make_prefill(1, 4, 2, 300, 128, dtype="bf16", seed=121)
    t = {n: to_device(x).clone() for n, x in wl.tensors.items()}
    o = torch.empty((1, 4, 300, 128), dtype=torch.float32, device="cuda")

    def call():
        plx_fwd_prefill(t["q"], t["k"], t["v"], t["rho"], wl.scale, o=o, lse=False)

    g = _capture(call)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(6)
    for rep in range(3):
        t["q"].copy_(torch.randn(t["q"].shape, generator=gen, device="cuda").bfloat16())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = o.clone()
        o.zero_()
        call()
        torch.cuda.synchronize()
        assert torch.equal(got, o), f"replay {rep} differs from eager"
    del g


def test_bwd_graph_replays_match_eager(gpu_lib):
    """The bf16 backward (dO scale reduction, its scale, dQ/drho, dK/dV) in one
    graph: each replay takes the dO in memory at replay time, including its
    power-of-two scale, and matches the eager call bit for bit."""
    import torch

    from parallax_local_linear_plx_amd import bwd_workspace_size, plx_bwd, plx_fwd_prefill

    B, Hq, Hkv, T, d = 1, 4, 2, 300, 128
    say(f"case bwd graph replay B{B} Hq{Hq} Hkv{Hkv} T{T} d{d}")
    wl = inputs.make_prefill(B, Hq, Hkv, T, d, dtype="bf16", seed=122, with_grad=True)
    t = {n: to_device(x).clone() for n, x in wl.tensors.items()}
    fwd = plx_fwd_prefill(t["q"], t["k"], t["v"], t["rho"], wl.scale, aux=True)
    ws = torch.empty(bwd_workspace_size(B, Hq, Hkv, T, d), dtype=torch.uint8, device="cuda")
    grads = {n: torch.empty(shape, dtype=torch.float32, device="cuda")
             for n, shape in (("dq", (B, Hq, T, d)), ("dk", (B, Hkv, T, d)), ("dv", (B, Hkv, T, d)),
                              ("drho", (B, Hq, T, d)))}
    d_o = t["d_o"]
    base = d_o.clone()

    def call():
        plx_bwd(t["q"], t["k"], t["v"], t["rho"], d_o, fwd["o"], fwd["lse"], fwd["c"], fwd["vbar"], wl.scale,
                workspace=ws, grads=grads)

    g = _capture(call)
    for rep, sc in enumerate((1.0, 2.0 ** -20, 2.0 ** 12, 1.0)):
        d_o.copy_(base * sc)  # exact in bf16: a power of two
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {n: x.clone() for n, x in grads.items()}
        ws.fill_(0xFF)  # eager work between replays, and a dirty workspace
        for x in grads.values():
            x.zero_()
        call()
        torch.cuda.synchronize()
        for n, x in grads.items():
            assert torch.equal(got[n], x), f"replay {rep} (dO x {sc}) differs from eager in {n}"
    del g


def test_projection_graph_replays_match_eager(gpu_lib):
    import torch

    from parallax_local_linear_plx_amd import plx_qkvr_proj

    B, T, D, Hq, Hkv, d = 2, 300, 256, 4, 2, 64
    say(f"case projection graph replay B{B} T{T} D{D} Hq{Hq} Hkv{Hkv} d{d}")
    wl = inputs.make_projection(B, T, D, Hq, Hkv, d, seed=123)
    x = to_device(wl.tensors["x"]).clone()
    w = to_device(wl.tensors["w"]).clone()
    out = {n: torch.empty((B, H, T, d), dtype=torch.bfloat16, device="cuda")
           for n, H in (("q", Hq), ("k", Hkv), ("v", Hkv), ("rho", Hq))}

    def call():
        plx_qkvr_proj(x, w, Hq, Hkv, d, out=out)

    g = _capture(call)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    for rep in range(3):
        x.copy_(torch.randn(x.shape, generator=gen, device="cuda").bfloat16())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {n: y.clone() for n, y in out.items()}
        for y in out.values():
            y.zero_()
        call()
        torch.cuda.synchronize()
        for n, y in out.items():
            assert torch.equal(got[n], y), f"replay {rep} differs from eager in {n}"
    del g
