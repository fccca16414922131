"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call."""

import ctypes
import os
import re

import pytest

from parallax_local_linear_plx_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "plx.h")

FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(plx_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_library_loads_and_exports_every_declared_symbol():
    L = binding.lib()
    names = _declared_functions()
    assert {"plx_fwd_prefill", "plx_decode", "plx_bwd"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"symbol {n} declared in plx.h but not exported"


def test_ceiling_library_loads_and_validates_arguments():
    """libplx_peak.so (the benchmark's measured ceilings) is built beside
    libplx.so; its entry points reject bad arguments before any launch."""
    path = os.path.join(ROOT, "parallax_local_linear_plx_amd", "libplx_peak.so")
    L = ctypes.CDLL(path)
    L.plx_peak_mfma_flops.restype = ctypes.c_double
    L.plx_peak_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    assert L.plx_peak_mfma_flops(1024, 500) == 1024 * 4 * 500 * 8 * 2 * 16 * 16 * 32
    L.plx_peak_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert L.plx_peak_mfma_bf16(None, 1, 1, None) == 1
    assert L.plx_peak_mfma_bf16(FAKE, 0, 1, None) == 1
    L.plx_peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p]
    assert L.plx_peak_hbm_read(FAKE, 24, FAKE, 1, None) == 1  # not a multiple of 16
    assert L.plx_peak_hbm_read(ctypes.c_void_p(0x10008), 32, FAKE, 1, None) == 1  # misaligned
    assert L.plx_peak_hbm_read(None, 32, FAKE, 1, None) == 1


def test_abi_version_and_status_strings():
    L = binding.lib()
    assert L.plx_abi_version() == 1
    for s in range(5):
        assert binding.status_string(s)
    assert binding.status_string(99) == "unknown status"


def _fwd(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, rho=FAKE, o=FAKE, lse=None, c=None, vb=None,
                B=1, Hq=2, Hkv=1, T=16, d=64, scale=0.125, dtype=binding.PLX_BF16)
    args.update(kw)
    return binding.lib().plx_fwd_prefill(args["q"], args["k"], args["v"], args["rho"], args["o"],
                                         args["lse"], args["c"], args["vb"], args["B"], args["Hq"],
                                         args["Hkv"], args["T"], args["d"], args["scale"],
                                         args["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), binding.PLX_ERR_INVALID_ARG),
    (dict(o=None), binding.PLX_ERR_INVALID_ARG),
    (dict(T=0), binding.PLX_ERR_INVALID_ARG),
    (dict(B=0), binding.PLX_ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), binding.PLX_ERR_INVALID_ARG),
    (dict(d=96), binding.PLX_ERR_UNSUPPORTED),
    (dict(d=256, dtype=binding.PLX_F32), binding.PLX_ERR_UNSUPPORTED),  # d = 256: bf16 only
    (dict(d=512), binding.PLX_ERR_UNSUPPORTED),
    (dict(scale=0.0), binding.PLX_ERR_INVALID_ARG),
    (dict(scale=float("nan")), binding.PLX_ERR_INVALID_ARG),
    (dict(dtype=7), binding.PLX_ERR_INVALID_ARG),
    (dict(q=ctypes.c_void_p(0x10002)), binding.PLX_ERR_INVALID_ARG),
])
def test_prefill_validation(kw, status):
    assert _fwd(**kw) == status


def _dec(**kw):
    args = dict(q=FAKE, rho=FAKE, k=FAKE, v=FAKE, ctx=FAKE, o=FAKE, lse=None, B=2, Hq=4, Hkv=2,
                S=1024, d=128, scale=0.1, ns=0, ws=FAKE, ws_bytes=1 << 30, dtype=binding.PLX_BF16)
    args.update(kw)
    return binding.lib().plx_decode(args["q"], args["rho"], args["k"], args["v"], args["ctx"],
                                    args["o"], args["lse"], args["B"], args["Hq"], args["Hkv"],
                                    args["S"], args["d"], args["scale"], args["ns"], args["ws"],
                                    args["ws_bytes"], args["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ctx=None), binding.PLX_ERR_INVALID_ARG),
    (dict(S=0), binding.PLX_ERR_INVALID_ARG),
    (dict(ns=-1), binding.PLX_ERR_INVALID_ARG),
    (dict(Hq=5, Hkv=2), binding.PLX_ERR_INVALID_ARG),  # Hq not a multiple of Hkv
    (dict(d=32), binding.PLX_ERR_UNSUPPORTED),
    (dict(d=256, dtype=binding.PLX_F32), binding.PLX_ERR_UNSUPPORTED),
    (dict(ws=None), binding.PLX_ERR_WORKSPACE),
    (dict(ws_bytes=16), binding.PLX_ERR_WORKSPACE),
])
def test_decode_validation(kw, status):
    assert _dec(**kw) == status


def test_decode_workspace_size_is_consistent():
    n0 = binding.decode_workspace_size(64, 16, 8, 8192, 128, 0)
    assert n0 > 0 and n0 % 16 == 0
    n4 = binding.decode_workspace_size(64, 16, 8, 8192, 128, 4)
    rec = 2 * 128 + 4
    assert n4 == 64 * 16 * 4 * rec * 4
    assert binding.decode_workspace_size(0, 16, 8, 8192, 128, 0) == 0
    # exactly the reported size is accepted by validation (up to the launch)
    assert _dec(ws_bytes=binding.decode_workspace_size(2, 4, 2, 1024, 128, 0) - 1) == binding.PLX_ERR_WORKSPACE


def _bwd(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, rho=FAKE, do=FAKE, o=FAKE, lse=FAKE, c=FAKE, vb=FAKE,
                dq=FAKE, dk=FAKE, dv=FAKE, dr=FAKE, B=1, Hq=2, Hkv=1, T=64, d=128, scale=0.1,
                ws=FAKE, ws_bytes=1 << 20, dtype=binding.PLX_BF16)
    args.update(kw)
    return binding.lib().plx_bwd(args["q"], args["k"], args["v"], args["rho"], args["do"], args["o"],
                                 args["lse"], args["c"], args["vb"], args["dq"], args["dk"], args["dv"],
                                 args["dr"], args["B"], args["Hq"], args["Hkv"], args["T"], args["d"],
                                 args["scale"], args["ws"], args["ws_bytes"], args["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(lse=None), binding.PLX_ERR_INVALID_ARG),
    (dict(vb=None), binding.PLX_ERR_INVALID_ARG),
    (dict(dr=None), binding.PLX_ERR_INVALID_ARG),
    (dict(T=-1), binding.PLX_ERR_INVALID_ARG),
    (dict(d=80), binding.PLX_ERR_UNSUPPORTED),
    (dict(d=256, dtype=binding.PLX_F32), binding.PLX_ERR_UNSUPPORTED),  # fp32 stops at d = 128
    (dict(d=256, ws_bytes=8), binding.PLX_ERR_WORKSPACE),  # bf16 d = 256 is served
    (dict(ws_bytes=8), binding.PLX_ERR_WORKSPACE),
    (dict(ws=None), binding.PLX_ERR_WORKSPACE),
])
def test_bwd_validation(kw, status):
    assert _bwd(**kw) == status


@pytest.mark.parametrize("B,Hq,Hkv,S_max,d", [
    (64, 16, 8, 8192, 128),   # 512 workgroups
    (1, 16, 8, 1024, 128),    # 16 workgroups of 512 keys
    (3, 4, 2, 700, 64),       # ceil(4200 / 512) = 9
    (1, 1, 1, 1, 256),        # a single workgroup
])
def test_balanced_decode_workspace_follows_the_schedule(B, Hq, Hkv, S_max, d):
    """The automatic schedule's workspace covers both automatic schedules:
    the balanced one (bf16) keeps one record of 2d + 4 floats per query head
    for each of the P + B Hkv (workgroup, segment) pieces, with
    P = min(512, ceil(B Hkv S_max / 512)) workgroups; the automatic split
    count (fp32) takes min(ceil(512 / (B Hkv)), ceil(S_max / 256)) splits of
    whole 128-key steps, one record per (b, query head, split)."""
    rec = (2 * d + 4) * 4
    P = min(512, -(-B * Hkv * S_max // 512))
    balanced = (P + B * Hkv) * (Hq // Hkv) * rec
    ns = max(1, min(-(-512 // (B * Hkv)), -(-S_max // 256)))
    chunk = -(-(-(-S_max // ns)) // 128) * 128
    split = B * Hq * -(-S_max // chunk) * rec
    assert binding.decode_workspace_size(B, Hq, Hkv, S_max, d, 0) == max(balanced, split)


def test_bwd_workspace_size():
    # G and delta (fp32 per query row, padded to 256 bytes); the dO scale, its
    # inverse and 2048 partial maxima (4 + 2048 words, padded to 256 bytes);
    # then fp16 copies of q, rho, dO ([B, Hq, T, d]) and k ([B, Hkv, T, d])
    for B, Hq, Hkv, T, d in ((8, 16, 8, 4096, 128), (1, 2, 1, 3, 64), (2, 16, 1, 300, 256)):
        head = (2 * B * Hq * T * 4 + 255) // 256 * 256 + (4 * (4 + 2048) + 255) // 256 * 256
        want = head + (3 * B * Hq * T * d + B * Hkv * T * d) * 2
        assert binding.bwd_workspace_size(B, Hq, Hkv, T, d) == want
    assert binding.bwd_workspace_size(8, 16, 8, 0, 128) == 0


def _fwd_ex(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, rho=FAKE, o=FAKE, lse=None, c=None, vb=None, cor=None,
                B=1, Hq=2, Hkv=1, T=16, d=64, scale=0.125, flags=0, dtype=binding.PLX_BF16)
    args.update(kw)
    return binding.lib().plx_fwd_prefill_ex(
        args["q"], args["k"], args["v"], args["rho"], args["o"], args["lse"], args["c"], args["vb"],
        args["cor"], args["B"], args["Hq"], args["Hkv"], args["T"], args["d"], args["scale"],
        args["flags"], args["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(flags=4), binding.PLX_ERR_INVALID_ARG),
    (dict(flags=0xFFFFFFFF), binding.PLX_ERR_INVALID_ARG),
    (dict(cor=ctypes.c_void_p(0x10002)), binding.PLX_ERR_INVALID_ARG),
    (dict(lse=ctypes.c_void_p(0x10001)), binding.PLX_ERR_INVALID_ARG),
    (dict(q=None, flags=3), binding.PLX_ERR_INVALID_ARG),
    (dict(d=96, flags=1), binding.PLX_ERR_UNSUPPORTED),
    (dict(T=0, flags=2), binding.PLX_ERR_INVALID_ARG),
])
def test_prefill_ex_validation(kw, status):
    assert _fwd_ex(**kw) == status


def _dec_ex(**kw):
    args = dict(q=FAKE, rho=FAKE, k=FAKE, v=FAKE, ctx=FAKE, o=FAKE, lse=None, cor=None, B=2, Hq=4,
                Hkv=2, S=1024, d=128, scale=0.1, ns=0, flags=0, ws=FAKE, ws_bytes=1 << 30,
                dtype=binding.PLX_BF16)
    args.update(kw)
    return binding.lib().plx_decode_ex(
        args["q"], args["rho"], args["k"], args["v"], args["ctx"], args["o"], args["lse"],
        args["cor"], args["B"], args["Hq"], args["Hkv"], args["S"], args["d"], args["scale"],
        args["ns"], args["flags"], args["ws"], args["ws_bytes"], args["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(flags=8), binding.PLX_ERR_INVALID_ARG),
    (dict(cor=ctypes.c_void_p(0x10003)), binding.PLX_ERR_INVALID_ARG),
    (dict(ctx=ctypes.c_void_p(0x10002)), binding.PLX_ERR_INVALID_ARG),
    (dict(d=96, flags=2), binding.PLX_ERR_UNSUPPORTED),
    (dict(ws_bytes=16, flags=3), binding.PLX_ERR_WORKSPACE),
])
def test_decode_ex_validation(kw, status):
    assert _dec_ex(**kw) == status


def _proj(**kw):
    args = dict(x=FAKE, w=FAKE, q=FAKE, k=FAKE, v=FAKE, r=FAKE, B=1, T=16, D=128, Hq=2, Hkv=1, d=64,
                dtype=binding.PLX_BF16)
    args.update(kw)
    return binding.lib().plx_qkvr_proj(args["x"], args["w"], args["q"], args["k"], args["v"], args["r"],
                                       args["B"], args["T"], args["D"], args["Hq"], args["Hkv"],
                                       args["d"], args["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), binding.PLX_ERR_INVALID_ARG),
    (dict(r=None), binding.PLX_ERR_INVALID_ARG),
    (dict(T=0), binding.PLX_ERR_INVALID_ARG),
    (dict(D=0), binding.PLX_ERR_INVALID_ARG),
    (dict(D=96), binding.PLX_ERR_UNSUPPORTED),
    (dict(d=32), binding.PLX_ERR_UNSUPPORTED),
    (dict(Hq=3, Hkv=2), binding.PLX_ERR_INVALID_ARG),
    (dict(dtype=binding.PLX_F32), binding.PLX_ERR_UNSUPPORTED),
    (dict(dtype=9), binding.PLX_ERR_INVALID_ARG),
    (dict(w=ctypes.c_void_p(0x10008)), binding.PLX_ERR_INVALID_ARG),
])
def test_proj_validation(kw, status):
    assert _proj(**kw) == status


# -- the Python binding rejects malformed tensors before any library call -----

def _bf16(*shape):
    import torch

    return torch.zeros(*shape, dtype=torch.bfloat16)


def test_binding_rejects_noncontiguous_decode_query():
    """The last-token slice q[:, :, -1, :] of a [B, H, T, d] tensor is not
    contiguous; the binding must refuse it rather than read it with the wrong
    strides."""
    import torch

    from parallax_local_linear_plx_amd import plx_decode

    B, Hq, Hkv, S, d = 2, 4, 2, 16, 64
    q = _bf16(B, Hq, 5, d)[:, :, -1, :]
    assert not q.is_contiguous()
    with pytest.raises(ValueError, match="contiguous"):
        plx_decode(q, _bf16(B, Hq, d), _bf16(B, Hkv, S, d), _bf16(B, Hkv, S, d),
                   torch.full((B,), S, dtype=torch.int32))


def test_binding_rejects_wrong_output_buffers():
    import torch

    from parallax_local_linear_plx_amd import plx_bwd, plx_decode, plx_fwd_prefill

    B, Hq, Hkv, T, d = 1, 2, 1, 8, 64
    q, k = _bf16(B, Hq, T, d), _bf16(B, Hkv, T, d)
    with pytest.raises(ValueError, match="dtype"):
        plx_fwd_prefill(q, k, k, q, o=torch.zeros(B, Hq, T, d, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        plx_fwd_prefill(q, k, k, q, o=torch.zeros(B, Hq, T + 1, d))
    with pytest.raises(ValueError, match="dtype"):
        plx_decode(_bf16(B, Hq, d), _bf16(B, Hq, d), k, k, torch.full((B,), T, dtype=torch.int32),
                   o=torch.zeros(B, Hq, d, dtype=torch.float16))
    f32 = lambda *s: torch.zeros(*s)  # noqa: E731
    grads = {"dq": f32(B, Hq, T, d), "dk": f32(B, Hkv, T, d), "dv": f32(B, Hkv, T, d),
             "drho": f32(B, Hq, T + 1, d)}
    with pytest.raises(ValueError, match="shape"):
        plx_bwd(q, k, k, q, q, f32(B, Hq, T, d), f32(B, Hq, T), f32(B, Hq, T), f32(B, Hq, T, d),
                grads=grads)
    with pytest.raises(ValueError, match="contiguous"):
        plx_bwd(q.transpose(2, 3).contiguous().transpose(2, 3), k, k, q, q, f32(B, Hq, T, d),
                f32(B, Hq, T), f32(B, Hq, T), f32(B, Hq, T, d))


def test_binding_refuses_host_tensors():
    """Host tensors would hand the kernels host pointers."""
    import torch

    from parallax_local_linear_plx_amd import plx_fwd_prefill

    q, k = _bf16(1, 2, 8, 64), _bf16(1, 1, 8, 64)
    with pytest.raises(ValueError, match="GPU tensors only"):
        plx_fwd_prefill(q, k, k, q)
    assert torch.zeros(1).device.type == "cpu"


def test_decode_noalloc_refuses_problems_beyond_its_buffer():
    """plx_decode_noalloc keeps its records in a fixed per-GPU array of
    PLX_DECODE_SCRATCH_BYTES; a problem needing more is refused before any HIP
    call, with the workspace status.  Other validation matches plx_decode."""
    L = binding.lib()
    i32 = ctypes.c_int
    args = lambda B, Hq, Hkv, S, d, ns, dtype=binding.PLX_BF16: (  # noqa: E731
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, B, Hq, Hkv, S, d, ctypes.c_float(0.1), ns, dtype, None)
    big = (64, 16, 1, 1 << 16, 128, 256)
    assert binding.decode_workspace_size(*big) > binding.DECODE_SCRATCH_BYTES
    assert L.plx_decode_noalloc(*args(*big)) == binding.PLX_ERR_WORKSPACE
    assert L.plx_decode_noalloc(*args(2, 4, 2, 64, 96, 0)) == binding.PLX_ERR_UNSUPPORTED  # d = 96
    assert L.plx_decode_noalloc(*args(2, 4, 2, 0, 128, 0)) == binding.PLX_ERR_INVALID_ARG
    a = list(args(2, 4, 2, 64, 128, 0))
    a[0] = None
    assert L.plx_decode_noalloc(*a) == binding.PLX_ERR_INVALID_ARG
    assert i32(binding.DECODE_SCRATCH_BYTES).value == 16 << 20
