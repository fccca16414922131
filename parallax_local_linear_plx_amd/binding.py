"""Thin ctypes binding over libplx.so.

Argument marshalling only: every step of the operator runs in the HIP
kernels behind the C ABI.  Torch tensors provide device memory and the
current HIP stream.  There is no fallback: a missing library raises.
"""

from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libplx.so")

PLX_OK, PLX_ERR_INVALID_ARG, PLX_ERR_UNSUPPORTED, PLX_ERR_WORKSPACE, PLX_ERR_HIP = range(5)
PLX_F32, PLX_BF16 = 0, 1
# family-corner flags of the _ex entry points
PLX_UNIFORM_WEIGHTS, PLX_NO_INTERCEPT = 1, 2

_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t


class PlxError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libplx.so (built in-tree).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m parallax_local_linear_plx_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.plx_abi_version.restype = _i
    L.plx_abi_version.argtypes = []
    L.plx_status_string.restype = ctypes.c_char_p
    L.plx_status_string.argtypes = [_i]
    L.plx_fwd_prefill.restype = _i
    L.plx_fwd_prefill.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _i, _i, _i, _i, _i, _f, _i, _vp]
    L.plx_fwd_prefill_ex.restype = _i
    L.plx_fwd_prefill_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _i, _i, _i, _i, _i, _f, ctypes.c_uint, _i, _vp]
    L.plx_decode_ex.restype = _i
    L.plx_decode_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _i, _i, _i, _i, _i, _f, _i, ctypes.c_uint, _vp, _sz, _i, _vp]
    L.plx_decode_workspace_size.restype = _sz
    L.plx_decode_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i]
    L.plx_decode.restype = _i
    L.plx_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _i, _vp]
    L.plx_decode_noalloc.restype = _i
    L.plx_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _i, _i, _i, _i, _i, _f, _i, _i, _vp]
    L.plx_qkvr_proj.restype = _i
    L.plx_qkvr_proj.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]
    L.plx_bwd_workspace_size.restype = _sz
    L.plx_bwd_workspace_size.argtypes = [_i, _i, _i, _i, _i]
    L.plx_bwd.restype = _i
    L.plx_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                          _vp, _vp, _vp, _vp,
                          _i, _i, _i, _i, _i, _f, _vp, _sz, _i, _vp]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().plx_status_string(status).decode()


def _check(status: int, what: str):
    if status != PLX_OK:
        raise PlxError(status, what)


# ---------------------------------------------------------------------------
# tensor-level helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return PLX_BF16
    if t.dtype == torch.float32:
        return PLX_F32
    raise TypeError(f"unsupported input dtype {t.dtype}; use bfloat16 or float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _need_workspace(ws, device, need):
    """A caller-supplied workspace: device memory of at least ``need`` bytes."""
    if ws.device != device:
        raise ValueError(f"workspace: on {ws.device}, expected {device}")
    if not ws.is_contiguous():
        raise ValueError("workspace: must be contiguous")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace: {ws.numel() * ws.element_size()} bytes < {need} needed")


def _need_gpu(device):
    if device.type != "cuda":
        raise ValueError(f"tensors are on {device}; the HIP library takes GPU tensors only")


def plx_fwd_prefill(q, k, v, rho, scale=None, *, o=None, lse=True, aux=False):
    """Causal prefill forward.  q, rho [B,Hq,T,d]; k, v [B,Hkv,T,d] (bf16 or fp32, cuda).

    Returns dict with o [B,Hq,T,d] fp32, and lse [B,Hq,T] when ``lse``; with
    ``aux`` also c [B,Hq,T] and vbar [B,Hq,T,d] (the backward's auxiliaries).
    """
    return _prefill(q, k, v, rho, scale, o=o, lse=lse, aux=aux, ex=None)


def plx_fwd_prefill_ex(q, k, v, rho, scale=None, *, flags=0, cor=True, o=None, lse=True,
                       aux=False):
    """Prefill at a corner of the family (``flags``: PLX_UNIFORM_WEIGHTS |
    PLX_NO_INTERCEPT); with ``cor`` the result also holds cor [B,Hq,T], the
    correction-to-output ratio.  Otherwise as ``plx_fwd_prefill``."""
    return _prefill(q, k, v, rho, scale, o=o, lse=lse, aux=aux, ex=(int(flags), bool(cor)))


def _prefill(q, k, v, rho, scale, *, o, lse, aux, ex):
    torch = _torch()
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    for name, t, shp in (("q", q, (B, Hq, T, d)), ("k", k, (B, Hkv, T, d)),
                         ("v", v, (B, Hkv, T, d)), ("rho", rho, (B, Hq, T, d))):
        _need(t, name, shp, q.dtype, dev)
    if o is not None:
        _need(o, "o", (B, Hq, T, d), torch.float32, dev)
    _need_gpu(dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty((B, Hq, T, d), dtype=torch.float32, device=dev)
    out = {"o": o}
    lse_t = torch.empty((B, Hq, T), dtype=torch.float32, device=dev) if (lse or aux) else None
    c_t = torch.empty((B, Hq, T), dtype=torch.float32, device=dev) if aux else None
    vb_t = torch.empty((B, Hq, T, d), dtype=torch.float32, device=dev) if aux else None
    if ex is None:
        st = lib().plx_fwd_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(rho), _ptr(o), _ptr(lse_t),
                                   _ptr(c_t), _ptr(vb_t), B, Hq, Hkv, T, d, float(scale),
                                   _dtype_code(q), _stream(dev))
        _check(st, "plx_fwd_prefill")
    else:
        flags, want_cor = ex
        cor_t = torch.empty((B, Hq, T), dtype=torch.float32, device=dev) if want_cor else None
        st = lib().plx_fwd_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(rho), _ptr(o), _ptr(lse_t),
                                      _ptr(c_t), _ptr(vb_t), _ptr(cor_t), B, Hq, Hkv, T, d,
                                      float(scale), flags, _dtype_code(q), _stream(dev))
        _check(st, "plx_fwd_prefill_ex")
        if cor_t is not None:
            out["cor"] = cor_t
    if lse_t is not None:
        out["lse"] = lse_t
    if aux:
        out["c"] = c_t
        out["vbar"] = vb_t
    return out


def decode_workspace_size(B, Hq, Hkv, S_max, d, num_splits=0) -> int:
    return int(lib().plx_decode_workspace_size(B, Hq, Hkv, S_max, d, num_splits))


def plx_decode(q, rho, k_cache, v_cache, ctx_len, scale=None, *, num_splits=0, workspace=None,
               o=None, lse=True):
    """Decode.  q, rho [B,Hq,d]; caches [B,Hkv,S_max,d]; ctx_len int32 [B] on the device."""
    return _decode(q, rho, k_cache, v_cache, ctx_len, scale, num_splits=num_splits,
                   workspace=workspace, o=o, lse=lse, ex=None)


def plx_decode_ex(q, rho, k_cache, v_cache, ctx_len, scale=None, *, flags=0, cor=True,
                  num_splits=0, workspace=None, o=None, lse=True):
    """Decode at a corner of the family; with ``cor`` the result also holds
    cor [B,Hq].  Otherwise as ``plx_decode``."""
    return _decode(q, rho, k_cache, v_cache, ctx_len, scale, num_splits=num_splits,
                   workspace=workspace, o=o, lse=lse, ex=(int(flags), bool(cor)))


def _decode(q, rho, k_cache, v_cache, ctx_len, scale, *, num_splits, workspace, o, lse, ex):
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError(f"q must be [B, Hq, d] and the caches [B, Hkv, S_max, d]; got "
                         f"{tuple(q.shape)} and {tuple(k_cache.shape)}")
    B, Hq, d = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    _need(q, "q", (B, Hq, d), q.dtype, dev)
    _need(rho, "rho", (B, Hq, d), q.dtype, dev)
    _need(k_cache, "k_cache", (B, Hkv, S_max, d), q.dtype, dev)
    _need(v_cache, "v_cache", (B, Hkv, S_max, d), q.dtype, dev)
    _need(ctx_len, "ctx_len", (B,), torch.int32, dev)
    if o is not None:
        _need(o, "o", (B, Hq, d), torch.float32, dev)
    _need_gpu(dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = decode_workspace_size(B, Hq, Hkv, S_max, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    else:
        _need_workspace(workspace, dev, need)
    if o is None:
        o = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    lse_t = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse else None
    ws_bytes = workspace.numel() * workspace.element_size()
    out = {"o": o}
    if ex is None:
        st = lib().plx_decode(_ptr(q), _ptr(rho), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len),
                              _ptr(o), _ptr(lse_t), B, Hq, Hkv, S_max, d, float(scale),
                              int(num_splits), _ptr(workspace), ws_bytes, _dtype_code(q),
                              _stream(dev))
        _check(st, "plx_decode")
    else:
        flags, want_cor = ex
        cor_t = torch.empty((B, Hq), dtype=torch.float32, device=dev) if want_cor else None
        st = lib().plx_decode_ex(_ptr(q), _ptr(rho), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len),
                                 _ptr(o), _ptr(lse_t), _ptr(cor_t), B, Hq, Hkv, S_max, d,
                                 float(scale), int(num_splits), flags, _ptr(workspace), ws_bytes,
                                 _dtype_code(q), _stream(dev))
        _check(st, "plx_decode_ex")
        if cor_t is not None:
            out["cor"] = cor_t
    if lse_t is not None:
        out["lse"] = lse_t
    return out


# Size limit of plx_decode_noalloc's records (PLX_DECODE_SCRATCH_BYTES).
DECODE_SCRATCH_BYTES = 16 << 20


def plx_decode_noalloc(q, rho, k_cache, v_cache, ctx_len, scale=None, *, num_splits=0, o=None,
                       lse=True):
    """Decode with the partial records in the library's own per-GPU buffer
    (no workspace argument; the C call allocates nothing).  Same arguments and
    results as ``plx_decode``; calls that overlap on one GPU race.  Outputs not
    supplied are allocated here, by torch, before the call."""
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError(f"q must be [B, Hq, d] and the caches [B, Hkv, S_max, d]; got "
                         f"{tuple(q.shape)} and {tuple(k_cache.shape)}")
    B, Hq, d = q.shape
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    _need(q, "q", (B, Hq, d), q.dtype, dev)
    _need(rho, "rho", (B, Hq, d), q.dtype, dev)
    _need(k_cache, "k_cache", (B, Hkv, S_max, d), q.dtype, dev)
    _need(v_cache, "v_cache", (B, Hkv, S_max, d), q.dtype, dev)
    _need(ctx_len, "ctx_len", (B,), torch.int32, dev)
    if o is not None:
        _need(o, "o", (B, Hq, d), torch.float32, dev)
    _need_gpu(dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    lse_t = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse else None
    st = lib().plx_decode_noalloc(_ptr(q), _ptr(rho), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len),
                                  _ptr(o), _ptr(lse_t), B, Hq, Hkv, S_max, d, float(scale),
                                  int(num_splits), _dtype_code(q), _stream(dev))
    _check(st, "plx_decode_noalloc")
    out = {"o": o}
    if lse_t is not None:
        out["lse"] = lse_t
    return out


def plx_qkvr_proj(x, w, Hq, Hkv, d, *, out=None):
    """Stacked projection.  x [B,T,D] bf16; w [(2Hq+2Hkv)d, D] bf16 (rows W_Q,
    W_K, W_V, W_R).  Returns dict(q, k, v, rho) in the [B,H,T,d] layout (bf16)."""
    torch = _torch()
    B, T, D = x.shape
    dev = x.device
    N = (2 * Hq + 2 * Hkv) * d
    _need(x, "x", (B, T, D), x.dtype, dev)
    _need(w, "w", (N, D), x.dtype, dev)
    if out is None:
        out = {
            "q": torch.empty((B, Hq, T, d), dtype=x.dtype, device=dev),
            "k": torch.empty((B, Hkv, T, d), dtype=x.dtype, device=dev),
            "v": torch.empty((B, Hkv, T, d), dtype=x.dtype, device=dev),
            "rho": torch.empty((B, Hq, T, d), dtype=x.dtype, device=dev),
        }
    for n, H in (("q", Hq), ("k", Hkv), ("v", Hkv), ("rho", Hq)):
        _need(out[n], n, (B, H, T, d), x.dtype, dev)
    _need_gpu(dev)
    st = lib().plx_qkvr_proj(_ptr(x), _ptr(w), _ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]),
                             _ptr(out["rho"]), B, T, D, Hq, Hkv, d, _dtype_code(x), _stream(dev))
    _check(st, "plx_qkvr_proj")
    return out


def bwd_workspace_size(B, Hq, Hkv, T, d) -> int:
    return int(lib().plx_bwd_workspace_size(B, Hq, Hkv, T, d))


def plx_bwd(q, k, v, rho, d_o, o, lse, c, vbar, scale=None, *, workspace=None, grads=None):
    """Backward of the causal prefill; returns dict(dq, dk, dv, drho) in fp32."""
    torch = _torch()
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    for name, t, shp in (("q", q, (B, Hq, T, d)), ("k", k, (B, Hkv, T, d)), ("v", v, (B, Hkv, T, d)),
                         ("rho", rho, (B, Hq, T, d)), ("d_o", d_o, (B, Hq, T, d))):
        _need(t, name, shp, q.dtype, dev)
    for name, t, shp in (("o", o, (B, Hq, T, d)), ("lse", lse, (B, Hq, T)), ("c", c, (B, Hq, T)),
                         ("vbar", vbar, (B, Hq, T, d))):
        _need(t, name, shp, torch.float32, dev)
    if grads is not None:
        for name, shp in (("dq", (B, Hq, T, d)), ("dk", (B, Hkv, T, d)), ("dv", (B, Hkv, T, d)),
                          ("drho", (B, Hq, T, d))):
            if name not in grads:
                raise ValueError(f"grads: missing {name}")
            _need(grads[name], name, shp, torch.float32, dev)
    _need_gpu(dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = bwd_workspace_size(B, Hq, Hkv, T, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    else:
        _need_workspace(workspace, dev, need)
    if grads is None:
        grads = {
            "dq": torch.empty((B, Hq, T, d), dtype=torch.float32, device=dev),
            "dk": torch.empty((B, Hkv, T, d), dtype=torch.float32, device=dev),
            "dv": torch.empty((B, Hkv, T, d), dtype=torch.float32, device=dev),
            "drho": torch.empty((B, Hq, T, d), dtype=torch.float32, device=dev),
        }
    st = lib().plx_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(rho), _ptr(d_o), _ptr(o), _ptr(lse),
                       _ptr(c), _ptr(vbar), _ptr(grads["dq"]), _ptr(grads["dk"]), _ptr(grads["dv"]),
                       _ptr(grads["drho"]), B, Hq, Hkv, T, d, float(scale), _ptr(workspace),
                       workspace.numel() * workspace.element_size(), _dtype_code(q), _stream(dev))
    _check(st, "plx_bwd")
    return grads
