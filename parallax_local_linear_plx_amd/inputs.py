"""Seeded synthetic inputs for the Parallax operator.

This module only draws random numbers and rounds them to the storage dtype
the kernels receive.  It holds none of the operator's arithmetic, so both the
HIP path and the fp64 CPU oracle can consume what it produces.

Draw recipe (one ``numpy.random.SeedSequence(seed)`` per workload):

* the root sequence is spawned into fixed roles, in this order:
  ``ctx_len, q, k, v, rho (or x), w_r, d_o, x_in, w_qkvr`` (the last two for
  the stacked projection in front of the operator);
* every large tensor is drawn per leading ``(b, h)`` slice from a further
  ``spawn`` of its role, so any slice can be regenerated on its own and the
  slices can be filled by threads in parallel;
* values are drawn in fp32 and rounded once, round-to-nearest-even, to bf16
  where the workload is bf16; the oracle upcasts exactly those rounded values.

The distributions are the ones the Parallax write-ups' workloads use:
q, k, v ~ N(0, 1); the probe rho ~ N(0, 0.1^2) per component, or, for the
projected-probe prefill, rho_i = W_R x_i with x ~ N(0, 1) in R^1024 and
W_R ~ N(0, 1/1024) per head (a plain projection outside the operator).
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# Fixed role order inside one workload's SeedSequence.
_ROLES = ("ctx_len", "q", "k", "v", "rho", "w_r", "d_o", "x_in", "w_qkvr")


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exactly equal fp32 values."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Tensor:
    """A generated input: storage bits plus its exact fp64 value on demand."""

    dtype: str  # "f32" or "bf16"
    data: np.ndarray  # float32 array ("f32") or uint16 bf16 bit patterns ("bf16")

    @property
    def shape(self):
        return self.data.shape

    def f64(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.data).astype(np.float64)
        return self.data.astype(np.float64)

    def f64_slice(self, idx) -> np.ndarray:
        sub = self.data[idx]
        if self.dtype == "bf16":
            return bf16_bits_to_f32(np.asarray(sub)).astype(np.float64)
        return np.asarray(sub).astype(np.float64)


def _fill_normal(seq: np.random.SeedSequence, shape, std: float, dtype: str,
                 valid_rows=None, fill_bits: int = 0x7FC0) -> Tensor:
    """N(0, std^2) draw over ``shape``; one spawned stream per (i0, i1) slice.

    ``valid_rows`` (optional, per leading index i0) limits the draw to the first
    ``valid_rows[i0]`` rows of each slice's third axis; the rest is filled with
    ``fill_bits`` (a bf16 quiet NaN by default), so reads past a ragged end show.
    """
    shape = tuple(int(s) for s in shape)
    n0, n1 = shape[0], shape[1]
    rest = shape[2:]
    children = seq.spawn(n0 * n1)
    if dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
    else:
        out = np.empty(shape, dtype=np.float32)

    def work(flat):
        i0, i1 = divmod(flat, n1)
        g = np.random.default_rng(children[flat])
        if valid_rows is None:
            vals = g.standard_normal(rest, dtype=np.float32)
            if std != 1.0:
                vals *= np.float32(std)
            out[i0, i1] = bf16_round_bits(vals) if dtype == "bf16" else vals
        else:
            nv = int(valid_rows[i0])
            vals = g.standard_normal((nv,) + rest[1:], dtype=np.float32)
            if std != 1.0:
                vals *= np.float32(std)
            if dtype == "bf16":
                out[i0, i1, :nv] = bf16_round_bits(vals)
                out[i0, i1, nv:] = np.uint16(fill_bits)
            else:
                out[i0, i1, :nv] = vals
                out[i0, i1, nv:] = np.float32(np.nan)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(n0 * n1)))
    return Tensor(dtype, out)


@dataclass
class Workload:
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    d: int
    scale: float
    T: int = 0  # prefill / training sequence length
    S_max: int = 0  # decode cache capacity
    tensors: dict = field(default_factory=dict)
    ctx_len: np.ndarray | None = None


def _roles(seed: int):
    kids = np.random.SeedSequence(seed).spawn(len(_ROLES))
    return dict(zip(_ROLES, kids))


def make_prefill(B, Hq, Hkv, T, d, dtype="bf16", seed=0, rho_std=0.1,
                 rho_projected=False, x_dim=1024, with_grad=False, scale=None,
                 name="prefill") -> Workload:
    """Causal prefill (and optionally training-step) inputs, layout [B, H, T, d]."""
    r = _roles(seed)
    wl = Workload(name, dtype, B, Hq, Hkv, d,
                  scale if scale is not None else 1.0 / np.sqrt(d), T=T)
    wl.tensors["q"] = _fill_normal(r["q"], (B, Hq, T, d), 1.0, dtype)
    wl.tensors["k"] = _fill_normal(r["k"], (B, Hkv, T, d), 1.0, dtype)
    wl.tensors["v"] = _fill_normal(r["v"], (B, Hkv, T, d), 1.0, dtype)
    if rho_projected:
        wl.tensors["rho"] = _projected_probe(r["rho"], r["w_r"], B, Hq, T, d, x_dim, dtype)
    else:
        wl.tensors["rho"] = _fill_normal(r["rho"], (B, Hq, T, d), rho_std, dtype)
    if with_grad:
        wl.tensors["d_o"] = _fill_normal(r["d_o"], (B, Hq, T, d), 1.0, dtype)
    return wl


def make_projection(B, T, D, Hq, Hkv, d, dtype="bf16", seed=0, name="projection") -> Workload:
    """Layer input x [B, T, D] ~ N(0, 1) and the stacked weight
    [W_Q; W_K; W_V; W_R] [(2 Hq + 2 Hkv) d, D] ~ N(0, 1/D), so every projected
    component is ~ N(0, 1) like the operator's q, k, v and projected rho."""
    r = _roles(seed)
    N = (2 * Hq + 2 * Hkv) * d
    wl = Workload(name, dtype, B, Hq, Hkv, d, 1.0 / np.sqrt(d), T=T)
    wl.tensors["x"] = _fill_normal(r["x_in"], (B, T, D), 1.0, dtype)
    w = _fill_normal(r["w_qkvr"], (1, N, D), 1.0 / np.sqrt(D), dtype)
    wl.tensors["w"] = Tensor(w.dtype, w.data.reshape(N, D))
    return wl


def _projected_probe(seq_x, seq_w, B, Hq, T, d, x_dim, dtype) -> Tensor:
    """rho[b,h,t] = W_R[h] x[b,t]: x ~ N(0,1)^x_dim per token, W_R ~ N(0, 1/x_dim).

    The projection is an ordinary linear layer that sits before the operator;
    it is evaluated here in fp32 only to give the probe its distribution.
    """
    xs = seq_x.spawn(B)
    ws = seq_w.spawn(Hq)
    x = np.empty((B, T, x_dim), np.float32)
    w = np.empty((Hq, d, x_dim), np.float32)

    def fx(b):
        x[b] = np.random.default_rng(xs[b]).standard_normal((T, x_dim), dtype=np.float32)

    def fw(h):
        w[h] = np.random.default_rng(ws[h]).standard_normal((d, x_dim), dtype=np.float32)
        w[h] *= np.float32(1.0 / np.sqrt(x_dim))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fx, range(B)))
        list(ex.map(fw, range(Hq)))
    rho = np.empty((B, Hq, T, d), np.float32)
    for b in range(B):
        for h in range(Hq):
            rho[b, h] = x[b] @ w[h].T
    if dtype == "bf16":
        return Tensor("bf16", bf16_round_bits(rho))
    return Tensor("f32", rho)


def make_decode(B, Hq, Hkv, d, ctx, S_max=None, dtype="bf16", seed=0, rho_std=0.1,
                ctx_range=None, scale=None, name="decode", ctx_list=None) -> Workload:
    """One new query and probe per sequence against a [B, Hkv, S_max, d] KV cache.

    ``ctx`` is the uniform context length, or ignored when ``ctx_range=(lo, hi)``
    is given: then ctx_len[b] ~ U{lo..hi}, both ends inclusive, drawn first;
    ``ctx_list`` gives the lengths explicitly.
    Cache rows at or beyond ctx_len[b] hold bf16 NaN canaries.
    """
    r = _roles(seed)
    if ctx_list is not None:
        ctx_len = np.asarray(ctx_list, dtype=np.int32)
    elif ctx_range is not None:
        lo, hi = ctx_range
        ctx_len = np.random.default_rng(r["ctx_len"]).integers(lo, hi, size=B,
                                                               endpoint=True).astype(np.int32)
    else:
        ctx_len = np.full(B, ctx, np.int32)
    if S_max is None:
        S_max = int(ctx_len.max())
    wl = Workload(name, dtype, B, Hq, Hkv, d,
                  scale if scale is not None else 1.0 / np.sqrt(d), S_max=S_max)
    wl.ctx_len = ctx_len
    wl.tensors["q"] = _fill_normal(r["q"], (B, Hq, 1, d), 1.0, dtype)
    wl.tensors["k"] = _fill_normal(r["k"], (B, Hkv, S_max, d), 1.0, dtype, valid_rows=ctx_len)
    wl.tensors["v"] = _fill_normal(r["v"], (B, Hkv, S_max, d), 1.0, dtype, valid_rows=ctx_len)
    wl.tensors["rho"] = _fill_normal(r["rho"], (B, Hq, 1, d), rho_std, dtype)
    # q and rho are stored [B, Hq, 1, d]; the decode ABI reads them as [B, Hq, d].
    return wl


# ---------------------------------------------------------------------------
# The five workloads of the Parallax operator, by what they are.
# ---------------------------------------------------------------------------

def fp32_single_head(seed=1, T=128, d=64):
    """Single-head causal forward in fp32: B=1, H=1, T=128, d=64, rho ~ N(0, 0.1^2)."""
    return make_prefill(1, 1, 1, T, d, dtype="f32", seed=seed, scale=1.0 / np.sqrt(64),
                        name="fp32_prefill_B1_H1_T128_d64")


def bf16_prefill(seed=2, B=4, Hq=16, Hkv=8, T=4096, d=128):
    """Causal GQA prefill, bf16 in / fp32 accumulate, rho = W_R x per head."""
    return make_prefill(B, Hq, Hkv, T, d, dtype="bf16", seed=seed, rho_projected=True,
                        name=f"bf16_prefill_B{B}_Hq{Hq}_Hkv{Hkv}_T{T}_d{d}")


def bf16_decode(seed=3, B=64, Hq=16, Hkv=8, ctx=8192, d=128):
    """Batched decode over a uniform-length KV cache."""
    return make_decode(B, Hq, Hkv, d, ctx, dtype="bf16", seed=seed,
                       name=f"bf16_decode_B{B}_Hq{Hq}_Hkv{Hkv}_ctx{ctx}_d{d}")


def bf16_long_decode(seed=4, B=8, Hq=16, Hkv=8, lo=16384, hi=131072, d=128, S_max=131072):
    """Long-context decode, ragged contexts ~ U{lo..hi}, split over workgroups."""
    return make_decode(B, Hq, Hkv, d, 0, S_max=S_max, dtype="bf16", seed=seed,
                       ctx_range=(lo, hi),
                       name=f"bf16_long_decode_B{B}_Hq{Hq}_Hkv{Hkv}_ctx{lo}-{hi}_d{d}")


def bf16_training(seed=5, B=8, Hq=16, Hkv=8, T=4096, d=128):
    """Training step: causal forward + backward with upstream dO ~ N(0, 1)."""
    return make_prefill(B, Hq, Hkv, T, d, dtype="bf16", seed=seed, with_grad=True,
                        name=f"bf16_train_B{B}_Hq{Hq}_Hkv{Hkv}_T{T}_d{d}")


# ---------------------------------------------------------------------------
# Device-side draws for timing runs (same shapes and distributions, seeded
# torch generators on the GPU, so multi-GB caches need no host round trip).
# ---------------------------------------------------------------------------

def device_normal(shape, std, seed, device="cuda", dtype="bf16"):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def device_projected_probe(B, Hq, T, d, seed, x_dim=1024, device="cuda"):
    """rho = W_R x on the device: x ~ N(0,1)^x_dim per token, W_R ~ N(0, 1/x_dim) per head."""
    import torch

    x = device_normal((B, T, x_dim), 1.0, seed, device, "f32")
    w = device_normal((Hq, d, x_dim), 1.0 / np.sqrt(x_dim), seed + 1, device, "f32")
    wt = w.transpose(1, 2).contiguous()  # [Hq, x_dim, d], fp32
    rho = torch.matmul(x[:, None], wt[None])  # [B, Hq, T, d]
    return rho.to(torch.bfloat16).contiguous()


def long_decode_ctx(seed=4, B=8, lo=16384, hi=131072):
    """The ragged context lengths of the long-context decode workload (drawn first)."""
    r = _roles(seed)
    return np.random.default_rng(r["ctx_len"]).integers(lo, hi, size=B, endpoint=True).astype(np.int32)
