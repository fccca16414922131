"""Shared test helpers: moving generated inputs to the device and the parity bars."""

from __future__ import annotations

import sys

import numpy as np

# Parity bars.  fp32: elementwise |d| <= 1e-5 * max(|ref|, 1).  bf16 inputs with
# fp32 accumulation: max-abs <= 2e-2 and mean-abs <= 2e-3 per output tensor.
FP32_REL = 1e-5
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
LSE_ABS = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(t, device="cuda"):
    """inputs.Tensor -> torch tensor on ``device`` with the kernel dtype."""
    import torch

    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(t.data)).to(device)


def check_fp32(got, ref, what, floor=1.0):
    """|d| <= 1e-5 * max(|ref|, floor), elementwise.  Forward outputs use
    floor = 1; gradient tensors, which are sums of up to T*G terms that cancel,
    pass floor = RMS of the reference tensor (see grad_floor)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = FP32_REL * np.maximum(np.abs(ref), floor)
    worst = float(np.max(err / bound)) if err.size else 0.0
    assert np.all(err <= bound), f"{what}: max |d|/bound = {worst:.3f} (max |d| {err.max():.3e})"
    return float(err.max()) if err.size else 0.0


def grad_floor(ref):
    ref = np.asarray(ref, dtype=np.float64)
    return max(1.0, float(np.sqrt(np.mean(ref * ref)))) if ref.size else 1.0


def check_bf16(got, ref, what, max_abs=BF16_MAX_ABS, mean_abs=BF16_MEAN_ABS):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mn = float(err.max()), float(err.mean())
    say(f"  {what}: max-abs {mx:.3e}  mean-abs {mn:.3e}  max|ref| {np.abs(ref).max():.3e}")
    assert mx <= max_abs, f"{what}: max-abs {mx:.3e} > {max_abs}"
    assert mn <= mean_abs, f"{what}: mean-abs {mn:.3e} > {mean_abs}"
    return mx, mn
