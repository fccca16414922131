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


def check_fp32(got, ref, what):
    """|d| <= 1e-5 * max(|ref|, 1), elementwise (forward outputs)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = FP32_REL * np.maximum(np.abs(ref), 1.0)
    worst = float(np.max(err / bound)) if err.size else 0.0
    assert np.all(err <= bound), f"{what}: max |d|/bound = {worst:.3f} (max |d| {err.max():.3e})"
    return float(err.max()) if err.size else 0.0


U32 = 2.0 ** -24  # fp32 unit roundoff


def check_fp32_grad(got, ref, mag, n_terms, what):
    """fp32 gradients: |d| <= 1e-5 * max(|ref|, 1) + gamma * mag, elementwise.

    A gradient element is a sum of n_terms products (one per query row and
    head for dK / dV, one per key for dQ / drho) whose factors are themselves
    fp32 dot products over d.  ``mag`` is the oracle's per-element sum of the
    absolute values of those products (``prefill_backward_group`` with
    ``magnitudes``), and gamma = n_terms * u with u = 2^-24 is the first-order
    worst-case bound for evaluating such a sum in fp32 (|fl(sum x) - sum x| <=
    gamma_n sum |x|).  The 1e-5 relative bar applies on top of it; where the
    terms do not cancel, mag ~ |ref| and the second term is small."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape == np.shape(mag), (what, got.shape, ref.shape, np.shape(mag))
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = FP32_REL * np.maximum(np.abs(ref), 1.0) + n_terms * U32 * np.asarray(mag)
    worst = float(np.max(err / bound)) if err.size else 0.0
    say(f"  {what}: max |d| {err.max():.3e}  max |d|/bound {worst:.3f}  max|ref| {np.abs(ref).max():.3e}")
    assert np.all(err <= bound), f"{what}: max |d|/bound = {worst:.3f} (max |d| {err.max():.3e})"
    return float(err.max()) if err.size else 0.0


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
