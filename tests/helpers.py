"""Shared helpers of the GPU parity tests (no attention arithmetic here)."""

from __future__ import annotations

import numpy as np
import torch

from exact_blockwise_long_amd import blockattn as ba
from exact_blockwise_long_amd import synth

# Tolerances.  bf16 output: max abs 2e-2 and mean abs 2e-3.  fp32 path: 1e-5.
# State statistics (a reading: the bf16 output tolerance says nothing about
# m, l): bf16 m abs 1e-3 (m is a max of fp32-accumulated bf16 products),
# LSE abs 1e-2, l relative 2e-2; fp32 m and LSE abs 1e-5, l relative 1e-5.
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
BF16_M, BF16_LSE, BF16_LREL = 1e-3, 1e-2, 2e-2
F32_TOL = 1e-5


def to_device(t: synth.Tensor, device="cuda") -> torch.Tensor:
    return ba.from_host(t.storage, t.dtype == "bf16", device)


def host(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def err_stats(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def assert_bf16_out(got, ref, what=""):
    mx, mn = err_stats(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert mx <= BF16_MAX and mn <= BF16_MEAN, f"{what}: max abs {mx:.3e} mean abs {mn:.3e}"
    return mx, mn


def assert_close(got, ref, atol, what="", rel=False):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    same_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    with np.errstate(invalid="ignore"):  # inf - inf where both are the same infinity; masked out
        d = np.where(same_inf, 0.0, np.abs(got - ref))
    if rel:
        d = d / np.maximum(np.abs(ref), 1e-30)
        d = np.where(same_inf | ((ref == 0) & (got == 0)), 0.0, d)
    bad = ~(d <= atol)
    assert not bad.any(), f"{what}: worst {np.nanmax(np.where(bad, np.nan_to_num(d, nan=np.inf), 0))} " \
                          f"at {np.argwhere(bad)[:3].tolist()}"
