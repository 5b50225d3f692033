"""Comparison helpers for the parity tests (GPU result vs the fp64 oracle).

Tolerances: coefficients |gpu - oracle| <= 1e-4 |oracle| elementwise;
bf16 outputs |gpu - oracle| <= 1e-2 * max(|oracle|, rms of the oracle row)
(a row-RMS floor, because cancellation in sums makes isolated elements tiny
while the row's scale fixes the absolute rounding error).  Denominators are
floored at the smallest normal binary64 value, so an all-zero oracle row
requires exact zeros.
"""
import numpy as np
import torch

COEF_RTOL = 1e-4
BF16_RTOL = 1e-2


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


# Floor of the denominators: an all-zero oracle row (an exactly cancelling
# pre combination gives h = 0) then demands exact zeros instead of 0/0.
TINY = np.finfo(np.float64).tiny


def assert_coeffs_close(gpu, ref, rtol=COEF_RTOL, what="coeffs"):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    err = np.abs(gpu - ref) / np.maximum(np.abs(ref), TINY)
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    assert err.max() <= rtol, f"{what}: max rel err {err.max():.3e} at {worst} (gpu {gpu[worst]!r}, oracle {ref[worst]!r})"
    return float(err.max())


def bf16_rel_err(gpu, ref):
    """Elementwise error relative to max(|ref|, rms of the ref row)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    row_rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    return np.abs(gpu - ref) / np.maximum(np.maximum(np.abs(ref), row_rms), TINY)


def assert_bf16_close(gpu, ref, rtol=BF16_RTOL, what="bf16"):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    err = bf16_rel_err(gpu, ref)
    worst = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= rtol, f"{what}: max rel err {err.max():.3e} at {worst} (gpu {gpu[worst]!r}, oracle {ref[worst]!r})"
    return float(err.max())
