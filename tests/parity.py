"""Comparison rules between the GPU path and the fp64 oracle.

Tolerances (per element, |gpu - oracle| <= bound):
  per-token values (loss, KL, entropy, log-probabilities):
      fp32 inputs:       1e-6 + 1e-5 * |oracle|
      bf16/fp16 inputs:  1e-5 + 2e-4 * |oracle|
  gradients:
      fp32 inputs:       1e-7 + 1e-4 * |oracle|
      bf16/fp16 inputs:  one unit in the last place of the output dtype at the
                         oracle value, + 1e-6
  row statistics: max bit-exact; ln sum exp within 4e-6 (fp32 accumulation over
      up to 2^17 terms).
Masking decisions are exact: NaN and +-inf where the oracle has them, and exactly
0 gradient wherever the oracle's is exactly 0 because of a -inf logit or an
undefined row.
"""
from __future__ import annotations

import math

import numpy as np
import torch

MANT = {torch.bfloat16: 7, torch.float16: 10}
EMIN = {torch.bfloat16: -126, torch.float16: -14}


def value_bounds(ref: np.ndarray, dtype) -> np.ndarray:
    if dtype == torch.float32:
        return 1e-6 + 1e-5 * np.abs(ref)
    return 1e-5 + 2e-4 * np.abs(ref)


def ulp(ref: np.ndarray, dtype) -> np.ndarray:
    a = np.abs(ref)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, EMIN[dtype])
    return np.exp2(e - MANT[dtype])


def grad_bounds(ref: np.ndarray, dtype) -> np.ndarray:
    if dtype == torch.float32:
        return 1e-7 + 1e-4 * np.abs(ref)
    return ulp(ref, dtype) + 1e-6


def _np(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def assert_special_pattern(gpu, ref, what):
    """NaN and infinities must sit exactly where the oracle puts them."""
    assert np.array_equal(np.isnan(gpu), np.isnan(ref)), f"{what}: NaN pattern differs"
    for sign in (1, -1):
        assert np.array_equal(gpu == sign * math.inf, ref == sign * math.inf), \
            f"{what}: infinity pattern differs"


def assert_values(gpu, ref, dtype, what="value"):
    g, r = _np(gpu), _np(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert_special_pattern(g, r, what)
    fin = np.isfinite(r)
    err = np.abs(g[fin] - r[fin])
    bound = value_bounds(r[fin], dtype)
    bad = err > bound
    if bad.any():
        i = np.argmax(err - bound)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst gpu="
                             f"{g[fin][i]!r} oracle={r[fin][i]!r} err={err[i]:.3e} "
                             f"bound={bound[i]:.3e}")


def temperature_grad_scale(dtype, temperature: float) -> float:
    """Factor on the fp32 gradient bound at a temperature: the kernels round the
    exponent argument of the tempered logits x / T, whose magnitude (and so whose fp32
    rounding error) grows as 1 / T; T >= 1 leaves the bound unchanged.  16-bit
    gradients are bounded by their own output rounding and are not scaled."""
    return max(1.0, 1.0 / temperature) if dtype == torch.float32 else 1.0


def assert_grads(gpu, ref, dtype, what="grad", exact_zero=None, scale=1.0):
    """``exact_zero``: boolean mask of positions whose gradient must be exactly 0;
    ``scale`` multiplies the bound (temperature_grad_scale)."""
    g, r = _np(gpu), _np(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert not np.isnan(g[~np.isnan(r)]).any(), f"{what}: NaN where the oracle is finite"
    if exact_zero is not None:
        assert np.all(g[exact_zero] == 0.0), f"{what}: masked positions not exactly 0"
    fin = np.isfinite(r)
    err = np.abs(g[fin] - r[fin])
    bound = grad_bounds(r[fin], dtype) * scale
    bad = err > bound
    if bad.any():
        i = np.argmax(err - bound)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst gpu="
                             f"{g[fin][i]!r} oracle={r[fin][i]!r} err={err[i]:.3e} "
                             f"bound={bound[i]:.3e}")


def grad_ulp_report(gpu, ref, dtype, quantile=1.0) -> float:
    """Error in units of the output dtype's last place at the given quantile
    (diagnostic: gradients that suffer cancellation in fp32 can exceed 1 ulp)."""
    g, r = _np(gpu), _np(ref)
    fin = np.isfinite(r) & (np.abs(r) > 1e-30)
    if dtype == torch.float32 or not fin.any():
        return 0.0
    return float(np.quantile(np.abs(g[fin] - r[fin]) / ulp(r[fin], dtype), quantile))


def assert_stats(gpu_stats, m_ref, lz_ref, side=0, what="stats"):
    st = _np(gpu_stats)
    m = st[:, 2 * side]
    lz = st[:, 2 * side + 1]
    assert np.array_equal(m, m_ref), f"{what}: row max differs"
    fin = np.isfinite(lz_ref)
    assert np.array_equal(np.isfinite(lz), fin), f"{what}: undefined rows differ"
    assert np.all(lz[~fin] == lz_ref[~fin])
    err = np.abs(lz[fin] - lz_ref[fin])
    assert err.max(initial=0.0) <= 4e-6, f"{what}: ln sum exp off by {err.max():.3e}"


def sample_rows(N: int, n: int, seed: int, must=()) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = set(int(r) for r in must if 0 <= r < N)
    rows.update({0, N - 1})
    rows.update(int(r) for r in rng.choice(N, size=min(n, N), replace=False))
    return np.array(sorted(rows), dtype=np.int64)
