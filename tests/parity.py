"""Comparison rules shared by the parity tests (test infrastructure).

Float outputs: the tolerance is tol = 1e-2 * rms(oracle) + 1e-3.  Because the
GPU's result is a bf16 value while the oracle's is exact, an element passes
when some real within tol of the oracle value rounds to the GPU's bf16 value:
    |gpu - ref| <= tol + ulp_bf16(gpu) / 2.
The literal max |gpu - bf16(ref)| is reported next to it.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (the gap above |v|'s binade floor)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(a > 0, np.exp2(e - 7.0), np.exp2(-133.0))


def tolerance(ref: np.ndarray) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    return 1e-2 * rms + 1e-3


def compare_bf16(gpu_bits: np.ndarray, ref: np.ndarray, tol: float | None = None):
    """Returns (ok, stats).  gpu_bits: bf16 bit patterns; ref: exact values."""
    g = bf16_to_f64(gpu_bits)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    if tol is None:
        tol = tolerance(ref)
    err = np.abs(g - ref)
    bound = tol + 0.5 * ulp_bf16(g)
    bad = ~(err <= bound)  # NaN fails
    # margin used: the worst error as a fraction of the element's own bound,
    # and the worst error of the rounded result beyond bf16's own rounding
    # of the oracle value (|gpu - bf16(ref)|, in units of tol)
    used = float(np.nanmax(err / bound)) if g.size else 0.0
    excess = np.maximum(err - 0.5 * ulp_bf16(ref), 0.0)
    stats = dict(n=int(g.size), tol=tol, max_err=float(err.max()) if g.size else 0.0,
                 n_bad=int(bad.sum()), rms_ref=float(np.sqrt(np.mean(ref * ref))) if g.size else 0.0,
                 worst_err_over_bound=used,
                 worst_excess_over_tol=float(np.nanmax(excess) / tol) if g.size else 0.0)
    return (not bad.any()), stats


def report(name: str, st: dict) -> None:
    """One line per full-size comparison: the worst error against its bound."""
    print(f"PARITY {name}: n={st['n']} max_err={st['max_err']:.4g} tol={st['tol']:.4g} "
          f"worst err/bound={st['worst_err_over_bound']:.3f} "
          f"worst excess over bf16(ref)/tol={st['worst_excess_over_tol']:.3f} n_bad={st['n_bad']}", flush=True)
