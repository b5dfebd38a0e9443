"""Accuracy measures used to compare the GPU path with the oracle.

"Online Pseudo-average Shifting Attention (PASA) ...", Abstract: accuracy is
assessed through root mean square error against high-precision attention; the
page gives no formula.  Relative RMSE here is ||O_gpu - O_ref||_F / ||O_ref||_F
in float64 over the whole output.
"""
import numpy as np


def nonfinite(x) -> int:
    return int(np.size(x) - np.count_nonzero(np.isfinite(np.asarray(x, np.float64))))


def rel_rmse(out, ref) -> float:
    a = np.asarray(out, np.float64)
    r = np.asarray(ref, np.float64)
    den = np.sqrt(np.sum(r * r))
    if not np.all(np.isfinite(a)):
        return float("inf")
    num = np.sqrt(np.sum((a - r) ** 2))
    return float(num / den) if den > 0 else float(num)


def per_head_rel_rmse(out, ref):
    """out/ref in [B,S,H,D]; returns [B,H] relative RMSE per (batch, head)."""
    a = np.asarray(out, np.float64)
    r = np.asarray(ref, np.float64)
    num = np.sqrt(np.sum((a - r) ** 2, axis=(1, 3)))
    den = np.sqrt(np.sum(r * r, axis=(1, 3)))
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(den > 0, num / den, num)


def lse_error(lse, ref):
    """Largest |lse - ref|, and largest relative error among |ref| > 1e4, over
    entries where the reference is finite; -inf must match -inf exactly."""
    a = np.asarray(lse, np.float64)
    r = np.asarray(ref, np.float64)
    fin = np.isfinite(r)
    mism = int(np.count_nonzero(~fin & (a != r)))
    d = np.abs(a[fin] - r[fin])
    big = np.abs(r[fin]) > 1e4
    rel_big = float(np.max(d[big] / np.abs(r[fin][big]))) if np.any(big) else 0.0
    return (float(d.max()) if d.size else 0.0), rel_big, mism
