"""Accuracy measures used to compare the GPU path with the oracle.

"Online Pseudo-average Shifting Attention (PASA) ...", Abstract: accuracy is
assessed through root mean square error against high-precision attention; the
page gives no formula.  Relative RMSE here is ||O_gpu - O_ref||_F / ||O_ref||_F
in float64 over the whole output.  The same measure is also taken per
(batch, head) and per query row, so that a defect confined to a few rows or
one head cannot hide inside the norm of a large tensor ("Is Flash Attention
Stable?", summary: deviation measured against a high-precision reference in an
isolated forward pass).
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


def grouped_rel_rmse(out, ref, groups):
    """out/ref [n, D] rows with a group label each (e.g. the flat (b, h) index
    of a sampled row); returns {label: relative RMSE over that group's rows}."""
    a = np.asarray(out, np.float64)
    r = np.asarray(ref, np.float64)
    g = np.asarray(groups)
    res = {}
    for lab in np.unique(g):
        sel = g == lab
        num = np.sqrt(np.sum((a[sel] - r[sel]) ** 2))
        den = np.sqrt(np.sum(r[sel] ** 2))
        res[int(lab)] = float(num / den) if den > 0 else float(num)
    return res


def row_rel_err(out, ref, floor):
    """Per-row error ||o_i - r_i|| / max(||r_i||, floor) over the last axis.

    A row whose reference nearly cancels (a small weighted mean of values) is
    measured against `floor` instead of its own tiny norm; callers pass a
    fraction of the typical norm of a value row."""
    a = np.asarray(out, np.float64)
    r = np.asarray(ref, np.float64)
    num = np.sqrt(np.sum((a - r) ** 2, axis=-1))
    den = np.maximum(np.sqrt(np.sum(r * r, axis=-1)), floor)
    return num / den


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
