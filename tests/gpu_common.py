"""Helpers for the GPU parity tests: run the HIP path and the oracle on the
same seeded fp16 inputs and compare.

Every comparison of an output O with the oracle applies four gates
(`check_o`), because a single norm over a large tensor can hide a defect
confined to a few rows ("Online Pseudo-average Shifting Attention (PASA) ...",
Abstract: RMSE against high-precision attention):
  * no inf/NaN in O;
  * relative RMSE over the whole output  <= REL_RMSE_MAX (2e-3);
  * relative RMSE of every (batch, head)  <= REL_RMSE_MAX, for heads with
    at least MIN_ROWS_PER_HEAD rows in the comparison (a head of a decode
    output is a single row and is gated as a row);
  * the worst row's relative error       <= ROW_REL_MAX (1e-2), where a row
    whose reference nearly cancels is measured against a quarter of the
    norm of a typical value row instead of its own norm.
The row bound: the fp16 rounding of an output element is at most 2^-11
relative, and the weights' fp16 roundings (exponent argument, exponential)
move a row by a few 1e-4 on these inputs.  Where scores reach ~2e5 (the
key-bias jump recipe) the matrix cores' fp32 accumulation of each score is
off by a few 1e-2 in the score, i.e. a few 1e-3 in its weight, and a row
whose weight is shared by two nearly tied keys carries that almost fully
(up to ~2e-3 measured); a head's RMSE over many rows averages it out, a
single row does not.  1e-2 leaves a wide margin while a single wrong 16-byte
chunk (8 of 64 or 128 values) moves its row by 0.1 or more.
"""
import sys

import numpy as np

import workloads as W
from workloads.metrics import (grouped_rel_rmse, lse_error, nonfinite, per_head_rel_rmse,
                               rel_rmse, row_rel_err)

REL_RMSE_MAX = 2e-3      # relative RMSE of O against the binary64 oracle
ROW_REL_MAX = 1e-2       # worst single row (see the module docstring)
MIN_ROWS_PER_HEAD = 32   # heads with fewer rows compared are reported, not gated


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_gpu(*arrs):
    import torch
    return [torch.from_numpy(a).cuda() for a in arrs]


def lse_ok(lse, ref, abs_tol=1e-2, rel_tol=1e-6):
    """|dlse| <= abs_tol, or <= rel_tol*|lse| where |lse| > 1e4; -inf must match."""
    a = np.asarray(lse, np.float64)
    r = np.asarray(ref, np.float64)
    fin = np.isfinite(r)
    if np.any(a[~fin] != r[~fin]):
        return False
    d = np.abs(a[fin] - r[fin])
    tol = np.maximum(abs_tol, rel_tol * np.abs(r[fin]))
    return bool(np.all(d <= tol))


def value_floor(v):
    """A quarter of the RMS norm of a value row: the denominator floor of the
    per-row relative error."""
    vf = np.asarray(v, np.float64)
    return 0.25 * float(np.sqrt(np.mean(vf * vf) * vf.shape[-1]))


def check_o(o, ro, v, heads=None, label="", rel_max=REL_RMSE_MAX, row_max=ROW_REL_MAX):
    """Gate an output against the oracle (see the module docstring).

    o, ro: [B,S,H,D] full outputs, or [n,D] sampled rows with `heads` giving
    each row's flat (batch, head) index.  Returns the measured figures."""
    o = np.asarray(o)
    ro = np.asarray(ro)
    bad = nonfinite(o)
    glob = rel_rmse(o, ro)
    rows = row_rel_err(o, ro, value_floor(v))
    if heads is None:
        ph = per_head_rel_rmse(o, ro).ravel()
        gated = ph if o.shape[1] >= MIN_ROWS_PER_HEAD else np.zeros(0)
    else:
        g = grouped_rel_rmse(o, ro, heads)
        ph = np.array(list(g.values()))
        counts = {lab: int(np.sum(np.asarray(heads) == lab)) for lab in g}
        gated = np.array([g[lab] for lab in g if counts[lab] >= MIN_ROWS_PER_HEAD])
    res = dict(nonfinite=bad, rel_rmse=glob, head_max=float(ph.max()) if ph.size else 0.0,
               row_max=float(rows.max()) if rows.size else 0.0)
    say(label, "rel_rmse %.3e  worst head %.3e  worst row %.3e  nonfinite %d"
        % (glob, res["head_max"], res["row_max"], bad))
    assert bad == 0, res
    assert glob <= rel_max, res
    if gated.size:
        assert float(gated.max()) <= rel_max, res
    assert res["row_max"] <= row_max, res
    return res


def sample_rows(w, n, rng):
    """Row ids (b*Hq + h)*Sq + i: random rows plus first/last rows of tiles."""
    total = w.batch * w.heads_q * w.seqlen_q
    picks = set(rng.choice(total, min(n, total), replace=False).tolist())
    for b in range(w.batch):
        for h in (0, w.heads_q - 1):
            for i in (0, 1, 127, 128, w.seqlen_q // 2, w.seqlen_q - 1):
                if 0 <= i < w.seqlen_q:
                    picks.add((b * w.heads_q + h) * w.seqlen_q + i)
    return np.array(sorted(picks), np.int64)


def head_rows(w, heads, frac_others, rng):
    """All rows of the given flat (batch, head) indices, plus a random fraction
    of the rows of every other head (at least one row each)."""
    Sq = w.seqlen_q
    out = []
    for bh in range(w.batch * w.heads_q):
        if bh in heads:
            out.append(bh * Sq + np.arange(Sq, dtype=np.int64))
        else:
            m = max(1, int(round(frac_others * Sq)))
            out.append(bh * Sq + np.sort(rng.choice(Sq, m, replace=False)).astype(np.int64))
    return np.concatenate(out)


def row_heads(w, rows):
    """Flat (batch, head) index of each flat row id."""
    return np.asarray(rows) // w.seqlen_q


def gather_rows(o, lse, w, rows):
    """o [B,Sq,Hq,D], lse [B,Hq,Sq] -> o[rows] [n,D], lse[rows] [n]."""
    b, rem = np.divmod(rows, w.heads_q * w.seqlen_q)
    h, i = np.divmod(rem, w.seqlen_q)
    return o[b, i, h], lse[b, h, i]
