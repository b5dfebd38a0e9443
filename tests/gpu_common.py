"""Helpers for the GPU parity tests: run the HIP path and the oracle on the
same seeded fp16 inputs and compare."""
import math
import sys

import numpy as np

import workloads as W
from workloads.metrics import lse_error, nonfinite, rel_rmse

REL_RMSE_MAX = 2e-3      # relative RMSE of O against the binary64 oracle


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


def gather_rows(o, lse, w, rows):
    """o [B,Sq,Hq,D], lse [B,Hq,Sq] -> o[rows] [n,D], lse[rows] [n]."""
    b, rem = np.divmod(rows, w.heads_q * w.seqlen_q)
    h, i = np.divmod(rem, w.seqlen_q)
    return o[b, i, h], lse[b, h, i]
