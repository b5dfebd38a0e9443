"""Designed-random sweep: overflow onset and error of the three forward kernels.

The PASA page validates on "designed random benchmarks" ("Online Pseudo-average
Shifting Attention (PASA) ...", Abstract): inputs whose query/key bias,
amplitude and resonance are set on purpose.  This module runs such a grid
through the naive fp16 kernel, the strict PASA variant (fp16 running maximum
and offset) and PASA, and compares each with the binary64 oracle on sampled
rows.  It is test infrastructure (it calls the oracle): `tests/test_sweep_gpu.py`
runs the quick grid with assertions, and

    python -m tests.sweep [--full]

prints one JSON line per grid point (the full grid reaches 131072 keys, twice
the 65504 that one fp16 running sum could hold).

What a point reports
  max_abs_s        largest |q.k| (unscaled) over the rows it was taken on
  s_rows           "all" or "sampled"
  naive_overflow   predicted: some unscaled score rounds to fp16 infinity
                   (|q.k| >= 65520, round-to-nearest-even)
  max_abs_cs       largest |scale * q.k * log2(e)| (the strict variant's range)
  refine_rate      fraction of (row, key block) steps in which PASA's rule
                   re-centres the fp16 tile at the row's own maximum, replayed
                   in binary64 on the sampled rows (the kernels take the same
                   decision in fp32, branch-free, and keep no count)
  <kernel>_nonfinite, <kernel>_rel_rmse   per kernel, on the sampled rows
  <kernel>_head_max, <kernel>_row_max     worst per-head relative RMSE and
                   worst per-row relative error over the sampled rows

`python -m tests.sweep --replay-only [--full]` computes only the columns that
need no GPU (scores, predicted overflow, refine rate).
"""
import argparse
import json
import math

import numpy as np

import workloads as W
from oracle import attn_fp64
from workloads.metrics import grouped_rel_rmse, nonfinite, rel_rmse, row_rel_err

FP16_INF_EDGE = 65520.0          # smallest magnitude that rounds to fp16 infinity
STRICT_RANGE = 3.2e4             # |c * score| below which the strict variant is specified
THETA = 4.0                      # the kernels' refine threshold on the tile maximum (log2 units)


def block_keys(head_dim):
    """Keys per block in the prefill kernels: 128 at head_dim 64, else 64."""
    return 128 if head_dim == 64 else 64


def points(full=False):
    """The grid: bias and amplitude sweeps, resonance amplitudes, sequence
    lengths and head dimensions."""
    pts = []
    # 65504 keys fill one fp16 running sum; 131072 spans four fp32-carried segments
    seqs = (1024, 4096, 16384, 65504, 131072) if full else (512,)
    dims = (64, 128)
    for D in dims:
        for S in seqs:
            for bias in ((0, 10, 20, 25, 30, 35, 40) if full else (0, 20, 30, 40)):
                pts.append(dict(kind="bias", seq=S, D=D, causal=True, bias=float(bias)))
            for amp in ((0.25, 1.0, 2.0, 4.0, 8.0) if full else (0.25, 4.0, 8.0)):
                pts.append(dict(kind="amp_bias", seq=S, D=D, causal=True, amp=amp, bias=20.0))
    for S in seqs:
        for amp in ((16, 32, 48, 64) if full else (16, 48)):
            pts.append(dict(kind="resonance", seq=S, D=64, causal=False, amp=float(amp)))
        # resonance phase offset between query and key (the whole key range
        # offset by the same angle): scores ~ 48^2 * 32 * cos(offset)
        for eighths in ((0, 1, 2, 3, 4, 5, 6, 7, 8) if full else (0, 2, 4, 6, 8)):
            pts.append(dict(kind="phase", seq=S, D=64, causal=False, amp=48.0,
                            offset=eighths * math.pi / 8))
    return pts


def workload(pt, seed):
    S, D = pt["seq"], pt["D"]
    heads = 2 if S <= 4096 else 1
    if pt["kind"] == "bias":
        return W.custom(1, S, S, heads, 1, D, pt["causal"], kind="bias", seed=seed,
                        bias=pt["bias"])
    if pt["kind"] == "amp_bias":
        a, b = pt["amp"], pt["bias"]
        return W.custom(1, S, S, heads, 1, D, pt["causal"], kind="amp_bias", seed=seed,
                        amp_lo=a, amp_hi=a, bias_lo=b, bias_hi=b)
    if pt["kind"] == "phase":
        return W.custom(1, S, S, heads, heads, D, pt["causal"], kind="resonance", seed=seed,
                        amp=pt["amp"], period=64, flip_at=S, per_row_phase=False,
                        phase_offset=pt["offset"])
    return W.custom(1, S, S, heads, heads, D, pt["causal"], kind="resonance", seed=seed,
                    amp=pt["amp"], period=64, flip_at=S // 2, per_row_phase=False)


def _rows(w, n, rng):
    total = w.batch * w.heads_q * w.seqlen_q
    rows = set(rng.choice(total, min(n, total), replace=False).tolist())
    for h in range(w.heads_q):
        rows.update({h * w.seqlen_q, h * w.seqlen_q + w.seqlen_q - 1})
    return np.array(sorted(rows), np.int64)


def _max_abs_scores(q, k, w, rows=None):
    """max |q.k| in binary64, over all rows or over the given flat row ids."""
    g = w.heads_q // w.heads_kv
    best = 0.0
    qf = q.astype(np.float64)
    kf = k.astype(np.float64)
    if rows is None:
        for h in range(w.heads_q):
            s = qf[0, :, h, :] @ kf[0, :, h // g, :].T
            if w.causal:
                s = np.where(np.tril(np.ones(s.shape, bool), w.seqlen_kv - w.seqlen_q), s, 0.0)
            best = max(best, float(np.max(np.abs(s))))
        return best
    h, i = np.divmod(rows, w.seqlen_q)
    for hh in np.unique(h):
        ii = i[h == hh]
        s = qf[0, ii, hh, :] @ kf[0, :, hh // g, :].T
        if w.causal:
            s = np.where(np.arange(w.seqlen_kv)[None, :] <= (ii + w.seqlen_kv - w.seqlen_q)[:, None],
                         s, 0.0)
        best = max(best, float(np.max(np.abs(s))))
    return best


def refine_rate(q, k, w, rows):
    """Replay of PASA's per-block shift rule on the given flat row ids, in
    binary64: per key block, mu = mean and m = max of the row's visible scaled
    scores c*s (c = scale * log2 e); off = mu on the row's first visible block,
    else max(mu, R); the block refines when fp16(m - off) exceeds THETA (or
    overflows), and then off = m; R <- max(R, off + fp16(m - off)).  Returns
    the refined fraction of (row, block) steps with a visible key."""
    c = w.scale / math.log(2.0)
    g = w.heads_q // w.heads_kv
    bc = block_keys(w.head_dim)
    h, i = np.divmod(rows, w.seqlen_q)
    n_ref = n_tot = 0
    for hh in np.unique(h):
        ii = i[h == hh]
        s = c * (q[0, ii, hh, :].astype(np.float64) @ k[0, :, hh // g, :].astype(np.float64).T)
        lim = (ii + w.seqlen_kv - w.seqlen_q + 1) if w.causal else np.full(len(ii), w.seqlen_kv)
        R = np.full(len(ii), -np.inf)
        for b0 in range(0, w.seqlen_kv, bc):
            blk = s[:, b0:b0 + bc]
            vis = np.arange(b0, b0 + blk.shape[1])[None, :] < lim[:, None]
            cnt = vis.sum(axis=1)
            act = cnt > 0
            mu = np.where(vis, blk, 0.0).sum(axis=1) / np.maximum(cnt, 1)
            m = np.where(vis, blk, -np.inf).max(axis=1)
            off = np.where(np.isinf(R), mu, np.maximum(mu, R))
            with np.errstate(over="ignore", invalid="ignore"):
                mb = (m - off).astype(np.float16).astype(np.float64)
            ref = act & ~(mb <= THETA)
            off = np.where(ref, m, off)
            mb = np.where(ref, 0.0, mb)
            R = np.where(act, np.maximum(R, off + mb), R)
            n_ref += int(ref.sum())
            n_tot += int(act.sum())
    return n_ref / max(n_tot, 1)


def replay(pt, seed=0, n_rows=256):
    """The grid point's columns that need no GPU."""
    w = workload(pt, seed)
    q, k, _ = W.generate(w)
    rng = np.random.default_rng(seed + 17)
    rows = _rows(w, n_rows, rng)
    all_rows = w.seqlen_q * w.seqlen_kv * w.heads_q <= (1 << 24)
    mx = _max_abs_scores(q, k, w, None if all_rows else rows)
    return dict(pt, heads=w.heads_q, max_abs_s=mx, s_rows="all" if all_rows else "sampled",
                naive_overflow=bool(mx >= FP16_INF_EDGE),
                max_abs_cs=mx * w.scale / math.log(2.0),
                refine_rate=refine_rate(q, k, w, rows))


def measure(pasa, pt, seed=0, n_rows=256):
    """Run one grid point through the three kernels and the oracle."""
    import torch
    w = workload(pt, seed)
    q, k, v = W.generate(w)
    rng = np.random.default_rng(seed + 17)
    rows = _rows(w, n_rows, rng)
    all_rows = w.seqlen_q * w.seqlen_kv * w.heads_q <= (1 << 24)
    mx = _max_abs_scores(q, k, w, None if all_rows else rows)
    ro, _ = attn_fp64(q, k, v, w.scale, w.causal, rows=rows)
    tq, tk, tv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    h, i = np.divmod(rows, w.seqlen_q)
    vf = v.astype(np.float64)
    floor = 0.25 * float(np.sqrt(np.mean(vf * vf) * vf.shape[-1]))
    res = dict(pt, heads=w.heads_q, max_abs_s=mx, s_rows="all" if all_rows else "sampled",
               naive_overflow=bool(mx >= FP16_INF_EDGE),
               max_abs_cs=mx * w.scale / math.log(2.0),
               refine_rate=refine_rate(q, k, w, rows))
    for name, fn in (("naive", pasa.naive_attn_fwd), ("strict", pasa.attn_fwd_strict),
                     ("pasa", pasa.attn_fwd)):
        o, _ = fn(tq, tk, tv, causal=w.causal, scale=w.scale)
        torch.cuda.synchronize()
        o = o.cpu().numpy()
        bad = nonfinite(o)
        sel = o[0, i, h].astype(np.float64)
        res[f"{name}_nonfinite"] = int(bad)
        fin = bool(np.all(np.isfinite(sel)))
        res[f"{name}_rel_rmse"] = rel_rmse(sel, ro) if fin else float("nan")
        res[f"{name}_head_max"] = (max(grouped_rel_rmse(sel, ro, h).values()) if fin
                                   else float("nan"))
        res[f"{name}_row_max"] = (float(row_rel_err(sel, ro, floor).max()) if fin
                                  else float("nan"))
    return res


def onsets(results):
    """Smallest bias (amplitude; |cos| of the phase offset) at which the naive
    kernel produced inf/NaN, per (kind, seq, D), beside the smallest one
    predicted from the scores."""
    out = {}
    for r in results:
        key = (r["kind"], r["seq"], r["D"])
        x = (r.get("bias") if r["kind"] == "bias"
             else abs(math.cos(r["offset"])) if r["kind"] == "phase" else r.get("amp"))
        o = out.setdefault(key, {"observed": None, "predicted": None})
        if r["naive_nonfinite"] and (o["observed"] is None or x < o["observed"]):
            o["observed"] = x
        if r["naive_overflow"] and (o["predicted"] is None or x < o["predicted"]):
            o["predicted"] = x
    return out


def main():
    ap = argparse.ArgumentParser(description="designed-random sweep of the forward kernels")
    ap.add_argument("--full", action="store_true", help="the long grid (sequences to 65504)")
    ap.add_argument("--replay-only", action="store_true",
                    help="only the columns that need no GPU (scores, predicted overflow, refine rate)")
    ap.add_argument("--part", default="0/1", metavar="K/N",
                    help="run only grid points with index = K mod N (to split a long grid)")
    args = ap.parse_args()
    k_part, n_part = (int(x) for x in args.part.split("/"))
    if args.replay_only:
        for n, pt in enumerate(points(args.full)):
            if n % n_part == k_part:
                print(json.dumps(replay(pt, seed=100 + n)), flush=True)
        return
    import precision_flashattention_numerics_amd as pasa
    results = []
    for n, pt in enumerate(points(args.full)):
        if n % n_part != k_part:
            continue
        r = measure(pasa, pt, seed=100 + n)
        results.append(r)
        print(json.dumps(r), flush=True)
    for (kind, seq, D), o in sorted(onsets(results).items()):
        print(json.dumps({"onset": kind, "seq": seq, "D": D, **o}), flush=True)


if __name__ == "__main__":
    main()
