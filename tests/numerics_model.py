"""A CPU model of the PASA kernels' per-block fp16 arithmetic, for studying
what each step of the method contributes.  Test infrastructure: it is neither
the oracle (that is plain binary64 attention, oracle/) nor a fallback (nothing
outside tests/ imports it).

"Online Pseudo-average Shifting Attention (PASA) ...", Abstract: each key
block's scores are shifted by a pseudo-average so that the half-precision
tile stays in range; softmax statistics and exponentials are half precision;
a global recovering step restores the normalisation.  The model replays the
kernels' reading of those steps (the rules in csrc/pasa_tile.hpp) with numpy's
IEEE fp16 and fp32 types, one row block at a time, and offers variants that
differ in one step:

  fused         the kernels' rule: off = c*mu (first visible block) or
                max(c*mu, R); m_b = fp16(c*max S - off), refine to the row
                maximum when m_b > 4; R' = max(R, off + m_b); s = fp16(R' - off);
                X = fp16(fp32(c*S - (off + s))) straight from the fp32 score
  fused_no_mu   the same with the pseudo-average replaced by the running
                maximum: off = R, and on a row's first block the row maximum
  two_round     the shifted fp16 tile T = fp16(c*S - off) formed first, its
                fp16 maximum, then X = fp16(T - s) (two roundings; mu decides
                where T is centred)
  two_round_no_mu   two_round with off = R (first block: row maximum)
  mu_only       the tile centred at the pseudo-average alone, off = c*mu on
                every block (no running maximum in the shift, no refine)
  no_refine     the kernels' rule without the refine step
  kshift        the shift applied to the keys before the product, as on
                hardware whose matrix unit emits fp16 scores: K' = fp16(K -
                kbar_b) with kbar_b the block's mean key, S' = Q K'^T (fp32),
                then the fused rule on S'; the removed q.kbar_b is restored in
                R (global recovering)

Scores are formed in binary64 from the fp16 inputs and rounded to fp32 (the
matrix cores accumulate fp16 products exactly enough for this purpose);
exponentials are evaluated in binary64 and rounded to fp16 (the hardware's
v_exp_f16 is within about one fp16 ulp of that).
"""
import math

import numpy as np

THETA = 4.0
F16 = np.float16
F32 = np.float32

VARIANTS = ("fused", "fused_no_mu", "two_round", "two_round_no_mu", "mu_only", "no_refine",
            "kshift")


def _h(x):
    return np.asarray(x, np.float64).astype(F16)


def _comp_add(hi, lo, alpha, r):
    """(hi, lo) <- alpha*(hi, lo) + r as a two-sum in fp16."""
    a = (alpha * hi).astype(F16)
    b = (alpha * lo).astype(F16)
    s = (a + r).astype(F16)
    bb = (s - a).astype(F16)
    err = ((a - (s - bb).astype(F16)).astype(F16) + (r - bb).astype(F16)).astype(F16)
    return s, (b + err).astype(F16)


def _tree_sum(P):
    """fp16 pairwise sum over the last axis (a power of two or padded with 0)."""
    x = P.astype(F16)
    n = x.shape[-1]
    m = 1 << (n - 1).bit_length()
    if m != n:
        x = np.concatenate([x, np.zeros(x.shape[:-1] + (m - n,), F16)], axis=-1)
    while x.shape[-1] > 1:
        x = (x[..., 0::2] + x[..., 1::2]).astype(F16)
    return x[..., 0]


def emulate_rows(q_rows, k, v, scale, limits, block, variant="fused"):
    """Attention of n query rows against one key/value head.

    q_rows [n, D], k/v [Skv, D] (fp16 values), limits [n]: row i sees keys
    [0, limits[i]).  Returns (o [n, D] float64, lse [n] float64)."""
    if variant not in VARIANTS:
        raise ValueError(variant)
    qd = np.asarray(q_rows, np.float64)
    kd = np.asarray(k, np.float64)
    vf = np.asarray(v, F16).astype(F32)
    n, D = qd.shape
    Skv = kd.shape[0]
    c = scale / math.log(2.0)
    lim = np.asarray(limits, np.int64)
    R = np.full(n, -np.inf)
    hi = np.zeros(n, F16)
    lo = np.zeros(n, F16)
    lc = np.zeros(n, F32)
    acc = np.zeros((n, D), F32)
    no_mu = variant.endswith("no_mu")
    two = variant.startswith("two_round")
    for b0 in range(0, Skv, block):
        kb = kd[b0:b0 + block]
        nb = kb.shape[0]
        vis = (np.arange(b0, b0 + nb)[None, :] < lim[:, None])
        cnt = vis.sum(axis=1)
        act = cnt > 0
        if not act.any():
            continue
        if variant == "kshift":
            kbar = kb.mean(axis=0)
            kp = _h(kb - kbar).astype(np.float64)
            S = (qd @ kp.T).astype(F32).astype(np.float64)
            base = c * (qd @ kbar)                     # restored in R
        else:
            S = (qd @ kb.T).astype(F32).astype(np.float64)
            base = np.zeros(n)
        Sv = np.where(vis, S, 0.0)
        mu = (Sv.astype(F32).sum(axis=1, dtype=F32)).astype(np.float64) / np.maximum(cnt, 1)
        m32 = np.where(vis, S, -np.inf).max(axis=1)
        Rl = R - base                                   # running max in this block's frame
        first = np.isinf(Rl)
        cmu = (c * mu).astype(F32)
        if no_mu:
            off = np.where(first, (c * m32).astype(F32), Rl)
        elif variant == "mu_only":
            off = cmu
        else:
            off = np.where(first, cmu, np.maximum(cmu, Rl))
        off = np.asarray(off, np.float64)
        with np.errstate(over="ignore", invalid="ignore"):
            if two:
                T = _h(c * S - off[:, None])
                T = np.where(vis, T.astype(np.float64), -np.inf)
                mb = T.max(axis=1)
            else:
                mb = _h(c * m32 - off).astype(np.float64)
            ref = act & ~(mb <= THETA)
            if variant in ("mu_only", "no_refine"):
                ref = np.zeros_like(ref)
            off = np.where(ref, np.asarray((c * m32).astype(F32), np.float64), off)
            if two:
                T = np.where(ref[:, None], _h(c * S - off[:, None]).astype(np.float64), T)
                T = np.where(vis, T, -np.inf)
                mb = np.where(ref, T.max(axis=1), mb)
            else:
                mb = np.where(ref, _h(c * m32 - off).astype(np.float64), mb)
        top = (off + mb).astype(F32).astype(np.float64)
        Rn = np.where(act, np.maximum(Rl, top), Rl)
        s = np.where(act, _h(Rn - off).astype(np.float64), 0.0)
        with np.errstate(over="ignore", invalid="ignore"):
            if two:
                X = _h(T - s[:, None])
            else:
                # fp32 fused multiply-add, then the round-to-nearest-even convert
                z = (off + s).astype(F32).astype(np.float64)
                X = _h((c * S - z[:, None]).astype(F32))
        X = np.where(vis, X.astype(np.float64), -np.inf)
        P = _h(np.exp2(X))
        r = _tree_sum(P)
        d = np.where(act, _h(Rl - Rn).astype(np.float64), 0.0)
        d = np.where(np.isinf(Rl), -np.inf, d)           # first block: nothing to rescale
        alpha = _h(np.exp2(d))
        alpha = np.where(act, alpha, F16(1))
        hi, lo = _comp_add(hi, lo, alpha, r)
        lc = (lc * alpha.astype(F32)).astype(F32)
        acc = acc * alpha.astype(F32)[:, None] + (P.astype(F32) @ vf[b0:b0 + nb]).astype(F32)
        R = np.where(act, Rn + base, R)
    L = (lc + hi.astype(F32) + lo.astype(F32)).astype(np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(L[:, None] > 0, acc.astype(np.float64) / L[:, None], 0.0)
        lse = np.where(L > 0, (R + np.log2(np.maximum(L, 1e-300))) * math.log(2.0), -np.inf)
    return _h(o).astype(np.float64), lse


def emulate(q, k, v, scale, causal, rows, block, variant="fused"):
    """emulate_rows over flat row ids (b*Hq + h)*Sq + i of BSHD tensors.
    Returns (o [len(rows), D], lse [len(rows)])."""
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    rows = np.asarray(rows, np.int64)
    o = np.zeros((rows.size, D))
    lse = np.zeros(rows.size)
    b, rem = np.divmod(rows, Hq * Sq)
    h, i = np.divmod(rem, Sq)
    for bb in np.unique(b):
        for hq in np.unique(h[b == bb]):
            sel = np.nonzero((b == bb) & (h == hq))[0]
            ii = i[sel]
            lim = (np.minimum(ii + Skv - Sq + 1, Skv).clip(0) if causal
                   else np.full(ii.size, Skv))
            oo, ll = emulate_rows(q[bb, ii, hq], k[bb, :, hq // g], v[bb, :, hq // g], scale, lim,
                                  block, variant)
            o[sel], lse[sel] = oo, ll
    return o, lse
