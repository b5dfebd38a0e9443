"""Pins of the binary64 oracle against facts fixed outside the oracle itself.

Each test would fail under a plausible slip in the oracle: a dropped scale or
max subtraction, a wrong sign, a transposed operand, a wrong GQA head map, a
wrong causal alignment, or a mis-weighted combine.

Properties used (the PASA page, "Online Pseudo-average Shifting Attention (PASA)
for Robust Low-precision LLM Inference", Abstract, calls PASA mathematically
equivalent to attention; the "Block Sparse Flash Attention" topic page,
FoldAttention card, states that softmax is invariant to a common shift and that
normalised partials over disjoint key ranges compose):
  closed forms on hand cases; rows of P sum to one; a per-row constant on the
  scores changes nothing; Q = 0 averages the visible values; constant V is
  returned; a dominant key is selected; non-causal attention ignores key order;
  torch's own scaled_dot_product_attention in float64 agrees; a brute-force
  pure-Python evaluation agrees; split-then-combine equals the whole.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attn_fp64, combine_fp64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _eval(expr):
    return float(eval(expr, {"__builtins__": {}}, {"e": math.e, "ln": math.log}))


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------- closed forms
def test_hand_cases_closed_form():
    cases = json.load(open(os.path.join(GOLDEN, "hand_cases.json")))["cases"]
    assert len(cases) == 4
    for c in cases:
        q = np.array(c["q"], np.float64)[None, :, None, :]
        k = np.array(c["k"], np.float64)[None, :, None, :]
        v = np.array(c["v"], np.float64)[None, :, None, :]
        o, lse = attn_fp64(q, k, v, _eval(c["scale"]), causal=c["causal"])
        exp_o = np.array([[_eval(x) for x in row] for row in c["o"]])
        exp_l = np.array([_eval(x) for x in c["lse"]])
        np.testing.assert_allclose(o[0, :, 0, :], exp_o, rtol=0, atol=1e-15, err_msg=c["name"])
        np.testing.assert_allclose(lse[0, 0, :], exp_l, rtol=0, atol=1e-15, err_msg=c["name"])


def test_fp16_threshold_fixture():
    g = json.load(open(os.path.join(GOLDEN, "fp16_overflow.json")))
    assert g["fp16_max"] == float(np.finfo(np.float16).max)


# ---------------------------------------------------------------- brute force
def _brute(q, k, v, scale, causal):
    """Pure-Python loops straight from the definition (tiny inputs only)."""
    B, Sq, Hq, D = q.shape
    _, Skv, Hkv, _ = k.shape
    g = Hq // Hkv
    o = np.zeros(q.shape)
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            for i in range(Sq):
                vis = [j for j in range(Skv) if (not causal) or j <= i + Skv - Sq]
                if not vis:
                    lse[b, h, i] = -math.inf
                    continue
                s = [scale * sum(q[b, i, h, d] * k[b, j, kh, d] for d in range(D)) for j in vis]
                tot = sum(math.exp(x) for x in s)
                lse[b, h, i] = math.log(tot)
                for d in range(D):
                    o[b, i, h, d] = sum(math.exp(x) * v[b, j, kh, d] for x, j in zip(s, vis)) / tot
    return o, lse


@pytest.mark.parametrize("shape", [(1, 3, 5, 2, 1, 3, True), (2, 4, 4, 4, 2, 2, False),
                                   (1, 6, 3, 3, 3, 2, True), (1, 2, 7, 6, 2, 4, True)])
def test_brute_force_small(shape):
    B, Sq, Skv, Hq, Hkv, D, causal = shape
    rng = np.random.default_rng(11)
    q = _rand((B, Sq, Hq, D), rng)
    k = _rand((B, Skv, Hkv, D), rng)
    v = _rand((B, Skv, Hkv, D), rng)
    o, lse = attn_fp64(q, k, v, 0.7, causal=causal)
    ob, lb = _brute(q, k, v, 0.7, causal)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- invariants
def test_rows_sum_to_one():
    # With V = identity (Skv == D) each output row is the probability row itself.
    rng = np.random.default_rng(1)
    S, D = 16, 16
    q = _rand((1, S, 2, D), rng, 3.0)
    k = _rand((1, S, 1, D), rng, 3.0)
    v = np.eye(S)[None, :, None, :]
    for causal in (False, True):
        o, _ = attn_fp64(q, k, v, 0.5, causal=causal)
        assert np.all(o >= 0)
        np.testing.assert_allclose(o.sum(-1), 1.0, rtol=0, atol=1e-14)
        if causal:  # nothing above the diagonal
            for i in range(S):
                assert np.all(o[0, i, :, i + 1:] == 0.0)


@pytest.mark.parametrize("c", [1e3, -1e3, 1e5, -1e5])
def test_per_row_shift_invariance(c):
    rng = np.random.default_rng(2)
    q = _rand((2, 33, 4, 8), rng)
    k = _rand((2, 40, 2, 8), rng)
    v = _rand((2, 40, 2, 8), rng)
    o0, l0 = attn_fp64(q, k, v, 0.4, causal=True)
    off = c * (1.0 + rng.random((2, 4, 33)))     # a different constant per row
    o1, l1 = attn_fp64(q, k, v, 0.4, causal=True, offset=off)
    np.testing.assert_allclose(o1, o0, rtol=1e-9, atol=1e-10)
    fin = np.isfinite(l0)
    np.testing.assert_allclose(l1[fin] - off[fin], l0[fin], rtol=0, atol=1e-9 * abs(c))


def test_key_bias_shift_invariance():
    # k_j -> k_j + b for every key j adds scale*q_i.b to every score of row i:
    # a per-row constant, so O is unchanged while lse moves by exactly that.
    rng = np.random.default_rng(3)
    q = _rand((1, 20, 2, 16), rng) + 30.0
    k = _rand((1, 24, 1, 16), rng) + 30.0
    v = _rand((1, 24, 1, 16), rng)
    b = rng.uniform(-30, 30, 16)
    o0, l0 = attn_fp64(q, k, v, 0.25)
    o1, l1 = attn_fp64(q, k + b, v, 0.25)
    np.testing.assert_allclose(o1, o0, rtol=1e-10, atol=1e-11)
    shift = 0.25 * np.einsum("bshd,d->bhs", q, b)
    np.testing.assert_allclose(l1 - l0, shift, rtol=1e-11, atol=1e-9)


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(4)
    Sq, Skv = 9, 12
    q = np.zeros((1, Sq, 3, 4))
    k = _rand((1, Skv, 1, 4), rng)
    v = _rand((1, Skv, 1, 4), rng)
    o, lse = attn_fp64(q, k, v, 1.0)
    np.testing.assert_allclose(o[0], np.broadcast_to(v[0, :, 0].mean(0), (Sq, 3, 4)), atol=1e-15)
    np.testing.assert_allclose(lse, math.log(Skv), atol=1e-15)
    o, lse = attn_fp64(q, k, v, 1.0, causal=True)
    for i in range(Sq):
        n = i + Skv - Sq + 1
        np.testing.assert_allclose(o[0, i, 1], v[0, :n, 0].mean(0), atol=1e-15)
        assert abs(lse[0, 1, i] - math.log(n)) < 1e-15


def test_constant_values_returned():
    rng = np.random.default_rng(5)
    q = _rand((1, 10, 2, 8), rng, 4.0)
    k = _rand((1, 10, 2, 8), rng, 4.0)
    v = np.broadcast_to(np.arange(8.0) - 3.5, (1, 10, 2, 8)).copy()
    o, _ = attn_fp64(q, k, v, 1.0, causal=True)
    np.testing.assert_allclose(o, np.broadcast_to(v[:, :, :1, :], o.shape), rtol=0, atol=1e-13)


def test_dominant_key_is_selected():
    rng = np.random.default_rng(6)
    D = 8
    k = _rand((1, 6, 1, D), rng)
    v = _rand((1, 6, 1, D), rng)
    q = 200.0 * k[:, 3:4, :, :]          # q.k_3 exceeds every other score by > 50
    s = (q[0, 0, 0] @ k[0, :, 0].T)
    assert np.sort(s)[-1] - np.sort(s)[-2] > 50
    o, lse = attn_fp64(q, k, v, 1.0)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 3, 0], rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 0] - s[3]) < 1e-9


def test_noncausal_key_permutation_invariance():
    rng = np.random.default_rng(7)
    q = _rand((2, 7, 2, 8), rng)
    k = _rand((2, 11, 2, 8), rng)
    v = _rand((2, 11, 2, 8), rng)
    perm = rng.permutation(11)
    o0, l0 = attn_fp64(q, k, v, 0.3)
    o1, l1 = attn_fp64(q, k[:, perm], v[:, perm], 0.3)
    np.testing.assert_allclose(o1, o0, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l0, rtol=1e-14, atol=1e-14)


def test_gqa_head_map():
    # query head h reads key/value head h // (Hq/Hkv): compare against running
    # every query head with an explicitly repeated key/value head.
    rng = np.random.default_rng(8)
    Hq, Hkv = 6, 2
    q = _rand((1, 5, Hq, 4), rng)
    k = _rand((1, 9, Hkv, 4), rng)
    v = _rand((1, 9, Hkv, 4), rng)
    o, lse = attn_fp64(q, k, v, 0.5, causal=True)
    for h in range(Hq):
        kh = h // (Hq // Hkv)
        oh, lh = attn_fp64(q[:, :, h:h + 1], k[:, :, kh:kh + 1], v[:, :, kh:kh + 1], 0.5, causal=True)
        np.testing.assert_array_equal(o[:, :, h:h + 1], oh)
        np.testing.assert_array_equal(lse[:, h:h + 1], lh)


def test_empty_rows_when_more_queries_than_keys():
    rng = np.random.default_rng(9)
    q = _rand((1, 6, 1, 4), rng)
    k = _rand((1, 4, 1, 4), rng)
    v = _rand((1, 4, 1, 4), rng)
    o, lse = attn_fp64(q, k, v, 1.0, causal=True)
    assert np.all(o[0, :2] == 0.0) and np.all(np.isneginf(lse[0, 0, :2]))
    assert np.all(np.isfinite(lse[0, 0, 2:]))
    o2, _ = attn_fp64(q[:, 2:], k, v, 1.0, causal=True)  # row 2 sees key 0 only, ...
    np.testing.assert_allclose(o[0, 2, 0], v[0, 0, 0], atol=1e-15)


def test_row_sampling_matches_full():
    rng = np.random.default_rng(10)
    q = _rand((2, 13, 4, 8), rng)
    k = _rand((2, 17, 2, 8), rng)
    v = _rand((2, 17, 2, 8), rng)
    o, lse = attn_fp64(q, k, v, 0.35, causal=True)
    rows = rng.choice(2 * 4 * 13, 20, replace=False)
    os_, ls = attn_fp64(q, k, v, 0.35, causal=True, rows=rows)
    b, rem = np.divmod(rows, 4 * 13)
    h, i = np.divmod(rem, 13)
    np.testing.assert_array_equal(os_, o[b, i, h])
    np.testing.assert_array_equal(ls, lse[b, h, i])


# ---------------------------------------------------------------- library
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("Sq,Skv,Hq,Hkv,D,causal", [
    (64, 64, 4, 4, 16, False), (128, 128, 6, 2, 32, True),
    (100, 300, 2, 1, 64, True), (257, 257, 3, 3, 8, False), (1, 512, 7, 1, 64, False)])
def test_against_torch_sdpa_float64(Sq, Skv, Hq, Hkv, D, causal):
    rng = np.random.default_rng(Sq * 7 + Skv)
    q = _rand((2, Sq, Hq, D), rng, 2.0)
    k = _rand((2, Skv, Hkv, D), rng, 2.0)
    v = _rand((2, Skv, Hkv, D), rng)
    scale = 1.0 / math.sqrt(D)
    o, lse = attn_fp64(q, k, v, scale, causal=causal)
    g = Hq // Hkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    mask = None
    if causal:  # bottom-right aligned: key j visible to query i iff j <= i + Skv - Sq
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Skv)[None, :]
        mask = j <= i + (Skv - Sq)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-12)
    s = torch.einsum("bhid,bhjd->bhij", tq, tk) * scale
    if mask is not None:
        s = s.masked_fill(~mask, -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=1e-13, atol=1e-12)


# ---------------------------------------------------------------- combine
@pytest.mark.parametrize("n", [1, 2, 5, 8])
def test_split_combine_identity(n):
    rng = np.random.default_rng(12 + n)
    B, Skv, Hq, Hkv, D = 3, 61, 6, 2, 16
    q = _rand((B, 1, Hq, D), rng, 3.0) + 2.0
    k = _rand((B, Skv, Hkv, D), rng, 3.0) + 2.0
    v = _rand((B, Skv, Hkv, D), rng)
    o, lse = attn_fp64(q, k, v, 0.25)
    bounds = np.linspace(0, Skv, n + 1).astype(int)
    parts_o = np.zeros((B * Hq, n, D))
    parts_l = np.zeros((B * Hq, n))
    for s in range(n):
        a, e = bounds[s], bounds[s + 1]
        os_, ls = attn_fp64(q, k[:, a:e], v[:, a:e], 0.25)
        parts_o[:, s] = os_[:, 0].reshape(B * Hq, D)
        parts_l[:, s] = ls[:, :, 0].reshape(B * Hq)
    oc, lc = combine_fp64(parts_o, parts_l)
    np.testing.assert_allclose(oc, o[:, 0].reshape(B * Hq, D), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lc, lse[:, :, 0].reshape(B * Hq), rtol=1e-14, atol=1e-12)


def test_combine_empty_partials():
    op = np.ones((2, 3, 4))
    lp = np.array([[-np.inf, 0.5, -np.inf], [-np.inf, -np.inf, -np.inf]])
    o, l = combine_fp64(op, lp)
    np.testing.assert_allclose(o[0], 1.0)
    assert l[0] == 0.5
    assert np.all(o[1] == 0) and np.isneginf(l[1])
