"""GPU parity: the HIP path against the binary64 oracle on identical seeded
fp16 inputs.  The bar is relative RMSE of O <= 2e-3 over the output and over
every (batch, head), the worst row within 1e-2 (tests/gpu_common.py explains
the row measure), no inf/NaN; lse within 1e-2 absolute (or 1e-6 relative above
1e4).  The naive fp16 kernel's overflow on the large-bias and resonance inputs
is recorded alongside."""
import numpy as np
import pytest

import workloads as W
from oracle import attn_fp64, combine_fp64
from tests.gpu_common import (REL_RMSE_MAX, check_o, gather_rows, head_rows, lse_error, lse_ok,
                              nonfinite, rel_rmse, row_heads, sample_rows, say, to_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pasa():
    import precision_flashattention_numerics_amd as p
    return p


def run_fwd(pasa, w, naive=False, strict=False):
    import torch
    q, k, v = W.generate(w)
    tq, tk, tv = to_gpu(q, k, v)
    fn = pasa.naive_attn_fwd if naive else pasa.attn_fwd_strict if strict else pasa.attn_fwd
    o, lse = fn(tq, tk, tv, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return (q, k, v), o.cpu().numpy(), lse.cpu().numpy()


SMALL = [(B, Sq, Skv, Hq, Hkv, D, causal)
         for (B, Sq, Skv) in [(1, 1, 1), (1, 63, 63), (2, 64, 64), (1, 65, 65), (1, 127, 300),
                              (1, 300, 127), (1, 300, 300), (2, 129, 1000)]
         for (Hq, Hkv) in [(1, 1), (7, 1)]
         for D in (64, 128)
         for causal in (False, True)]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes_vs_oracle(pasa, shape):
    B, Sq, Skv, Hq, Hkv, D, causal = shape
    w = W.custom(B, Sq, Skv, Hq, Hkv, D, causal, kind="bias", seed=sum(shape), bias=3.0)
    say("case", shape)
    (q, k, v), o, lse = run_fwd(pasa, w)
    ro, rl = attn_fp64(q, k, v, w.scale, causal)
    # rows with no visible key (causal, Sq > Skv) are exactly zero
    empty = np.isneginf(rl)
    if empty.any():
        b, h, i = np.nonzero(empty)
        assert np.all(o[b, i, h] == 0)
    check_o(o, ro, v, label=str(shape))
    assert lse_ok(lse, rl)


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_config_full_vs_oracle(pasa, name):
    w = W.CONFIGS[name]
    say("config", name)
    (q, k, v), o, lse = run_fwd(pasa, w)
    ro, rl = attn_fp64(q, k, v, w.scale, w.causal)
    assert nonfinite(lse) == 0
    check_o(o, ro, v, label=name)
    say(name, "lse_err", lse_error(lse, rl)[:2])
    assert lse_ok(lse, rl)


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_strict_config_full_vs_oracle(pasa, name):
    """fp16 running maximum and offset as well: same bar (every config keeps
    |c * score| well below 3.2e4)."""
    w = W.CONFIGS[name]
    say("strict config", name)
    (q, k, v), o, lse = run_fwd(pasa, w, strict=True)
    ro, rl = attn_fp64(q, k, v, w.scale, w.causal)
    assert nonfinite(lse) == 0
    check_o(o, ro, v, label="strict " + name)
    say(name, "strict lse_err", lse_error(lse, rl)[:2])
    assert lse_ok(lse, rl)


@pytest.mark.parametrize("shape", [s for s in SMALL if s[0] * s[1] * s[3] <= 600 and s[2] >= 64],
                         ids=lambda s: "x".join(map(str, s)))
def test_strict_small_shapes_vs_oracle(pasa, shape):
    B, Sq, Skv, Hq, Hkv, D, causal = shape
    w = W.custom(B, Sq, Skv, Hq, Hkv, D, causal, kind="bias", seed=sum(shape) + 7, bias=10.0)
    say("strict case", shape)
    (q, k, v), o, lse = run_fwd(pasa, w, strict=True)
    ro, rl = attn_fp64(q, k, v, w.scale, causal)
    check_o(o, ro, v, label="strict " + str(shape))
    assert lse_ok(lse, rl)


@pytest.mark.parametrize("Sq,Skv", [(1024, 5120), (640, 8192), (1, 3000)])
def test_chunked_prefill_against_cache_vs_oracle(pasa, Sq, Skv):
    """A chunk of new queries against a cache that already holds earlier keys:
    bottom-right causal alignment (query i sees keys j <= i + Skv - Sq)."""
    w = W.custom(1, Sq, Skv, 28, 4, 128, True, kind="bias", seed=Sq + Skv, bias=30.0)
    say("chunked prefill", Sq, Skv)
    (q, k, v), o, lse = run_fwd(pasa, w)
    rows = sample_rows(w, 400, np.random.default_rng(Sq))
    ro, rl = attn_fp64(q, k, v, w.scale, True, rows=rows)
    go, gl = gather_rows(o, lse, w, rows)
    assert nonfinite(o) == 0
    check_o(go, ro, v, heads=row_heads(w, rows), label=f"chunked {Sq}x{Skv}")
    assert lse_ok(gl, rl)


@pytest.fixture(scope="module")
def c4_run(pasa):
    """The long-context workload through PASA and the naive kernel, once."""
    import torch
    w = W.CONFIGS["c4"]
    say("config c4: generating inputs")
    q, k, v = W.generate(w)
    tq, tk, tv = to_gpu(q, k, v)
    o, lse = pasa.attn_fwd(tq, tk, tv, causal=True, scale=w.scale)
    on, _ = pasa.naive_attn_fwd(tq, tk, tv, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    res = dict(w=w, q=q, k=k, v=v, o=o.cpu().numpy(), lse=lse.cpu().numpy(), naive=on.cpu().numpy())
    del tq, tk, tv, o, lse, on
    torch.cuda.empty_cache()
    return res


def c4_extreme_heads(w, n=4):
    """Query heads with the largest amplitude product a_q*a_k and the largest
    bias product b_q*b_k (n of each): the heads most exposed to the overflow
    mechanisms the PASA page names."""
    aq, bq, ak, bk = W.head_params(w)
    kv = np.arange(w.heads_q) // w.group
    amp, bias = aq * ak[kv], bq * bk[kv]
    return sorted(set(np.argsort(-amp)[:n].tolist()) | set(np.argsort(-bias)[:n].tolist()))


def test_c4_extreme_heads_and_one_percent_vs_oracle(c4_run):
    """All rows of the most exposed heads, 1 % of the rows of every other head."""
    w, q, k, v, o, lse = (c4_run[x] for x in ("w", "q", "k", "v", "o", "lse"))
    assert nonfinite(o) == 0 and nonfinite(lse) == 0
    heads = c4_extreme_heads(w)
    say("c4 full heads", heads)
    rows = head_rows(w, set(heads), 0.01, np.random.default_rng(44))
    ro, rl = attn_fp64(q, k, v, w.scale, w.causal, rows=rows)
    go, gl = gather_rows(o, lse, w, rows)
    check_o(go, ro, v, heads=row_heads(w, rows), label="c4")
    full = np.isin(row_heads(w, rows), heads)
    for h in heads:
        sel = row_heads(w, rows) == h
        say("c4 head", h, "rel_rmse", rel_rmse(go[sel], ro[sel]))
    say("c4 rows compared", rows.size, "of which in full heads", int(full.sum()))
    assert lse_ok(gl, rl)


def c4_head_bounds(w, q, k):
    """Per query head: an upper bound on max |q.k| (Cauchy-Schwarz over the
    largest row norms) and a lower bound (the largest |q.k| over a sample of
    query rows against every key)."""
    kmax = [float(np.sqrt(np.sum(k[0, :, j].astype(np.float64) ** 2, axis=-1)).max())
            for j in range(w.heads_kv)]
    rng = np.random.default_rng(45)
    upper, lower = [], []
    for h in range(w.heads_q):
        kvh = h // w.group
        qmax = float(np.sqrt(np.sum(q[0, :, h].astype(np.float64) ** 2, axis=-1)).max())
        upper.append(qmax * kmax[kvh])
        ii = rng.choice(w.seqlen_q, 16, replace=False)
        s = q[0, ii, h].astype(np.float64) @ k[0, :, kvh].astype(np.float64).T
        s = np.where(np.arange(w.seqlen_kv)[None, :] <= ii[:, None], s, 0.0)
        lower.append(float(np.abs(s).max()))
    return np.array(upper), np.array(lower)


def test_c4_naive_overflows_on_the_exposed_heads(c4_run):
    """The naive fp16 kernel: heads with some unscaled |q.k| above the fp16
    range produce inf/NaN, heads whose every |q.k| provably stays below it do
    not, and the finite heads' error is reported."""
    w, q, k, v, on = (c4_run[x] for x in ("w", "q", "k", "v", "naive"))
    upper, lower = c4_head_bounds(w, q, k)
    bad = np.array([nonfinite(on[0, :, h]) for h in range(w.heads_q)])
    say("c4 naive non-finite per head", bad.tolist())
    say("c4 naive heads with inf/NaN", int(np.count_nonzero(bad)), "of", w.heads_q,
        "outputs", int(bad.sum()), "of", on.size)
    assert bad.sum() > 0
    for h in range(w.heads_q):
        if lower[h] > 66000.0:
            assert bad[h] > 0, (h, lower[h])
        if upper[h] < 65000.0:
            assert bad[h] == 0, (h, upper[h])
    fin = [h for h in range(w.heads_q) if bad[h] == 0]
    if fin:
        rng = np.random.default_rng(46)
        rows = np.concatenate([h * w.seqlen_q + np.sort(rng.choice(w.seqlen_q, 64, replace=False))
                               for h in fin])
        ro, _ = attn_fp64(q, k, v, w.scale, True, rows=rows)
        go = on[0, rows % w.seqlen_q, rows // w.seqlen_q]
        say("c4 naive rel_rmse on its finite heads (sampled rows)", rel_rmse(go, ro))


def test_stress_jump_above_fp16_range(pasa):
    # keys jump from bias 2 to bias 60 half way: unscaled scores ~2.3e5
    w = W.custom(1, 512, 512, 4, 1, 128, True, kind="jump", seed=77, jump_at=200)
    (q, k, v), o, lse = run_fwd(pasa, w)
    ro, rl = attn_fp64(q, k, v, w.scale, True)
    check_o(o, ro, v, label="jump")
    assert lse_ok(lse, rl)


def test_resonance_per_row_phase_stress(pasa):
    w = W.custom(1, 1024, 1024, 2, 2, 64, False, kind="resonance", seed=31, amp=48.0,
                 period=64, flip_at=512, per_row_phase=True)
    (q, k, v), o, lse = run_fwd(pasa, w)
    ro, rl = attn_fp64(q, k, v, w.scale, False)
    check_o(o, ro, v, label="per-row-phase resonance")


def test_deterministic(pasa):
    w = W.custom(1, 300, 300, 7, 1, 128, True, kind="bias", seed=5, bias=30.0)
    _, o1, l1 = run_fwd(pasa, w)
    _, o2, l2 = run_fwd(pasa, w)
    assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16))
    assert np.array_equal(l1, l2)


# ----------------------------------------------------------------- naive kernel
def test_naive_matches_oracle_without_overflow(pasa):
    w = W.CONFIGS["c1"]
    (q, k, v), o, lse = run_fwd(pasa, w, naive=True)
    ro, rl = attn_fp64(q, k, v, w.scale, w.causal)
    err = rel_rmse(o, ro)
    say("naive c1 rel_rmse", err)
    assert nonfinite(o) == 0
    assert err <= 5e-3   # unscaled fp16 scores lose ~4 bits more than PASA's tile


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_naive_overflows_where_pasa_does_not(pasa, name):
    w = W.CONFIGS[name]
    (_, _, _), o, _ = run_fwd(pasa, w, naive=True)
    bad = nonfinite(o)
    per_head = [nonfinite(o[:, :, h]) for h in range(w.heads_q)]
    say(name, "naive non-finite outputs:", bad, "of", o.size, "per head", per_head)
    # every head of these inputs has unscaled scores beyond the fp16 range
    assert all(x > 0 for x in per_head)


# ----------------------------------------------------------------- decode
def test_c5_decode_vs_oracle(pasa):
    import torch
    w = W.CONFIGS["c5"]
    say("config c5 decode")
    q, k, v = W.generate(w)
    tq, tk, tv = to_gpu(q, k, v)
    o, lse = pasa.attn_decode(tq, tk, tv, scale=w.scale)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    ro, rl = attn_fp64(q, k, v, w.scale, False)
    assert nonfinite(lse) == 0
    check_o(o, ro, v, label="c5 decode")
    assert lse_ok(lse, rl[:, :, 0])


@pytest.mark.parametrize("Skv,n,Hq,Hkv,D", [(1, 0, 4, 1, 128), (129, 3, 7, 7, 64),
                                            (1000, 0, 28, 4, 128), (5000, 7, 40, 1, 64),
                                            (8192, 1, 8, 8, 128), (300, 64, 14, 2, 128),
                                            (2000, 0, 16, 2, 64)])
def test_decode_shapes_vs_oracle(pasa, Skv, n, Hq, Hkv, D):
    import torch
    w = W.custom(3, 1, Skv, Hq, Hkv, D, False, kind="bias", seed=Skv + n, bias=30.0)
    q, k, v = W.generate(w)
    tq, tk, tv = to_gpu(q, k, v)
    o, lse = pasa.attn_decode(tq, tk, tv, num_splits=n, scale=w.scale)
    torch.cuda.synchronize()
    ro, rl = attn_fp64(q, k, v, w.scale, False)
    check_o(o.cpu().numpy(), ro, v, label=f"decode {(Skv, n, Hq, Hkv, D)}")
    assert lse_ok(lse.cpu().numpy(), rl[:, :, 0])


@pytest.mark.parametrize("B,Skv,Hq,Hkv,D,splits", [(64, 1500, 28, 4, 64, 6), (16, 700, 32, 32, 64, 3),
                                                    (8, 3000, 32, 8, 64, 12)])
def test_decode_default_splits_head_dim_64_vs_oracle(pasa, B, Skv, Hq, Hkv, D, splits):
    """The library's split count at head_dim 64 (six waves per CU from 256
    (sequence, kv head) units up, three below) against the oracle."""
    import torch
    assert pasa.decode_splits(B, Skv, Hq, Hq // Hkv, D) == splits
    w = W.custom(B, 1, Skv, Hq, Hkv, D, False, kind="bias", seed=B + Skv, bias=30.0)
    q, k, v = W.generate(w)
    tq, tk, tv = to_gpu(q, k, v)
    say("decode default splits", (B, Skv, Hq, Hkv, D, splits))
    o, lse = pasa.attn_decode(tq, tk, tv, scale=w.scale)
    torch.cuda.synchronize()
    ro, rl = attn_fp64(q, k, v, w.scale, False)
    check_o(o.cpu().numpy(), ro, v, label=f"decode default splits {(B, Skv, Hq, Hkv, D)}")
    assert lse_ok(lse.cpu().numpy(), rl[:, :, 0])


def test_decode_combine_entry_on_oracle_partials(pasa):
    """pasa_attn_decode_combine fed with oracle partials over disjoint key
    ranges must reproduce the unsplit oracle (up to fp32/fp16 rounding)."""
    import torch
    B, Skv, Hq, Hkv, D, n = 2, 700, 6, 2, 128, 5
    w = W.custom(B, 1, Skv, Hq, Hkv, D, False, kind="bias", seed=3, bias=30.0)
    q, k, v = W.generate(w)
    bounds = [0, 100, 101, 350, 700, 700]          # includes an empty range
    po = np.zeros((B, Hq, n, D))
    pl = np.zeros((B, Hq, n))
    for s in range(n):
        a, e = bounds[s], bounds[s + 1]
        if e == a:
            pl[:, :, s] = -np.inf
            continue
        os_, ls = attn_fp64(q, k[:, a:e], v[:, a:e], w.scale)
        po[:, :, s] = os_[:, 0]
        pl[:, :, s] = ls[:, :, 0]
    ro, rl = attn_fp64(q, k, v, w.scale)
    oc, lc = combine_fp64(po.reshape(B * Hq, n, D), pl.reshape(B * Hq, n))
    assert np.allclose(oc, ro[:, 0].reshape(B * Hq, D), atol=1e-12)
    tpo = torch.from_numpy(po.astype(np.float32)).cuda()
    tpl = torch.from_numpy(pl.astype(np.float32)).cuda()
    o, lse = pasa.attn_decode_combine(tpo, tpl)
    torch.cuda.synchronize()
    check_o(o.cpu().numpy(), ro, v, label="combine", rel_max=1e-3)
    assert lse_ok(lse.cpu().numpy(), rl[:, :, 0], abs_tol=1e-4)


# ----------------------------------------------------------------- ABI on GPU
def test_error_writes_nothing(pasa):
    import ctypes

    import torch
    lib = pasa.raw()
    q = torch.zeros((1, 8, 2, 96), dtype=torch.float16, device="cuda")
    o = torch.full_like(q, 7.0)
    rc = lib.pasa_attn_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), None, 1, 8, 8,
                           2, 1, 96, ctypes.c_float(0.1), 0, None)
    torch.cuda.synchronize()
    assert rc == -2
    assert bool((o == 7.0).all())


def test_binding_rejects_wrong_output_buffers(pasa):
    """The library writes through raw pointers, so the binding refuses output
    buffers of the wrong shape, dtype or device before anything is launched."""
    import torch
    q = torch.zeros((2, 1, 4, 64), dtype=torch.float16, device="cuda")
    k = torch.zeros((2, 64, 2, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        pasa.attn_decode(q, k, k, out=torch.empty((2, 1, 4, 32), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        pasa.attn_decode(q, k, k, lse=torch.empty((2, 3), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        pasa.attn_decode(q, k, k, out=torch.empty_like(q, dtype=torch.float32))
    with pytest.raises(ValueError):
        pasa.attn_decode(q, k, k, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    op = torch.zeros((2, 4, 3, 64), dtype=torch.float32, device="cuda")
    lp = torch.zeros((2, 4, 3), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        pasa.attn_decode_combine(op, lp, out=torch.empty((2, 4, 64), dtype=torch.float16, device="cuda"))
    qp = torch.zeros((1, 8, 2, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        pasa.attn_fwd(qp, qp, qp, out=torch.empty((1, 8, 2, 32), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        pasa.attn_fwd(qp, qp, qp, lse=torch.empty((1, 2, 7), dtype=torch.float32, device="cuda"))
    # the e4m3 entry point: wrong dtype, wrong shape, host tensor
    q8 = qp.to(torch.float8_e4m3fn)
    for bad in (torch.empty((1, 8, 2, 64), dtype=torch.float32, device="cuda"),
                torch.empty((1, 8, 2, 32), dtype=torch.float16, device="cuda"),
                torch.empty((1, 8, 2, 64), dtype=torch.float16)):
        with pytest.raises(ValueError):
            pasa.attn_fwd_fp8(q8, q8, qp, 1.0, 1.0, out=bad)
    for bad in (torch.empty((1, 2, 8), dtype=torch.float16, device="cuda"),
                torch.empty((1, 2, 9), dtype=torch.float32, device="cuda")):
        with pytest.raises(ValueError):
            pasa.attn_fwd_fp8(q8, q8, qp, 1.0, 1.0, lse=bad)
    torch.cuda.synchronize()


# ----------------------------------------------------------------- limits
@pytest.mark.parametrize("Skv,causal", [(65504, False), (65504, True), (131072, False),
                                         (131072 + 77, True)])
def test_long_kv_flat_rows(pasa, Skv, causal):
    """q = 0: every weight is 1, so the running sum counts the visible keys
    exactly and O is their values' mean.  65504 keys fill one fp16 sum to the
    fp16 maximum's worth; beyond that the sum spans several 32768-key segments
    carried in fp32."""
    import torch
    Sq, D = 5, 128
    w = W.custom(1, Sq, Skv, 2, 1, D, causal, kind="normal", seed=65504)
    q, k, v = W.generate(w)
    q[:] = 0
    tq, tk, tv = to_gpu(q, k, v)
    o, lse = pasa.attn_fwd(tq, tk, tv, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    ro, rl = attn_fp64(q, k, v, w.scale, causal)
    check_o(o.cpu().numpy(), ro, v, label=f"flat {Skv}")
    assert lse_ok(lse.cpu().numpy(), rl)


@pytest.mark.parametrize("Sq,Skv,D,causal", [(131072, 131072, 128, True),
                                             (2048, 131072 + 300, 64, False),
                                             (1000, 100000, 128, False),
                                             (70000, 70000, 64, True)])
def test_long_kv_vs_oracle(pasa, Sq, Skv, D, causal):
    """More keys than one fp16 running sum may hold (65504), biased inputs:
    sampled rows against the oracle, every head gated."""
    w = W.custom(1, Sq, Skv, 2, 1, D, causal, kind="bias", seed=Skv + D, bias=20.0)
    say("long kv", Sq, Skv, D, causal)
    (q, k, v), o, lse = run_fwd(pasa, w)
    assert nonfinite(o) == 0 and nonfinite(lse) == 0
    rng = np.random.default_rng(Skv)
    rows = sample_rows(w, 256, rng)
    # the last rows of a causal problem see the most keys
    rows = np.unique(np.concatenate([rows, [h * Sq + Sq - 1 - i for h in range(2) for i in range(8)]]))
    ro, rl = attn_fp64(q, k, v, w.scale, causal, rows=rows)
    go, gl = gather_rows(o, lse, w, rows)
    check_o(go, ro, v, heads=row_heads(w, rows), label=f"long kv {Sq}x{Skv} D{D}")
    assert lse_ok(gl, rl)


def test_decode_one_split_beyond_fp16_sum(pasa):
    """One decode split over 200000 keys (the fp16 sum is folded into fp32 every
    32768 keys) against the oracle, and against four splits."""
    import torch
    w = W.custom(2, 1, 200000, 8, 2, 128, False, kind="bias", seed=200, bias=20.0)
    q, k, v = W.generate(w)
    tq, tk, tv = to_gpu(q, k, v)
    o1, l1 = pasa.attn_decode(tq, tk, tv, num_splits=1, scale=w.scale)
    o4, l4 = pasa.attn_decode(tq, tk, tv, num_splits=4, scale=w.scale)
    torch.cuda.synchronize()
    ro, rl = attn_fp64(q, k, v, w.scale, False)
    check_o(o1.cpu().numpy(), ro, v, label="decode 1 split 200000 keys")
    check_o(o4.cpu().numpy(), ro, v, label="decode 4 splits 200000 keys")
    assert lse_ok(l1.cpu().numpy(), rl[:, :, 0])
    assert lse_ok(l4.cpu().numpy(), rl[:, :, 0])


def test_decode_deterministic_and_matches_prefill_shape(pasa):
    """The decode path twice gives identical bits; it agrees with the prefill
    kernel run on the same single-token queries."""
    import torch
    w = W.custom(4, 1, 3000, 14, 2, 128, False, kind="bias", seed=14, bias=30.0)
    q, k, v = W.generate(w)
    tq, tk, tv = to_gpu(q, k, v)
    o1, l1 = pasa.attn_decode(tq, tk, tv, num_splits=5, scale=w.scale)
    o2, l2 = pasa.attn_decode(tq, tk, tv, num_splits=5, scale=w.scale)
    op, lp = pasa.attn_fwd(tq, tk, tv, causal=False, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    a, b = o1.cpu().numpy(), op.cpu().numpy()
    assert rel_rmse(a, b) <= 2 * REL_RMSE_MAX
    assert np.max(np.abs(l1.cpu().numpy() - lp.cpu().numpy()[:, :, 0])) <= 1e-2


@pytest.mark.parametrize("D", [64, 128])
def test_noncausal_full_round_vs_oracle(pasa, D):
    """A non-causal problem of exactly one round of 256-row items on 256 CUs
    (64 heads x 1024 rows) keeps the 256-row kernel (the key split pays only for
    a partly idle last round); small non-causal problems take the key split."""
    w = W.custom(1, 1024, 1024, 64, 8, D, False, kind="bias", seed=75 + D, bias=25.0)
    say("case", w)
    (q, k, v), o, lse = run_fwd(pasa, w)
    rng = np.random.default_rng(76)
    rows = sample_rows(w, 3000, rng)
    ro, rl = attn_fp64(q, k, v, w.scale, False, rows=rows)
    go, gl = gather_rows(o, lse, w, rows)
    assert nonfinite(o) == 0
    check_o(go, ro, v, heads=row_heads(w, rows), label=f"one round D{D}")
    assert lse_ok(gl, rl)


@pytest.mark.parametrize("variant", ["pasa", "strict", "naive"])
def test_key_split_head_dim_128_vs_oracle(pasa, variant):
    """The key-split kernel at head_dim 128, whose matrix phase is laid out in
    slots by hand: a non-causal problem of few items (2 x 3 heads x 3 tiles of
    128 rows) takes it.  1000 keys are 16 blocks of 64, eight per half, the
    last one ragged (40 keys).  Checked against the oracle for each fp16
    variant of the per-block rule; the naive kernel gets N(0, 1) inputs, whose
    unscaled scores fp16 holds to a small fraction of a unit, and its own bar
    (with a bias its raw head_dim-128 scores reach the thousands, where an
    fp16 step is 1 or more)."""
    naive = variant == "naive"
    w = (W.custom(2, 300, 1000, 3, 1, 128, False, kind="normal", seed=91) if naive else
         W.custom(2, 300, 1000, 3, 1, 128, False, kind="bias", seed=91, bias=25.0))
    say("key split D128", variant, w)
    (q, k, v), o, lse = run_fwd(pasa, w, naive=naive, strict=variant == "strict")
    ro, rl = attn_fp64(q, k, v, w.scale, False)
    assert nonfinite(o) == 0
    if naive:
        assert rel_rmse(o, ro) <= 5e-3
    else:
        check_o(o, ro, v, label=f"key split D128 {variant}")
        assert lse_ok(lse, rl)


@pytest.mark.parametrize("heads", [7, 700], ids=["key_split", "full_rows"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Sq,Skv", [(300, 300), (300, 1000), (500, 260)])
def test_causal_item_shapes_vs_oracle(pasa, heads, D, Sq, Skv):
    """Causal prefill through both item shapes: few heads take the key split
    (two key halves merged in fp32), 700 heads exceed the split's item limit and
    keep 256-row items.  Ragged tiles, bottom-right alignment with Sq < Skv, and
    Sq > Skv, where the first rows see no key (O = 0, lse = -inf) and, with the
    split, later rows see keys in only one half."""
    split = pasa.fwd_key_split(1, Sq, Skv, heads, D, True)
    assert split == (1 if heads == 7 else 0)
    w = W.custom(1, Sq, Skv, heads, 1, D, True, kind="bias", seed=Sq + Skv + heads + D, bias=20.0)
    say("causal item shape", "split" if split else "256 rows", w)
    (q, k, v), o, lse = run_fwd(pasa, w)
    ro, rl = attn_fp64(q, k, v, w.scale, True)
    empty = np.isneginf(rl)
    if empty.any():
        b, h, i = np.nonzero(empty)
        assert np.all(o[b, i, h] == 0)
        assert np.all(np.isneginf(lse[empty]))
    assert nonfinite(o) == 0
    check_o(o, ro, v, label=f"causal {'split' if split else 'full'} D{D} {Sq}x{Skv}")
    assert lse_ok(lse, rl)


# ----------------------------------------------------------------- streams, graphs
def test_concurrent_streams_match_serial(pasa):
    """The library keeps no state: prefill and decode enqueued on two streams at
    once give the results of running them one after the other."""
    import torch
    wp = W.custom(1, 300, 300, 7, 1, 128, True, kind="bias", seed=71, bias=20.0)
    wd = W.custom(4, 1, 777, 8, 2, 64, False, kind="bias", seed=72, bias=20.0)
    qp, kp, vp = to_gpu(*W.generate(wp))
    qd, kd, vd = to_gpu(*W.generate(wd))
    ref_p, ref_pl = pasa.attn_fwd(qp, kp, vp, causal=True, scale=wp.scale)
    ws, n = pasa.decode_workspace(qd, kd)
    ref_d, ref_dl = pasa.attn_decode(qd, kd, vd, scale=wd.scale, workspace=ws, num_splits=n)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws2, _ = pasa.decode_workspace(qd, kd, n)
    outs = []
    for _ in range(3):
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            op, opl = pasa.attn_fwd(qp, kp, vp, causal=True, scale=wp.scale)
        with torch.cuda.stream(s2):
            od, odl = pasa.attn_decode(qd, kd, vd, scale=wd.scale, workspace=ws2, num_splits=n)
        torch.cuda.synchronize()
        outs.append((op, opl, od, odl))
    for op, opl, od, odl in outs:
        assert torch.equal(op, ref_p) and torch.equal(opl, ref_pl)
        assert torch.equal(od, ref_d) and torch.equal(odl, ref_dl)


def test_graph_replays_match_eager(pasa):
    """Prefill and decode (split + combine) captured in a HIP graph: every
    replay, with eager work and synchronisation between replays, reproduces the
    eager results bit for bit (the path records no memset)."""
    import torch
    wp = W.custom(1, 257, 257, 4, 2, 64, True, kind="bias", seed=73, bias=25.0)
    wd = W.custom(3, 1, 1000, 7, 1, 128, False, kind="bias", seed=74, bias=25.0)
    qp, kp, vp = to_gpu(*W.generate(wp))
    qd, kd, vd = to_gpu(*W.generate(wd))
    ws, n = pasa.decode_workspace(qd, kd)
    op = torch.empty_like(qp)
    lp = torch.empty((1, 4, 257), dtype=torch.float32, device="cuda")
    od = torch.empty_like(qd)
    ld = torch.empty((3, 7), dtype=torch.float32, device="cuda")

    on = torch.empty_like(qp)     # a non-causal prefill of few items takes the key split
    ln = torch.empty_like(lp)

    def step():
        pasa.attn_fwd(qp, kp, vp, causal=True, scale=wp.scale, out=op, lse=lp)
        pasa.attn_fwd(qp, kp, vp, causal=False, scale=wp.scale, out=on, lse=ln)
        pasa.attn_decode(qd, kd, vd, scale=wd.scale, out=od, lse=ld, workspace=ws, num_splits=n)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (op, lp, on, ln, od, ld)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm the capture stream, as torch recommends
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        for t in (op, lp, on, ln, od, ld):
            t.fill_(float("nan"))
        junk = torch.randn(1 << 16, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("replay", r, float(junk))
        for t, rt in zip((op, lp, on, ln, od, ld), ref):
            assert torch.equal(t, rt), f"replay {r} differs"
