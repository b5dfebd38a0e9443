"""Paged split-KV decode against the binary64 oracle: each sequence's keys are
gathered from its pages into a contiguous cache on the host and the oracle
runs on that; the decode itself reads the pages through the block table."""
import numpy as np
import pytest

import workloads as W
from oracle import attn_fp64
from tests.gpu_common import REL_RMSE_MAX, check_o, lse_ok, nonfinite, rel_rmse, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pasa():
    import precision_flashattention_numerics_amd as p
    return p


def paged_case(B, lens, Hq, Hkv, D, page_size, seed, bias=30.0, spare_pages=5):
    """Random pool: every sequence's pages are scattered over a shuffled pool;
    table entries past a sequence's end are -1."""
    rng = np.random.default_rng(seed)
    max_pages = max(1, max((n + page_size - 1) // page_size for n in lens))
    need = sum((n + page_size - 1) // page_size for n in lens)
    num_pages = need + spare_pages
    w = W.custom(1, 1, num_pages * page_size, Hkv, Hkv, D, False, kind="bias", seed=seed,
                 bias=bias)
    _, kpool, vpool = W.generate(w)          # [1, pages*page_size, Hkv, D]
    kpool = kpool.reshape(num_pages, page_size, Hkv, D)
    vpool = vpool.reshape(num_pages, page_size, Hkv, D)
    wq = W.custom(B, 1, 1, Hq, Hkv, D, False, kind="bias", seed=seed + 1, bias=bias)
    q = W.generate(wq)[0]
    perm = rng.permutation(num_pages)
    table = np.full((B, max_pages), -1, np.int32)
    nxt = 0
    for b, n in enumerate(lens):
        for p in range((n + page_size - 1) // page_size):
            table[b, p] = perm[nxt]
            nxt += 1
    return q, kpool, vpool, table, np.array(lens, np.int32)


def oracle_paged(q, kpool, vpool, table, lens, scale):
    B, _, Hq, D = q.shape
    page_size, Hkv = kpool.shape[1], kpool.shape[2]
    o = np.zeros((B, 1, Hq, D))
    lse = np.zeros((B, Hq))
    for b, n in enumerate(lens):
        if n == 0:
            lse[b] = -np.inf
            continue
        pages = table[b, :(n + page_size - 1) // page_size]
        k = np.concatenate([kpool[p] for p in pages])[:n][None]
        v = np.concatenate([vpool[p] for p in pages])[:n][None]
        ob, lb = attn_fp64(q[b:b + 1], k, v, scale, False)
        o[b], lse[b] = ob[0], lb[0, :, 0]
    return o, lse


def run_paged(pasa, q, kpool, vpool, table, lens, num_splits=0):
    import torch
    tq, tk, tv = (torch.from_numpy(x).cuda() for x in (q, kpool, vpool))
    tt, tl = torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda()
    scale = q.shape[-1] ** -0.5
    o, lse = pasa.attn_decode_paged(tq, tk, tv, tt, tl, num_splits=num_splits, scale=scale)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy(), scale


CASES = [
    # (lens, Hq, Hkv, D, page_size)
    ([1, 31, 32, 33, 64, 65, 1000, 4097], 28, 4, 128, 32),
    ([0, 5, 256, 257, 3000], 28, 4, 128, 256),
    ([129, 2048, 700], 8, 8, 64, 64),
    ([6000, 1, 511], 7, 1, 64, 128),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"ps{c[4]}-D{c[3]}-{c[1]}x{c[2]}")
def test_paged_decode_vs_oracle(pasa, case):
    lens, Hq, Hkv, D, ps = case
    say("paged case", case)
    q, kp, vp, table, ln = paged_case(len(lens), lens, Hq, Hkv, D, ps, seed=sum(lens) % 997)
    o, lse, scale = run_paged(pasa, q, kp, vp, table, ln)
    ro, rl = oracle_paged(q, kp, vp, table, ln, scale)
    assert nonfinite(o) == 0
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))
    nz = [b for b, n in enumerate(lens) if n > 0]
    check_o(o[nz], ro[nz], vp, label=f"paged {case}")
    assert lse_ok(lse, rl)


@pytest.mark.parametrize("splits", [0, 1, 7])
def test_paged_matches_contiguous_bitwise(pasa, splits):
    """With the pages in order and the same key bound, the paged decode makes
    the same splits and the same arithmetic as the contiguous one."""
    import torch
    B, S, Hq, Hkv, D, ps = 4, 2048, 28, 4, 128, 64
    w = W.custom(B, 1, S, Hq, Hkv, D, False, kind="bias", seed=77, bias=30.0)
    q, k, v = W.generate(w)
    tq, tk, tv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    oc, lc = pasa.attn_decode(tq, tk, tv, num_splits=splits, scale=w.scale)
    kpool = tk.reshape(B * S // ps, ps, Hkv, D)
    vpool = tv.reshape(B * S // ps, ps, Hkv, D)
    table = torch.arange(B * S // ps, dtype=torch.int32, device="cuda").reshape(B, S // ps)
    lens = torch.full((B,), S, dtype=torch.int32, device="cuda")
    op, lp = pasa.attn_decode_paged(tq, kpool, vpool, table, lens, num_splits=splits,
                                    scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(oc, op)
    assert torch.equal(lc, lp)


def test_paged_out_of_range_page_reads_zero(pasa):
    """A table entry outside the pool reads as zero keys and values (each such
    key still scores 0 and is visible), not as a fault."""
    lens, Hq, Hkv, D, ps = [300], 4, 4, 64, 64
    q, kp, vp, table, ln = paged_case(1, lens, Hq, Hkv, D, ps, seed=5, bias=1.0)
    bad = table.copy()
    bad[0, 1] = kp.shape[0] + 1000
    o, lse, scale = run_paged(pasa, q, kp, vp, bad, ln)
    kz, vz = kp.copy(), vp.copy()
    extra = np.zeros((1,) + kp.shape[1:], kp.dtype)
    kz = np.concatenate([kz, extra])
    vz = np.concatenate([vz, extra])
    ref_table = table.copy()
    ref_table[0, 1] = kz.shape[0] - 1
    ro, rl = oracle_paged(q, kz, vz, ref_table, ln, scale)
    check_o(o, ro, vp, label="paged out-of-range page")
    assert lse_ok(lse, rl)


@pytest.mark.parametrize("S,ps,splits", [(8192, 32, 1), (8192, 32, 3), (16384, 64, 3)])
def test_paged_long_splits_match_contiguous_bitwise(pasa, S, ps, splits):
    """Splits that span more than 64 pages: the page indices of a split are
    taken from the block table 64 at a time, so these cross one or more such
    boundaries (and at page_size 64 with 3 splits the second split starts in
    the middle of a page)."""
    import torch
    B, Hq, Hkv, D = 2, 8, 2, 128
    say("paged long split", S, ps, splits)
    w = W.custom(B, 1, S, Hq, Hkv, D, False, kind="bias", seed=91, bias=30.0)
    q, k, v = W.generate(w)
    tq, tk, tv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    oc, lc = pasa.attn_decode(tq, tk, tv, num_splits=splits, scale=w.scale)
    kpool = tk.reshape(B * S // ps, ps, Hkv, D)
    vpool = tv.reshape(B * S // ps, ps, Hkv, D)
    table = torch.arange(B * S // ps, dtype=torch.int32, device="cuda").reshape(B, S // ps)
    lens = torch.full((B,), S, dtype=torch.int32, device="cuda")
    op, lp = pasa.attn_decode_paged(tq, kpool, vpool, table, lens, num_splits=splits,
                                    scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(oc, op)
    assert torch.equal(lc, lp)


def test_paged_single_split_over_shuffled_pool_vs_oracle(pasa):
    """One split over 256 shuffled 32-key pages (four groups of 64 table
    entries), against the oracle on the gathered keys."""
    lens, Hq, Hkv, D, ps = [8192, 5000], 8, 2, 128, 32
    q, kp, vp, table, ln = paged_case(len(lens), lens, Hq, Hkv, D, ps, seed=13)
    o, lse, scale = run_paged(pasa, q, kp, vp, table, ln, num_splits=1)
    ro, rl = oracle_paged(q, kp, vp, table, ln, scale)
    check_o(o, ro, vp, label="paged single split")
    assert lse_ok(lse, rl)
