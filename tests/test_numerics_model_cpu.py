"""What each step of the per-block rule contributes, on the CPU fp16 model of
the kernels (tests/numerics_model.py), against the binary64 oracle.

"Online Pseudo-average Shifting Attention (PASA) ...", Abstract: the
pseudo-average shift keeps the half-precision tile in range.  On matrix
units that emit fp32 scores (CDNA's), the kernels form each fp16 exponent
argument straight from the fp32 score against the running maximum, so:
  * the pseudo-average only decides the base s is rounded against: on the
    biased inputs it is never selected (the running maximum dominates it) and
    the output is bit-identical without it; on unbiased inputs it moves the
    result at the rounding level, within the bar either way;
  * centring the tile at the pseudo-average alone, without the running
    maximum, multiplies the error on the Qwen2-shaped input about eightfold
    (to the edge of the output bar, and past the lse bar on some rows);
  * shifting the keys by their block mean in fp16 before the product (the
    placement hardware with fp16-output matrix units needs) adds rounding
    error amplified by |q|: about six times the error, and past the lse bar.
These pins fail if the rule the kernels follow loses the running-maximum
reference, and they record why the shift is applied to the fp32 scores.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attn_fp64
from tests.numerics_model import emulate
from workloads.metrics import rel_rmse

REL_BAR, LSE_BAR = 2e-3, 1e-2


def _slice(w, n, seed):
    q, k, v = W.generate(w)
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(w.batch * w.heads_q * w.seqlen_q, n, replace=False))
    ro, rl = attn_fp64(q, k, v, w.scale, w.causal, rows=rows)
    return q, k, v, rows, ro, rl


@pytest.fixture(scope="module")
def qwen2_slice():
    w = W.CONFIGS["c2"]
    return w, _slice(w, 200, 7)


def _run(w, sl, variant):
    q, k, v, rows, ro, rl = sl
    o, l = emulate(q, k, v, w.scale, w.causal, rows, 64 if w.head_dim == 128 else 128, variant)
    return o, l, rel_rmse(o, ro), float(np.max(np.abs(l - rl)))


def test_kernel_rule_within_bar_and_pseudo_average_inert_on_bias(qwen2_slice):
    w, sl = qwen2_slice
    o1, l1, e1, le1 = _run(w, sl, "fused")
    o2, l2, e2, le2 = _run(w, sl, "fused_no_mu")
    assert e1 <= REL_BAR and le1 <= LSE_BAR
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_pseudo_average_alone_loses_accuracy(qwen2_slice):
    w, sl = qwen2_slice
    _, _, e_fused, le_fused = _run(w, sl, "fused")
    _, _, e, le = _run(w, sl, "mu_only")
    assert e > 5 * e_fused and le > 5 * le_fused, (e, e_fused, le, le_fused)


def test_key_shift_before_the_product_misses_the_lse_bar(qwen2_slice):
    w, sl = qwen2_slice
    _, _, e_fused, le_fused = _run(w, sl, "fused")
    _, _, e, le = _run(w, sl, "kshift")
    assert le > LSE_BAR, le
    assert e > 4 * e_fused and le > 5 * le_fused, (e, e_fused, le, le_fused)


def test_pseudo_average_moves_unbiased_rows_at_rounding_level():
    w = W.CONFIGS["c1"]
    sl = _slice(w, 256, 6)
    o1, _, e1, le1 = _run(w, sl, "fused")
    o2, _, e2, le2 = _run(w, sl, "fused_no_mu")
    assert e1 <= REL_BAR and e2 <= REL_BAR and le1 <= LSE_BAR and le2 <= LSE_BAR
    d = rel_rmse(o1, o2)
    assert 0 < d < REL_BAR, d


def test_two_rounding_tile_within_bar(qwen2_slice):
    """Forming the shifted fp16 tile first and subtracting s in fp16 (two fp16
    roundings) stays within the bar as well; the kernels form X straight from
    the fp32 score."""
    w, sl = qwen2_slice
    _, _, e, le = _run(w, sl, "two_round")
    assert e <= REL_BAR and le <= LSE_BAR
