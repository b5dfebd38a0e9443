"""The designed-random sweep (tests/sweep.py) on its quick grid: PASA within the
bar everywhere, the strict variant within the bar inside its stated range, and
the naive fp16 kernel overflowing exactly where an unscaled score rounds to
fp16 infinity ("Online Pseudo-average Shifting Attention (PASA) ...",
Abstract: overflow above 65504)."""
import math

import pytest

from tests.gpu_common import REL_RMSE_MAX, ROW_REL_MAX, say
from tests.sweep import STRICT_RANGE, measure, onsets, points

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def results():
    import precision_flashattention_numerics_amd as pasa
    out = []
    for n, pt in enumerate(points(full=False)):
        say("sweep point", pt)
        r = measure(pasa, pt, seed=100 + n)
        say("  max|s|", round(r["max_abs_s"]), "naive bad", r["naive_nonfinite"],
            "strict", r["strict_rel_rmse"], "pasa", r["pasa_rel_rmse"])
        out.append(r)
    return out


def test_grid_spans_both_sides_of_the_overflow(results):
    assert any(r["naive_overflow"] for r in results)
    assert any(not r["naive_overflow"] for r in results)


def test_pasa_within_bar_everywhere(results):
    for r in results:
        assert r["pasa_nonfinite"] == 0, r
        assert r["pasa_rel_rmse"] <= REL_RMSE_MAX, r
        assert r["pasa_head_max"] <= REL_RMSE_MAX, r
        assert r["pasa_row_max"] <= ROW_REL_MAX, r


def test_grid_spans_phase_offsets(results):
    """At least three query/key phase offsets, with the naive overflow on the
    in-phase and anti-phase ends and none at a quarter turn."""
    ph = [r for r in results if r["kind"] == "phase"]
    assert len({round(r["offset"], 6) for r in ph}) >= 3
    for r in ph:
        if abs(math.cos(r["offset"])) < 0.75:
            assert not r["naive_overflow"] and r["naive_nonfinite"] == 0, r
        if abs(math.cos(r["offset"])) > 0.99:
            assert r["naive_overflow"] and r["naive_nonfinite"] > 0, r


def test_strict_within_bar_inside_its_range(results):
    inside = [r for r in results if r["max_abs_cs"] < STRICT_RANGE]
    assert inside
    for r in inside:
        assert r["strict_nonfinite"] == 0, r
        assert r["strict_rel_rmse"] <= REL_RMSE_MAX, r
        assert r["strict_head_max"] <= REL_RMSE_MAX, r


def test_naive_overflows_exactly_where_predicted(results):
    # a margin around the rounding edge absorbs the fp32 accumulation order
    for r in results:
        assert r["s_rows"] == "all"
        if r["max_abs_s"] > 66000.0:
            assert r["naive_nonfinite"] > 0, r
        elif r["max_abs_s"] < 65000.0:
            assert r["naive_nonfinite"] == 0, r
    for key, o in onsets(results).items():
        say("onset", key, o)
