"""CPU checks of the sweep's binary64 replay of PASA's per-block shift rule
(tests/sweep.py, refine_rate) on hand-built inputs whose outcome is known."""
import math

import numpy as np

import workloads as W
from tests.sweep import THETA, block_keys, refine_rate


def _one_row(scores, D=128):
    """q, k whose single row of unscaled scores is `scores` (one head)."""
    w = W.custom(1, 1, len(scores), 1, 1, D, False)
    q = np.zeros((1, 1, 1, D), np.float16)
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, len(scores), 1, D), np.float16)
    k[0, :, 0, 0] = np.asarray(scores, np.float16)
    return q, k, w


def test_flat_scores_never_refine():
    q, k, w = _one_row(np.zeros(3 * block_keys(128)))
    assert refine_rate(q, k, w, np.array([0])) == 0.0


def test_upward_jump_refines_once():
    bc = block_keys(128)
    c = (1.0 / math.sqrt(128)) / math.log(2.0)
    s = np.zeros(2 * bc)
    s[bc + 5] = (10 * THETA) / c          # second block: one key 10*THETA above the rest
    q, k, w = _one_row(s)
    assert refine_rate(q, k, w, np.array([0])) == 0.5


def test_jump_below_threshold_does_not_refine():
    bc = block_keys(128)
    c = (1.0 / math.sqrt(128)) / math.log(2.0)
    s = np.zeros(2 * bc)
    s[bc + 5] = (0.5 * THETA) / c
    q, k, w = _one_row(s)
    assert refine_rate(q, k, w, np.array([0])) == 0.0
