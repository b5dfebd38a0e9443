"""The kernel follows the per-block rule the CPU fp16 model replays
(tests/numerics_model.py): on sampled rows of the Qwen2-shaped input the
PASA prefill lands much closer to the model of its own rule (tile formed
against the running maximum, pseudo-average as the first block's reference)
than to the model of the pseudo-average-only centring, whose error is about
eight times larger ("Online Pseudo-average Shifting Attention (PASA) ...",
Abstract: pseudo-average shifting keeps the half-precision tile in range)."""
import numpy as np
import pytest

import workloads as W
from tests.gpu_common import gather_rows, say, to_gpu
from tests.numerics_model import emulate
from workloads.metrics import rel_rmse

pytestmark = pytest.mark.gpu


def test_prefill_tracks_the_modelled_rule():
    import torch
    import precision_flashattention_numerics_amd as pasa
    w = W.CONFIGS["c2"]
    q, k, v = W.generate(w)
    tq, tk, tv = to_gpu(q, k, v)
    o, lse = pasa.attn_fwd(tq, tk, tv, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(11).choice(w.heads_q * w.seqlen_q, 128, replace=False))
    go, _ = gather_rows(o.cpu().numpy(), lse.cpu().numpy(), w, rows)
    rule, _ = emulate(q, k, v, w.scale, True, rows, 64, "fused")
    alone, _ = emulate(q, k, v, w.scale, True, rows, 64, "mu_only")
    d_rule, d_alone = rel_rmse(go, rule), rel_rmse(go, alone)
    say("kernel vs modelled rule", d_rule, "vs pseudo-average-only centring", d_alone)
    assert d_rule < 0.3 * d_alone
