"""PASA forward with e4m3 queries and keys against the binary64 oracle run on
the dequantised inputs (the e4m3 values times their scales are exact reals,
so the oracle sees exactly what the kernel is given).

The output bar is the fp16 path's.  The lse bound is wider in relative terms:
the fp8 matrix instruction sums its 64 products less exactly than the fp16
one sums 16, so scores of magnitude 7e4 (the resonance input) come out with
errors of a few parts in 1e6; lse is held to max(1e-2, 4e-6 |lse|)."""
import numpy as np
import pytest

import workloads as W
from oracle import attn_fp64
from tests.gpu_common import (check_o, gather_rows, lse_error, lse_ok, nonfinite, row_heads,
                              sample_rows, say)

pytestmark = pytest.mark.gpu

E4M3_MAX = 448.0
LSE_REL = 4e-6


@pytest.fixture(scope="module")
def pasa():
    import precision_flashattention_numerics_amd as p
    return p


def quantize(x):
    """Per-tensor e4m3: scale = max|x| / 448, saturating round-to-nearest."""
    import torch
    t = torch.from_numpy(x.astype(np.float32))
    s = float(t.abs().max()) / E4M3_MAX or 1.0
    q8 = torch.clamp(t / s, -E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q8, s, q8.to(torch.float64).numpy() * s


def run(pasa, w, rows=None):
    import torch
    q, k, v = W.generate(w)
    q8, qs, qd = quantize(q)
    k8, ks, kd = quantize(k)
    o, lse = pasa.attn_fwd_fp8(q8.cuda(), k8.cuda(), torch.from_numpy(v).cuda(), qs, ks,
                               causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    ro, rl = attn_fp64(qd, kd, v, w.scale, w.causal, rows=rows)
    return o, lse, ro, rl, v


@pytest.mark.parametrize("shape", [(1, 127, 300, 7, 1, 64, True), (2, 300, 129, 2, 2, 128, False),
                                   (1, 1, 1, 1, 1, 128, False), (1, 257, 257, 4, 2, 128, True)],
                         ids=lambda s: "x".join(map(str, s)))
def test_fp8_small_shapes_vs_oracle(pasa, shape):
    B, Sq, Skv, Hq, Hkv, D, causal = shape
    w = W.custom(B, Sq, Skv, Hq, Hkv, D, causal, kind="bias", seed=sum(shape), bias=3.0)
    say("fp8 case", shape)
    o, lse, ro, rl, v = run(pasa, w)
    check_o(o, ro, v, label=f"fp8 {shape}")
    assert lse_ok(lse, rl, rel_tol=LSE_REL)


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_fp8_configs_vs_oracle(pasa, name):
    w = W.CONFIGS[name]
    say("fp8 config", name)
    rows = None if name == "c1" else sample_rows(w, 512, np.random.default_rng(8))
    o, lse, ro, rl, v = run(pasa, w, rows)
    assert nonfinite(o) == 0 and nonfinite(lse) == 0
    go, gl = (o, lse) if rows is None else gather_rows(o, lse, w, rows)
    check_o(go, ro, v, heads=None if rows is None else row_heads(w, rows), label=f"fp8 {name}")
    say(name, "fp8 lse_err", lse_error(gl, rl))
    assert lse_ok(gl, rl, rel_tol=LSE_REL)
