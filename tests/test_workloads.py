"""The synthetic inputs carry the overflow mechanisms the PASA page names
("Online Pseudo-average Shifting Attention (PASA) ...", Abstract): a large
sequence-dimension bias pushes unscaled QK^T past the fp16 maximum, and query/key
resonance (phase coincidence or a 180-degree shift) amplifies scores."""
import json
import os

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FP16_MAX = json.load(open(os.path.join(GOLDEN, "fp16_overflow.json")))["fp16_max"]


def _small(name, **over):
    w = W.CONFIGS[name]
    d = dict(batch=w.batch, seqlen_q=w.seqlen_q, seqlen_kv=w.seqlen_kv, heads_q=w.heads_q,
             heads_kv=w.heads_kv, head_dim=w.head_dim, causal=w.causal, kind=w.kind,
             seed=w.seed, **w.params)
    d.update(over)
    return W.custom(**d)


def test_deterministic_and_fp16():
    w = W.CONFIGS["c1"]
    a = W.generate(w)
    b = W.generate(w)
    for x, y in zip(a, b):
        assert x.dtype == np.float16 and x.flags["C_CONTIGUOUS"]
        np.testing.assert_array_equal(x, y)
    assert a[0].shape == (1, 256, 1, 64)
    # q, k, v come from independent streams
    assert not np.array_equal(a[0], a[1])


def test_bias_overflows_unscaled_fp16():
    w = _small("c2", seqlen_q=256, seqlen_kv=256)
    q, k, _ = W.generate(w)
    s = np.einsum("shd,sd->sh", q[0, :, :4].astype(np.float64), k[0, :, 0].astype(np.float64))
    assert s.max() > FP16_MAX          # naive fp16 conversion of QK^T overflows
    assert abs(s.mean() - 30 * 30 * 128) / (30 * 30 * 128) < 0.02
    # but the scaled score, in log2 units, stays inside the fp16 range
    assert s.max() / np.sqrt(128) * np.log2(np.e) < FP16_MAX


def test_resonance_amplitude_and_flip():
    w = _small("c3", batch=1, seqlen_q=64, seqlen_kv=9216, heads_q=2, heads_kv=2)
    q, k, _ = W.generate(w)
    qf = q[0, :, 0].astype(np.float64)
    kf = k[0, :, 0].astype(np.float64)
    s = qf @ kf.T
    same = s[:, :4608]
    flip = s[:, 4608:]
    assert abs(np.median(same) - 48 * 48 * 32) / (48 * 48 * 32) < 0.02   # ~7.37e4
    assert abs(np.median(flip) + 48 * 48 * 32) / (48 * 48 * 32) < 0.02
    assert np.abs(s).max() > FP16_MAX


def test_amp_bias_per_head_draws_differ():
    w = _small("c4", seqlen_q=64, seqlen_kv=64)
    q, k, _ = W.generate(w)
    mq = q[0].astype(np.float64).mean(axis=(0, 2))
    sq = q[0].astype(np.float64).std(axis=(0, 2))
    assert q.shape == (1, 64, 32, 128) and k.shape == (1, 64, 8, 128)
    assert np.all((mq > -1) & (mq < 31))
    assert np.all((sq > 0.4) & (sq < 4.3))
    assert np.ptp(mq) > 5 and np.ptp(sq) > 1


def test_flop_and_byte_accounting():
    c2 = W.CONFIGS["c2"]
    assert c2.visible_pairs() == 28 * 4096 * 4097 // 2
    assert c2.flops() == 4 * 128 * 28 * 4096 * 4097 // 2
    c5 = W.CONFIGS["c5"]
    assert c5.io_bytes() == 2 * 64 * 8192 * 4 * 128 * 2 + 2 * 64 * 28 * 128 * 2 + 64 * 28 * 4
    w = W.custom(1, 6, 4, 1, 1, 8, True)
    assert w.visible_pairs() == 0 + 0 + 1 + 2 + 3 + 4
