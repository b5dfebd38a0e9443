"""pasa_attn_decode_noalloc, called through the C ABI, against
pasa_attn_decode on the same inputs: the same kernels and split count, so the
outputs must agree bit for bit (the oracle bar is implied).  Two calls in a
row, the second with a smaller input, so the second reads the scratch area
the first left behind; and a call whose partials exceed the scratch area is
refused without touching the output."""
import ctypes

import numpy as np
import pytest

import workloads as W
from tests.gpu_common import say, to_gpu

pytestmark = pytest.mark.gpu


def _noalloc(lib, q, k, v, o, lse, w, n):
    import torch
    f = lib.pasa_attn_decode_noalloc
    f.restype = ctypes.c_int
    return f(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
             ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
             ctypes.c_void_p(lse.data_ptr()), w.batch, w.seqlen_kv, w.heads_q, w.group,
             w.head_dim, ctypes.c_float(w.scale), n,
             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_decode_matches_workspace_decode_twice():
    import torch
    import precision_flashattention_numerics_amd as pasa
    lib = pasa.raw()
    for w, n in ((W.CONFIGS["c5"], 0),
                 (W.custom(3, 1, 1000, 8, 2, 64, False, kind="bias", seed=12, bias=20.0), 5)):
        say("noalloc decode", w.batch, w.seqlen_kv, w.heads_q, w.heads_kv, w.head_dim, "splits", n)
        q, k, v = to_gpu(*W.generate(w))
        ref_o, ref_l = pasa.attn_decode(q, k, v, num_splits=n, scale=w.scale)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((w.batch, w.heads_q), float("nan"), dtype=torch.float32, device="cuda")
        assert _noalloc(lib, q, k, v, o, lse, w, n) == 0
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)
        assert bool(torch.isfinite(o).all())


def test_noalloc_refuses_partials_beyond_the_scratch_area():
    import torch
    import precision_flashattention_numerics_amd as pasa
    lib = pasa.raw()
    # 512 sequences x 64 heads x 8 splits x 128 floats of partials: 128 MiB
    w = W.custom(512, 1, 256, 64, 8, 128, False, kind="normal", seed=1)
    q = torch.zeros((w.batch, 1, w.heads_q, w.head_dim), dtype=torch.float16, device="cuda")
    k = torch.zeros((w.batch, w.seqlen_kv, w.heads_kv, w.head_dim), dtype=torch.float16,
                    device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.zeros((w.batch, w.heads_q), dtype=torch.float32, device="cuda")
    assert _noalloc(lib, q, k, k, o, lse, w, 8) == -3
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())


def test_noalloc_decode_in_a_graph_matches_eager():
    """The callers the entry point is for include code under HIP graph
    capture: captured once, every replay (with new inputs copied in, and eager
    work and synchronisation between replays) reproduces the workspace decode
    on those inputs bit for bit."""
    import torch
    import precision_flashattention_numerics_amd as pasa
    lib = pasa.raw()
    w = W.custom(4, 1, 3000, 14, 2, 128, False, kind="bias", seed=31, bias=25.0)
    q, k, v = to_gpu(*W.generate(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.heads_q), dtype=torch.float32, device="cuda")
    assert _noalloc(lib, q, k, v, o, lse, w, 0) == 0   # first call on the device: outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rc = _noalloc(lib, q, k, v, o, lse, w, 0)
    assert rc == 0
    for rep in range(3):
        w2 = W.custom(4, 1, 3000, 14, 2, 128, False, kind="bias", seed=40 + rep, bias=5.0 + 10 * rep)
        q2, k2, v2 = to_gpu(*W.generate(w2))
        q.copy_(q2); k.copy_(k2); v.copy_(v2)
        ref_o, ref_l = pasa.attn_decode(q2, k2, v2, scale=w.scale)
        torch.cuda.synchronize()
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        say("noalloc graph replay", rep)
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)
