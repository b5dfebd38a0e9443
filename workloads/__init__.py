"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This module draws inputs only; it holds none of the attention arithmetic.  Both
the CPU oracle and the HIP path receive the very same fp16 arrays it returns.

The overflow mechanisms come from "Online Pseudo-average Shifting Attention
(PASA) for Robust Low-precision LLM Inference", Abstract: a large bias along the
sequence dimension (Qwen2-7B) and query/key "resonance" in the head dimension,
i.e. phase coincidence or a 180-degree phase shift between query and key
(Stable-Video-Diffusion); amplitude is named as the other factor.  The real
model activations are not available, so these generators stand in for them by
shape and value structure only.

Recipe: values are drawn in float64 from numpy's PCG64, seeded through
SeedSequence(seed).spawn(4) -- one child stream each for Q, K, V and the
per-head parameters -- transformed, then rounded to fp16 (round-to-nearest-even,
numpy's cast).
"""
from dataclasses import dataclass, field
import math

import numpy as np

FP16_MAX = 65504.0


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen_q: int
    seqlen_kv: int
    heads_q: int
    heads_kv: int
    head_dim: int
    causal: bool
    kind: str            # "normal" | "bias" | "resonance" | "amp_bias" | "jump"
    seed: int
    description: str = ""
    params: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def is_decode(self) -> bool:
        return self.seqlen_q == 1 and not self.causal

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs the mask lets through, over all (b, hq)."""
        sq, skv = self.seqlen_q, self.seqlen_kv
        if not self.causal:
            per = sq * skv
        else:
            # bottom-right alignment: row i sees keys j <= i + skv - sq
            per = 0
            first = max(0, sq - skv)  # rows before this see nothing
            # rows first..sq-1 see (i + skv - sq + 1) keys, capped at skv
            for_rows = np.arange(first, sq, dtype=np.int64) + (skv - sq + 1)
            per = int(np.minimum(for_rows, skv).sum())
        return per * self.batch * self.heads_q

    def flops(self) -> int:
        """Algorithmic flops: 2*D for QK^T plus 2*D for PV per visible pair."""
        return 4 * self.head_dim * self.visible_pairs()

    def io_bytes(self) -> int:
        """Algorithmic HBM bytes: q, k, v read once, o written once (fp16), lse (fp32)."""
        b, d = self.batch, self.head_dim
        q = b * self.seqlen_q * self.heads_q * d * 2
        kv = 2 * b * self.seqlen_kv * self.heads_kv * d * 2
        return q + kv + q + b * self.heads_q * self.seqlen_q * 4


CONFIGS = {
    "c1": Workload("c1", 1, 256, 256, 1, 1, 64, False, "normal", 1,
                   "single head, N(0,1), non-causal, seq 256, D 64"),
    "c2": Workload("c2", 1, 4096, 4096, 28, 4, 128, True, "bias", 2,
                   "Qwen2-7B-shaped causal prefill, bias 30 on q and k",
                   {"bias": 30.0}),
    "c3": Workload("c3", 2, 9216, 9216, 5, 5, 64, False, "resonance", 3,
                   "Stable-Video-Diffusion-shaped resonance, amplitude 48, "
                   "key phase flipped by pi for rows >= 4608",
                   {"amp": 48.0, "period": 64, "flip_at": 4608, "per_row_phase": False}),
    "c4": Workload("c4", 1, 32768, 32768, 32, 8, 128, True, "amp_bias", 4,
                   "long-context causal prefill, per-head amplitude U(0.5,4) and bias U(0,30)",
                   {"amp_lo": 0.5, "amp_hi": 4.0, "bias_lo": 0.0, "bias_hi": 30.0}),
    "c5": Workload("c5", 64, 1, 8192, 28, 4, 128, False, "bias", 5,
                   "decode: 64 sequences, one query token, KV length 8192, bias 30",
                   {"bias": 30.0}),
}


def custom(batch, seqlen_q, seqlen_kv, heads_q, heads_kv, head_dim, causal,
           kind="normal", seed=0, name="custom", **params) -> Workload:
    """A workload of any shape with one of the value recipes below."""
    return Workload(name, batch, seqlen_q, seqlen_kv, heads_q, heads_kv, head_dim,
                    bool(causal), kind, int(seed), "", dict(params))


def _streams(seed):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(4)]


def _normal_fp16(rng, shape, mul=None, add=None, chunk_axis0=True):
    """N(0,1) draws in float64, optionally a*x + b (broadcast over the head
    axis), rounded to fp16.  Drawn one leading index at a time so that large
    tensors never exist in float64 all at once; the stream is consumed in the
    same order either way."""
    out = np.empty(shape, np.float16)
    for i in range(shape[0]):
        x = rng.standard_normal(shape[1:])
        if mul is not None:
            x *= mul
        if add is not None:
            x += add
        out[i] = x.astype(np.float16)
    return out


def _amp_bias_params(rp, w):
    """Per-head amplitude and bias draws of the "amp_bias" recipe, in the order
    they are taken from the parameter stream: a_q, b_q (one per query head),
    a_k, b_k (one per key/value head)."""
    p = w.params
    aq = rp.uniform(p.get("amp_lo", 0.5), p.get("amp_hi", 4.0), w.heads_q)
    bq = rp.uniform(p.get("bias_lo", 0.0), p.get("bias_hi", 30.0), w.heads_q)
    ak = rp.uniform(p.get("amp_lo", 0.5), p.get("amp_hi", 4.0), w.heads_kv)
    bk = rp.uniform(p.get("bias_lo", 0.0), p.get("bias_hi", 30.0), w.heads_kv)
    return aq, bq, ak, bk


def head_params(w: Workload):
    """(a_q, b_q, a_k, b_k) of an "amp_bias" workload, as generate() draws them."""
    if w.kind != "amp_bias":
        raise ValueError("head_params: only the amp_bias recipe has per-head draws")
    return _amp_bias_params(_streams(w.seed)[3], w)


def generate(w: Workload):
    """Return (q, k, v) as contiguous fp16 numpy arrays in BSHD layout."""
    rq, rk, rv, rp = _streams(w.seed)
    B, Sq, Skv, Hq, Hkv, D = (w.batch, w.seqlen_q, w.seqlen_kv, w.heads_q,
                              w.heads_kv, w.head_dim)
    qs, ks = (B, Sq, Hq, D), (B, Skv, Hkv, D)
    p = w.params
    if w.kind == "normal":
        q = _normal_fp16(rq, qs)
        k = _normal_fp16(rk, ks)
    elif w.kind == "bias":
        bias = p.get("bias", 30.0)
        q = _normal_fp16(rq, qs, add=bias)
        k = _normal_fp16(rk, ks, add=bias)
    elif w.kind == "amp_bias":
        aq, bq, ak, bk = _amp_bias_params(rp, w)
        q = _normal_fp16(rq, qs, mul=aq[:, None], add=bq[:, None])
        k = _normal_fp16(rk, ks, mul=ak[:, None], add=bk[:, None])
    elif w.kind == "resonance":
        amp = p.get("amp", 48.0)
        period = p.get("period", 64)
        flip_at = p.get("flip_at", Skv // 2)
        if Hq != Hkv:
            raise ValueError("resonance recipe assumes one key head per query head")
        dd = 2.0 * math.pi * np.arange(D) / period
        if p.get("per_row_phase", False):
            # stress reading: an independent phase for every query row
            phi_q = rp.uniform(0.0, 2.0 * math.pi, (B, Sq, Hq))
            phi_k = rp.uniform(0.0, 2.0 * math.pi, (B, 1, Hkv)) * np.ones((1, Skv, 1))
        else:
            phi = rp.uniform(0.0, 2.0 * math.pi, (B, Hq))
            phi_q = np.broadcast_to(phi[:, None, :], (B, Sq, Hq))
            phi_k = np.broadcast_to(phi[:, None, :], (B, Skv, Hkv)).copy()
        # key phase = query phase + phase_offset, plus pi from row flip_at on
        # (flip_at = Skv: no flip)
        phi_k = (phi_k + p.get("phase_offset", 0.0)
                 + math.pi * (np.arange(Skv) >= flip_at)[None, :, None])
        q = np.empty(qs, np.float16)
        k = np.empty(ks, np.float16)
        for b in range(B):
            q[b] = (amp * np.cos(dd[None, None, :] + phi_q[b][..., None])
                    + rq.standard_normal(qs[1:])).astype(np.float16)
            k[b] = (amp * np.cos(dd[None, None, :] + phi_k[b][..., None])
                    + rk.standard_normal(ks[1:])).astype(np.float16)
    elif w.kind == "jump":
        # Stress input: a small bias for the first keys, then a jump of the key
        # bias so that the later scores exceed the fp16 range by far when
        # unscaled and climb steeply in the scaled domain.
        b0 = p.get("bias_lo", 2.0)
        b1 = p.get("bias_hi", 60.0)
        at = p.get("jump_at", Skv // 2)
        q = _normal_fp16(rq, qs, add=p.get("q_bias", 30.0))
        kb = np.where(np.arange(Skv) >= at, b1, b0)[:, None, None]
        k = np.empty(ks, np.float16)
        for b in range(B):
            k[b] = (rk.standard_normal(ks[1:]) + kb).astype(np.float16)
    else:
        raise ValueError(f"unknown workload kind {w.kind!r}")
    v = _normal_fp16(rv, ks)
    return np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v)
