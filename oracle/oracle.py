"""ctypes binding of the binary64 CPU oracle (test infrastructure only).

Inputs are converted to float64 exactly (fp16 -> fp64 is exact) before the call,
so the oracle sees the very values the GPU path reads.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PASA_ORACLE_LIB selects another build of the same source (the sanitized one
# the CPU sanitizer test makes)
_LIB_PATH = os.environ.get("PASA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def load():
    """Load liboracle.so, building it with gcc if it is not there yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from .build import build
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_attn_fp64.restype = ctypes.c_int
        lib.oracle_attn_fp64.argtypes = [
            _dp, _dp, _dp,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_int, _dp, _i64p, ctypes.c_int64, _dp, _dp]
        lib.oracle_combine_fp64.restype = None
        lib.oracle_combine_fp64.argtypes = [_dp, _dp, ctypes.c_int64, ctypes.c_int,
                                            ctypes.c_int, _dp, _dp]
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _ptr(a, t=_dp):
    return a.ctypes.data_as(t)


def attn_fp64(q, k, v, scale, causal=False, offset=None, rows=None):
    """Plain softmax attention in binary64.

    q: [B,Sq,Hq,D]; k, v: [B,Skv,Hkv,D] (any real dtype; converted exactly).
    offset: None or [B,Hq,Sq] additive constant per row on the scaled scores.
    rows:   None, or an int array of flat row ids (b*Hq + h)*Sq + i.
    Returns (o, lse): o is [B,Sq,Hq,D] and lse [B,Hq,Sq] for all rows, or
    o [n,D] and lse [n] for the sampled rows.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    if Bk != B or Dk != D or v.shape != k.shape or Hq % Hkv != 0:
        raise ValueError("oracle: inconsistent shapes")
    off = None
    if offset is not None:
        off = _f64(offset)
        if off.shape != (B, Hq, Sq):
            raise ValueError("oracle: offset must be [B,Hq,Sq]")
    lib = load()
    if rows is None:
        o = np.zeros((B, Sq, Hq, D), np.float64)
        lse = np.zeros((B, Hq, Sq), np.float64)
        rp, n = None, 0
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        if r.size and (r.min() < 0 or r.max() >= B * Hq * Sq):
            raise ValueError("oracle: row id out of range")
        o = np.zeros((r.size, D), np.float64)
        lse = np.zeros((r.size,), np.float64)
        rp, n = _ptr(r, _i64p), r.size
    rc = lib.oracle_attn_fp64(_ptr(q), _ptr(k), _ptr(v), B, Sq, Skv, Hq, Hkv, D,
                              float(scale), int(bool(causal)),
                              _ptr(off) if off is not None else None, rp, n,
                              _ptr(o), _ptr(lse))
    if rc != 0:
        raise RuntimeError("oracle_attn_fp64 failed")
    return o, lse


def combine_fp64(o_part, lse_part):
    """Recombine normalised partials over disjoint key ranges.

    o_part: [rows, n, D]; lse_part: [rows, n]. Returns (o [rows,D], lse [rows]).
    """
    op = _f64(o_part)
    lp = _f64(lse_part)
    rows, n, D = op.shape
    if lp.shape != (rows, n):
        raise ValueError("oracle: lse_part must be [rows, n]")
    o = np.zeros((rows, D), np.float64)
    lse = np.zeros((rows,), np.float64)
    load().oracle_combine_fp64(_ptr(op), _ptr(lp), rows, n, D, _ptr(o), _ptr(lse))
    return o, lse


def num_threads():
    return int(load().oracle_num_threads())
