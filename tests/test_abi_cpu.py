"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/pasa_attn.h declares, and rejects invalid arguments
with the documented status before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pasa_attn.h")
LIB = os.path.join(ROOT, "precision_flashattention_numerics_amd", "libpasa_attn.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pasa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import torch  # noqa: F401  share torch's HIP runtime, as the binding does
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    names = declared()
    for fn in ("pasa_attn_fwd", "pasa_attn_fwd_strict", "pasa_attn_fwd_fp8", "pasa_naive_attn_fwd",
               "pasa_attn_decode",
               "pasa_attn_decode_paged",
               "pasa_attn_decode_combine", "pasa_attn_decode_workspace_bytes",
               "pasa_attn_decode_splits", "pasa_attn_fwd_key_split", "pasa_status_string"):
        assert fn in names


def test_every_declared_symbol_is_exported(lib):
    for fn in declared():
        assert hasattr(lib, fn), fn


P = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def _fwd(lib, name, q=P, k=P, v=P, o=P, B=1, Sq=8, Skv=8, Hq=2, g=1, D=64, scale=0.125, causal=0):
    f = getattr(lib, name)
    f.restype = ctypes.c_int
    return f(q, k, v, o, None, B, Sq, Skv, Hq, g, D, ctypes.c_float(scale), causal, None)


@pytest.mark.parametrize("name", ["pasa_attn_fwd", "pasa_attn_fwd_strict", "pasa_naive_attn_fwd"])
def test_fwd_validation(lib, name):
    assert _fwd(lib, name, q=None) == -1
    assert _fwd(lib, name, o=None) == -1
    assert _fwd(lib, name, B=0) == -1
    assert _fwd(lib, name, Sq=0) == -1
    assert _fwd(lib, name, Skv=-3) == -1
    assert _fwd(lib, name, Hq=7, g=2) == -1
    assert _fwd(lib, name, causal=2) == -1
    assert _fwd(lib, name, D=96) == -2
    assert _fwd(lib, name, D=256) == -2
    # one head's K/V slab beyond the 4 GiB a buffer descriptor addresses
    # (65505+ keys are accepted: the running sum is carried per segment)
    assert _fwd(lib, name, Skv=1 << 24, Hq=1, D=128) == -2
    assert _fwd(lib, name, Sq=2 ** 31 - 100) == -2   # rows past the int range of an item
    assert _fwd(lib, name, scale=0.0) == -2
    assert _fwd(lib, name, scale=float("nan")) == -2
    # more 256-row work items than an int counts (the tensors would not fit a GPU)
    assert _fwd(lib, name, B=65535, Sq=1, Skv=1, Hq=65535, g=65535) == -2


# (batch, seqlen, heads, head_dim) of causal prefills timed both ways on one
# MI355X (256 compute units), with the faster item shape: key split or not
CAUSAL_SPLIT_MEASURED = [
    ((1, 4096, 28, 128), 0),    # 148.4 vs 161.0 us with the split
    ((2, 4096, 28, 128), 0),    # 242.3 vs 269.5
    ((1, 8192, 28, 128), 0),    # 438.4 vs 480.2
    ((1, 2048, 32, 128), 1),    # 63.6 vs 49.6
    ((1, 1024, 16, 128), 1),    # 35.5 vs 24.0
    ((1, 8192, 32, 64), 0),     # 326.0 vs 399.8
    ((1, 16384, 6, 64), 0),     # 289.6 vs 305.3
    ((1, 32768, 32, 128), 0),   # 7.53 vs 8.10 ms
]


@pytest.mark.parametrize("shape,split", CAUSAL_SPLIT_MEASURED, ids=lambda x: str(x))
def test_fwd_key_split_picks_the_measured_faster_shape(lib, shape, split):
    B, S, H, D = shape
    assert lib.pasa_attn_fwd_key_split(B, S, S, H, D, 1, 256) == split


def test_fwd_key_split_rules_and_errors(lib):
    f = lib.pasa_attn_fwd_key_split
    # non-causal: 360 items of 256 rows on 256 units (two rounds, the second
    # partly idle) against 720 of 128 rows (three half-length rounds)
    assert f(2, 9216, 9216, 5, 64, 0, 256) == 1
    assert f(1, 1024, 1024, 64, 128, 0, 256) == 0    # exactly one full round
    assert f(4, 2048, 2048, 32, 128, 0, 256) == 0
    # causal, more than 8 * units split items: balanced, never split
    assert f(8, 8192, 8192, 32, 128, 1, 256) == 0
    # fewer units: the same problem has more items per unit
    assert f(1, 2048, 2048, 32, 128, 1, 64) == 0
    assert f(0, 64, 64, 1, 128, 0, 256) == -1
    assert f(1, 64, 64, 1, 128, 2, 256) == -1
    assert f(1, 64, 64, 1, 128, 0, 0) == -1
    assert f(1, 64, 64, 1, 128, 0, 65537) == -1
    assert f(1, 64, 64, 1, 96, 0, 256) == -2


def test_decode_validation_and_sizes(lib):
    lib.pasa_attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.pasa_attn_decode.restype = ctypes.c_int
    ws = lib.pasa_attn_decode_workspace_bytes(64, 28, 128, 4)
    rows = 64 * 28 * 4
    assert ws == ((rows * 128 * 4 + 255) // 256) * 256 + ((rows * 4 + 255) // 256) * 256
    assert lib.pasa_attn_decode_workspace_bytes(0, 28, 128, 4) == 0
    assert lib.pasa_attn_decode_splits(64, 8192, 28, 7, 128) == 2   # 512 waves over 256 units
    assert lib.pasa_attn_decode_splits(64, 8192, 28, 7, 64) == 6    # 1536 waves over 256 units
    assert lib.pasa_attn_decode_splits(8, 16384, 32, 4, 64) == 12   # 768 waves over 64 units
    assert lib.pasa_attn_decode_splits(1, 100, 1, 1, 128) == 4      # four 32-key sub-tiles
    assert lib.pasa_attn_decode_splits(1, 20, 1, 1, 64) == 1
    assert lib.pasa_attn_decode_splits(1, 8192, 28, 3, 128) == 0    # 28 % 3 != 0
    assert lib.pasa_attn_decode_splits(1, 8192, 28, 7, 96) == 0     # unsupported head_dim

    def dec(ws_ptr=P, ws_bytes=1 << 30, D=128, n=4, g=7, q=P):
        return lib.pasa_attn_decode(q, P, P, P, None, 64, 8192, 28, g, D, ctypes.c_float(0.08),
                                    n, ws_ptr, ctypes.c_size_t(ws_bytes), None)
    assert dec(q=None) == -1
    assert dec(g=3) == -1
    assert dec(n=-1) == -1
    assert dec(D=80) == -2
    assert dec(ws_ptr=None) == -3
    assert dec(ws_ptr=ctypes.c_void_p(0x1010)) == -3            # not 256-byte aligned
    assert dec(ws_bytes=ws - 1) == -3
    # a combine grid (batch * num_heads_q workgroups) beyond 2^31 - 1
    big = lib.pasa_attn_decode(P, P, P, P, None, 65535, 64, 65535, 65535, 64, ctypes.c_float(0.125),
                               1, P, ctypes.c_size_t(1 << 62), None)
    assert big == -2


def test_combine_validation(lib):
    f = lib.pasa_attn_decode_combine
    f.restype = ctypes.c_int
    assert f(None, P, P, None, 1, 1, 128, 2, None) == -1
    assert f(P, P, P, None, 1, 1, 128, 0, None) == -1
    assert f(P, P, P, None, 1, 1, 48, 2, None) == -2


def test_status_strings(lib):
    lib.pasa_status_string.restype = ctypes.c_char_p
    texts = {lib.pasa_status_string(s) for s in (0, -1, -2, -3, -4)}
    assert len(texts) == 5
    assert lib.pasa_status_string(17) == b"unknown status"


def test_fp8_fwd_validation(lib):
    f = lib.pasa_attn_fwd_fp8
    f.restype = ctypes.c_int

    def call(q=P, k=P, v=P, o=P, B=1, D=64, qs=1.0, ks=1.0, causal=0):
        return f(q, k, v, o, None, B, 8, 8, 2, 1, D, ctypes.c_float(0.125), ctypes.c_float(qs),
                 ctypes.c_float(ks), causal, None)
    assert call(q=None) == -1
    assert call(B=0) == -1
    assert call(D=96) == -2
    assert call(qs=0.0) == -2
    assert call(ks=-1.0) == -2
    assert call(qs=float("inf")) == -2
