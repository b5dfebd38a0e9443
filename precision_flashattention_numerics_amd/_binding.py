"""ctypes binding of libpasa_attn.so: argument marshalling only.

Every step of the attention computation runs in the HIP kernels behind the C
ABI (include/pasa_attn.h).  PyTorch provides device memory and the current HIP
stream.  If the library has not been built this module raises at import: there
is no fallback path.
"""
import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime our library then shares)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpasa_attn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with "
        "`python -m precision_flashattention_numerics_amd.build` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

_lib.pasa_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp]
_lib.pasa_attn_fwd.restype = _i
_lib.pasa_naive_attn_fwd.argtypes = _lib.pasa_attn_fwd.argtypes
_lib.pasa_naive_attn_fwd.restype = _i
_lib.pasa_attn_fwd_strict.argtypes = _lib.pasa_attn_fwd.argtypes
_lib.pasa_attn_fwd_strict.restype = _i
_lib.pasa_attn_fwd_fp8.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _f, _f, _i,
                                   _vp]
_lib.pasa_attn_fwd_fp8.restype = _i
_lib.pasa_attn_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]
_lib.pasa_attn_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]
_lib.pasa_attn_decode_noalloc.restype = _i
_lib.pasa_attn_decode_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                        _i, _f, _i, _vp, _sz, _vp]
_lib.pasa_attn_decode_paged.restype = _i
_lib.pasa_attn_decode.restype = _i
_lib.pasa_attn_decode_splits.argtypes = [_i, _i, _i, _i, _i]
_lib.pasa_attn_decode_splits.restype = _i
_lib.pasa_attn_fwd_key_split.argtypes = [_i, _i, _i, _i, _i, _i, _i]
_lib.pasa_attn_fwd_key_split.restype = _i
_lib.pasa_attn_decode_workspace_bytes.argtypes = [_i, _i, _i, _i]
_lib.pasa_attn_decode_workspace_bytes.restype = _sz
_lib.pasa_attn_decode_combine.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]
_lib.pasa_attn_decode_combine.restype = _i
_lib.pasa_status_string.argtypes = [_i]
_lib.pasa_status_string.restype = ctypes.c_char_p

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4


class PasaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def raw():
    """The ctypes library object (for callers that marshal pointers themselves)."""
    return _lib


def status_string(status: int) -> str:
    return _lib.pasa_status_string(int(status)).decode()


def _check(rc, where):
    if rc != OK:
        raise PasaError(rc, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _want(t, name, dtype=torch.float16):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor")


def _want_shape(t, name, shape, dtype):
    """A caller-supplied output buffer: the library writes through its pointer,
    so dtype, device, layout and shape are checked here."""
    _want(t, name, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _want_workspace(ws, device):
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    if ws.device != device:
        raise ValueError("workspace must be on q's device")


def _fwd(fn, where, q, k, v, causal, scale, out, lse, return_lse, stream):
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _want(t, nm)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,Sq,Hq,D]; k and v [B,Skv,Hkv,D]")
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    if Bk != B or Dk != D or Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("inconsistent q/k/v shapes")
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _want_shape(out, "out", q.shape, torch.float16)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _want_shape(lse, "lse", (B, Hq, Sq), torch.float32)
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Sq, Skv, Hq, Hq // Hkv, D,
            float(scale), int(bool(causal)), _stream(stream))
    _check(rc, where)
    return (out, lse) if return_lse or lse is not None else out


def attn_fwd(q, k, v, causal=False, scale=None, out=None, lse=None, return_lse=True,
             stream=None):
    """PASA forward. q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D] fp16 -> (o, lse)."""
    return _fwd(_lib.pasa_attn_fwd, "pasa_attn_fwd", q, k, v, causal, scale, out, lse,
                return_lse, stream)


def attn_fwd_strict(q, k, v, causal=False, scale=None, out=None, lse=None, return_lse=True,
                    stream=None):
    """PASA forward with fp16 running maximum and offset as well; same interface."""
    return _fwd(_lib.pasa_attn_fwd_strict, "pasa_attn_fwd_strict", q, k, v, causal, scale, out,
                lse, return_lse, stream)


def attn_fwd_fp8(q8, k8, v, q_scale, k_scale, causal=False, scale=None, out=None, lse=None,
                 return_lse=True, stream=None):
    """PASA forward with e4m3 queries and keys (torch.float8_e4m3fn, one
    dequantisation scale each) and fp16 values -> (o fp16, lse)."""
    _want(q8, "q8", torch.float8_e4m3fn)
    _want(k8, "k8", torch.float8_e4m3fn)
    _want(v, "v")
    if q8.dim() != 4 or k8.dim() != 4 or v.shape != k8.shape:
        raise ValueError("q8 [B,Sq,Hq,D], k8 and v [B,Skv,Hkv,D]")
    B, Sq, Hq, D = q8.shape
    Bk, Skv, Hkv, Dk = k8.shape
    if Bk != B or Dk != D or Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("inconsistent q/k/v shapes")
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty(q8.shape, dtype=torch.float16, device=q8.device)
    _want_shape(out, "out", q8.shape, torch.float16)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q8.device)
    if lse is not None:
        _want_shape(lse, "lse", (B, Hq, Sq), torch.float32)
    rc = _lib.pasa_attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v), _ptr(out), _ptr(lse), B, Sq, Skv, Hq,
                                Hq // Hkv, D, float(scale), float(q_scale), float(k_scale),
                                int(bool(causal)), _stream(stream))
    _check(rc, "pasa_attn_fwd_fp8")
    return (out, lse) if return_lse or lse is not None else out


def naive_attn_fwd(q, k, v, causal=False, scale=None, out=None, lse=None, return_lse=True,
                   stream=None):
    """Naive fp16 Flash-Attention forward (overflow exhibit); same interface."""
    return _fwd(_lib.pasa_naive_attn_fwd, "pasa_naive_attn_fwd", q, k, v, causal, scale, out,
                lse, return_lse, stream)


def fwd_key_split(batch, seqlen_q, seqlen_kv, num_heads_q, head_dim, causal, num_cus=256) -> int:
    """1 if the prefill runs this problem as key-split items on num_cus compute
    units, 0 if not, a negative status for invalid arguments."""
    return int(_lib.pasa_attn_fwd_key_split(batch, seqlen_q, seqlen_kv, num_heads_q, head_dim,
                                            int(causal), num_cus))


def decode_splits(batch, seqlen_kv, num_heads_q, gqa_group, head_dim) -> int:
    return int(_lib.pasa_attn_decode_splits(batch, seqlen_kv, num_heads_q, gqa_group, head_dim))


def decode_workspace_bytes(batch, num_heads_q, head_dim, num_splits) -> int:
    return int(_lib.pasa_attn_decode_workspace_bytes(batch, num_heads_q, head_dim, num_splits))


def decode_workspace(q, k_cache, num_splits=0):
    """Allocate a workspace (uint8 tensor, 256-byte aligned) for attn_decode."""
    B, _, Hq, D = q.shape
    _, Skv, Hkv, _ = k_cache.shape
    n = num_splits or decode_splits(B, Skv, Hq, Hq // Hkv, D)
    nbytes = decode_workspace_bytes(B, Hq, D, n)   # the library may use fewer splits
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=q.device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + nbytes], n


def attn_decode(q, k_cache, v_cache, num_splits=0, scale=None, out=None, lse=None,
                workspace=None, return_lse=True, stream=None):
    """Split-KV PASA decode. q [B,1,Hq,D]; caches [B,Skv,Hkv,D] -> (o, lse [B,Hq])."""
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _want(t, nm)
    if q.dim() != 4 or q.shape[1] != 1 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B,1,Hq,D]; caches [B,Skv,Hkv,D]")
    B, _, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k_cache.shape
    if Bk != B or Dk != D or Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("inconsistent q/cache shapes")
    if scale is None:
        scale = D ** -0.5
    if workspace is None:
        workspace, _ = decode_workspace(q, k_cache, num_splits)
    _want_workspace(workspace, q.device)
    if out is None:
        out = torch.empty_like(q)
    _want_shape(out, "out", q.shape, torch.float16)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _want_shape(lse, "lse", (B, Hq), torch.float32)
    rc = _lib.pasa_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), B,
                               Skv, Hq, Hq // Hkv, D, float(scale), int(num_splits),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(stream))
    _check(rc, "pasa_attn_decode")
    return (out, lse) if return_lse or lse is not None else out


def attn_decode_noalloc(q, k_cache, v_cache, out, lse=None, num_splits=0, scale=None,
                        stream=None):
    """attn_decode with the partials in the library's static per-GPU scratch
    area (no device allocation by the library; out and lse are the caller's).
    Calls that overlap in time on one GPU race for that area."""
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _want(t, nm)
    if q.dim() != 4 or q.shape[1] != 1 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B,1,Hq,D]; caches [B,Skv,Hkv,D]")
    B, _, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k_cache.shape
    if Bk != B or Dk != D or Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("inconsistent q/cache shapes")
    if scale is None:
        scale = D ** -0.5
    _want_shape(out, "out", q.shape, torch.float16)
    if lse is not None:
        _want_shape(lse, "lse", (B, Hq), torch.float32)
    rc = _lib.pasa_attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                                       B, Skv, Hq, Hq // Hkv, D, float(scale), int(num_splits),
                                       _stream(stream))
    _check(rc, "pasa_attn_decode_noalloc")
    return out, lse


def attn_decode_paged(q, k_pages, v_pages, block_table, seq_lens, num_splits=0, scale=None,
                      out=None, lse=None, workspace=None, return_lse=True, stream=None):
    """Split-KV PASA decode over a paged cache.  q [B,1,Hq,D]; pages
    [num_pages, page_size, Hkv, D]; block_table int32 [B, max_pages];
    seq_lens int32 [B] -> (o, lse [B,Hq])."""
    for t, nm in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _want(t, nm)
    _want(block_table, "block_table", torch.int32)
    _want(seq_lens, "seq_lens", torch.int32)
    if q.dim() != 4 or q.shape[1] != 1 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("q must be [B,1,Hq,D]; pages [num_pages,page_size,Hkv,D]")
    B, _, Hq, D = q.shape
    num_pages, page_size, Hkv, Dk = k_pages.shape
    if Dk != D or Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("inconsistent q/page shapes")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_pages], seq_lens [B]")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = D ** -0.5
    if workspace is None:
        n = num_splits or decode_splits(B, page_size * max_pages, Hq, Hq // Hkv, D)
        nbytes = decode_workspace_bytes(B, Hq, D, n)
        ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=q.device)
        off = (-ws.data_ptr()) % 256
        workspace = ws[off:off + nbytes]
    _want_workspace(workspace, q.device)
    if out is None:
        out = torch.empty_like(q)
    _want_shape(out, "out", q.shape, torch.float16)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _want_shape(lse, "lse", (B, Hq), torch.float32)
    rc = _lib.pasa_attn_decode_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens), _ptr(out),
        _ptr(lse), B, Hq, Hq // Hkv, D, page_size, num_pages, max_pages, float(scale),
        int(num_splits), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(rc, "pasa_attn_decode_paged")
    return (out, lse) if return_lse or lse is not None else out


def attn_decode_combine(o_part, lse_part, out=None, lse=None, stream=None):
    """Combine fp32 partials o_part [B,Hq,n,D], lse_part [B,Hq,n] -> (o [B,1,Hq,D], lse)."""
    _want(o_part, "o_part", torch.float32)
    _want(lse_part, "lse_part", torch.float32)
    B, Hq, n, D = o_part.shape
    if tuple(lse_part.shape) != (B, Hq, n):
        raise ValueError("lse_part must be [B,Hq,n]")
    if out is None:
        out = torch.empty((B, 1, Hq, D), dtype=torch.float16, device=o_part.device)
    _want_shape(out, "out", (B, 1, Hq, D), torch.float16)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=o_part.device)
    _want_shape(lse, "lse", (B, Hq), torch.float32)
    rc = _lib.pasa_attn_decode_combine(_ptr(o_part), _ptr(lse_part), _ptr(out), _ptr(lse), B, Hq,
                                       D, n, _stream(stream))
    _check(rc, "pasa_attn_decode_combine")
    return out, lse
