"""PASA (online pseudo-average shifting attention) forward pass for AMD MI355X.

The compute path is the HIP library libpasa_attn.so (C ABI in
include/pasa_attn.h); this package is its thin Python binding.  Importing the
package does not load the library; the first use of an entry point does, and
fails loudly if the library has not been built.
"""

_ENTRY = ("attn_fwd", "attn_fwd_strict", "attn_fwd_fp8", "naive_attn_fwd", "attn_decode",
          "attn_decode_noalloc", "attn_decode_paged", "attn_decode_combine",
          "decode_splits", "fwd_key_split", "decode_workspace_bytes", "decode_workspace", "status_string",
          "PasaError", "raw", "LIB_PATH")

__all__ = list(_ENTRY)


def __getattr__(name):
    if name in _ENTRY:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
