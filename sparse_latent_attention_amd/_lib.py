"""ctypes loader for libmla_sparse.so (argument marshalling only).

The library is the only compute path: if it is missing or fails to load,
every call raises.  There is no fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_sparse.so")

MLA_OK = 0
MLA_F32 = 0
MLA_BF16 = 1

STATUS_NAMES = {0: "MLA_OK", 1: "MLA_ERR_NULL", 2: "MLA_ERR_SHAPE", 3: "MLA_ERR_ALIGN",
                4: "MLA_ERR_DTYPE", 5: "MLA_ERR_WORKSPACE", 6: "MLA_ERR_INDEX", 7: "MLA_ERR_HIP"}

# name -> (restype, argtypes), one entry per function declared in include/mla_sparse.h
_VP, _I, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "mla_status_string": (ctypes.c_char_p, [_I]),
    "mla_abi_version": (_I, []),
    "mla_sparse_decode_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "mla_sparse_decode": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                               _I, _I, _I, _I, _F, _I, _VP, _SZ, _VP]),
    "mla_sparse_decode_noalloc": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                       _I, _I, _I, _I, _F, _I, _VP]),
    "mla_sparse_prefill_chunk_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "mla_sparse_prefill_chunk": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                      _I, _I, _I, _I, _F, _I, _VP, _SZ, _VP]),
    "mla_cache_append": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _F, _I, _VP]),
    "mla_output_projection_workspace_size": (_SZ, [_I, _I]),
    "mla_output_projection": (_I, [_VP, _VP, _VP, _I, _I, _VP, _SZ, _VP]),
    "mla_sparse_prefill_explicit_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
    "mla_sparse_prefill_explicit": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                         _I, _I, _I, _I, _F, _I, _VP, _SZ, _VP]),
    "mla_wkv_b_dequant": (_I, [_VP, _VP, _VP, _VP, _VP]),
    "mla_validate_indices": (_I, [_VP, _I, _I, _I, _I, _VP, _VP]),
    "mla_read_diagnostics": (_I, [_VP, _I, _I, _I, _VP, _VP]),
    "mla_set_attention_events": (_I, [_VP, _VP]),
}


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")


_lib = None


def load(path: str = LIB_PATH):
    """Load the library once and attach the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m sparse_latent_attention_amd.build` "
            "(the HIP library is the only compute path)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int, where: str) -> None:
    if status != MLA_OK:
        raise MLAError(status, where)
