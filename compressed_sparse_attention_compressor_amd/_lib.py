"""ctypes view of libcsa.so (the C ABI declared in include/csa.h).

Loading the library initialises no GPU; a missing library raises at once:
there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# CSA_LIBRARY names another build of the same ABI (the sanitized host-only
# build that the CPU tests can run against)
LIB_PATH = os.environ.get("CSA_LIBRARY") or os.path.join(_PKG, "libcsa.so")

c_void_p = ctypes.c_void_p
c_int = ctypes.c_int
c_int64 = ctypes.c_int64
c_size_t = ctypes.c_size_t
c_float = ctypes.c_float


class CacheT(ctypes.Structure):
    _fields_ = [
        ("nope", c_void_p),
        ("nscale", c_void_p),
        ("rope", c_void_p),
        ("ikey", c_void_p),
        ("iscale", c_void_p),
        ("n_entries", c_void_p),
        ("B", ctypes.c_int32),
        ("N_cap", ctypes.c_int32),
        ("d_nope", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("d_idx", ctypes.c_int32),
        ("m", ctypes.c_int32),
    ]


class Csa2LayerT(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32),
        ("cand", ctypes.c_int32),
        ("cache", ctypes.POINTER(CacheT)),
        ("q_idx", c_void_p),
        ("w_idx", c_void_p),
        ("H_I", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("pool_block", ctypes.c_int32),
        ("pool_blocks", ctypes.c_int32),
        ("idx_out", c_void_p),
        ("pool_out", c_void_p),
        ("q", c_void_p),
        ("H", ctypes.c_int32),
        ("n_win", ctypes.c_int32),
        ("swa", c_void_p),
        ("swa_pos0", c_void_p),
        ("S", ctypes.c_int32),
        ("softmax_scale", c_float),
        ("out_dtype", ctypes.c_int32),
        ("out", c_void_p),
        ("lse", c_void_p),
        ("rope_base", c_float),
    ]


_SIGS = {
    "csa_compress": (c_int, [c_void_p, c_int64, c_void_p, c_int64, c_int, c_void_p, c_void_p, c_int64, c_int64,
                             ctypes.POINTER(CacheT), c_void_p]),
    "csa_index_topk": (c_int, [ctypes.POINTER(CacheT), c_void_p, c_void_p, c_int, c_void_p, c_int, c_void_p, c_int,
                               c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "csa_index_topk_noalloc": (c_int, [ctypes.POINTER(CacheT), c_void_p, c_void_p, c_int, c_void_p, c_int, c_void_p,
                                       c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "csa_index_scores": (c_int, [ctypes.POINTER(CacheT), c_void_p, c_void_p, c_int, c_void_p, c_int, c_void_p,
                                 c_int, c_void_p, c_size_t, c_void_p]),
    "csa_topk": (c_int, [ctypes.POINTER(CacheT), c_void_p, c_void_p, c_int, c_void_p, c_int, c_int, c_void_p,
                         c_void_p, c_void_p, c_size_t, c_void_p]),
    "csa_compress_index_scores": (c_int, [c_void_p, c_int64, c_void_p, c_int64, c_int, c_void_p, c_void_p, c_int64,
                                          c_int64, ctypes.POINTER(CacheT), c_void_p, c_void_p, c_int, c_void_p, c_int,
                                          c_void_p, c_size_t, c_void_p]),
    "csa_compress_index_topk": (c_int, [c_void_p, c_int64, c_void_p, c_int64, c_int, c_void_p, c_void_p, c_int64,
                                        c_int64, ctypes.POINTER(CacheT), c_void_p, c_void_p, c_int, c_void_p, c_int,
                                        c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "csa_index_pool": (c_int, [ctypes.POINTER(CacheT), c_void_p, c_void_p, c_int, c_int, c_int, c_void_p, c_void_p,
                               c_size_t, c_void_p]),
    "csa_sparse_attn": (c_int, [ctypes.POINTER(CacheT), c_void_p, c_int, c_void_p, c_int, c_void_p, c_int, c_void_p,
                                c_void_p, c_int, c_int, c_float, c_float, c_int, c_void_p, c_void_p, c_void_p,
                                c_size_t, c_void_p]),
    "hca_dense_attn": (c_int, [ctypes.POINTER(CacheT), c_void_p, c_int, c_void_p, c_int, c_void_p, c_void_p, c_int,
                               c_int, c_float, c_float, c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "csa2_layer_stack": (c_int, [ctypes.POINTER(Csa2LayerT), c_int, c_void_p, c_int, c_void_p, c_size_t, c_void_p]),
    "csa2_stack_workspace_bytes": (c_size_t, [ctypes.POINTER(Csa2LayerT), c_int, c_int]),
    "csa_swa_encode": (c_int, [c_void_p, c_int64, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p]),
    "csa_sparse_attn_w8": (c_int, [ctypes.POINTER(CacheT), c_void_p, c_int, c_void_p, c_int, c_void_p, c_int,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_float, c_float, c_int,
                                   c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "hca_dense_attn_w8": (c_int, [ctypes.POINTER(CacheT), c_void_p, c_int, c_void_p, c_int, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_int, c_int, c_float, c_float, c_int, c_void_p, c_void_p,
                                  c_void_p, c_size_t, c_void_p]),
    "csa_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "csa_status_str": (ctypes.c_char_p, [c_int]),
    "csa_compress_hidden": (c_int, [c_void_p, c_int64, c_int, c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_int64,
                                    c_int64, ctypes.POINTER(CacheT), c_void_p, c_size_t, c_void_p]),
    "csa_compress_hidden_ws_bytes": (c_size_t, [c_int, c_int64, c_int, c_int]),
    "csa_version": (c_int, []),
    "csa_last_hip_error": (c_int, []),
    "csa_read_device_flags": (c_int, [c_void_p, ctypes.POINTER(ctypes.c_uint32)]),
}

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m compressed_sparse_attention_compressor_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class CsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        L = lib()
        msg = L.csa_status_str(status).decode()
        if status == -6:
            msg += f" (hipError {L.csa_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")
        self.status = status


def check(status: int, where: str) -> None:
    if status != 0:
        raise CsaError(status, where)
