"""ctypes loader for libcsa.so (declarations in include/csa.h).

Loading fails loudly when the library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa.so")

F32, BF16, FP8_E4M3_ROWSCALE, MXFP4_E8M0_B32, FP8_BF16_ROPE = 0, 1, 2, 3, 4
STATUS = {0: "CSA_OK", 1: "CSA_ERR_NULL", 2: "CSA_ERR_SHAPE", 3: "CSA_ERR_UNSUPPORTED", 4: "CSA_ERR_WORKSPACE",
          5: "CSA_ERR_LAUNCH"}



class KvPrep(C.Structure):
    """csa_kv_prep: RMSNorm gain / epsilon and RoPE dims / base of the KV preparation."""
    _fields_ = [("gamma", C.c_void_p), ("eps", C.c_float), ("rope_dims", C.c_int), ("rope_base", C.c_float)]


class Pages(C.Structure):
    """csa_pages: block table [B][max_pages] (device int32) and raw tokens per page."""
    _fields_ = [("block_table", C.c_void_p), ("max_pages", C.c_int), ("page_tokens", C.c_int)]


class AppendJob(C.Structure):
    """csa_append_job: one compression problem of csa_decode_append."""
    _fields_ = [("ca", C.c_void_p), ("cb", C.c_void_p), ("za", C.c_void_p), ("zb", C.c_void_p),
                ("bias_a", C.c_void_p), ("bias_b", C.c_void_p), ("c", C.c_int), ("m", C.c_int),
                ("ring_ca", C.c_void_p), ("ring_cb", C.c_void_p), ("ring_za", C.c_void_p), ("ring_zb", C.c_void_p),
                ("out", C.c_void_p), ("out_scale", C.c_void_p), ("out_t", C.c_int), ("prep", C.POINTER(KvPrep))]


class WindowJob(C.Structure):
    """csa_window_job: one sliding-window ring of csa_decode_append."""
    _fields_ = [("row", C.c_void_p), ("ring", C.c_void_p), ("c", C.c_int), ("n_win", C.c_int),
                ("prep", C.POINTER(KvPrep))]


# name -> (restype, argtypes); must match include/csa.h
_P, _I, _I64, _F, _SZ = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_size_t
_PREP = C.POINTER(KvPrep)
_PG = C.POINTER(Pages)
SIGNATURES = {
    "csa_status_string": (C.c_char_p, [_I]),
    "csa_abi_version": (_I, []),
    "csa_compress": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I64, _I64, _I, _I, _P, _P, _I, _I64, _PREP, _P]),
    "csa_compress_pair": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _I, _I64, _PREP, _P, _P, _P, _P, _P, _P, _I, _P,
                               _P, _I, _I64, _PREP, _I, _I, _I, _I64, _I64, _I, _I, _P]),
    "csa_prepare_kv": (_I, [_P, _I64, _P, _P, _I64, _I, _I, _I, _I, _I, _P, _I64, _I64, _PREP, _P]),
    "csa_compress_index": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _P, _I, _I64, _PREP,
                                _P, _P, _P, _P, _P, _P,
                                _I, _I, _I, _I64, _I64, _I,
                                _P, _P, _P, _P, _P, _I, _I, _I64, _P, _I, _P, _I, _P, _P]),
    "csa_index_bound_keys": (_I64, [_I64]),
    "csa_index": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I64, _P, _I, _I, _P, _I, _P, _P]),
    "csa_topk_workspace_bytes": (_SZ, [_I, _I, _I64, _I]),
    "csa_topk": (_I, [_P, _I, _I, _I, _I64, _P, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "csa_topk_compress": (_I, [_P, _I, _I, _I64, _P, _I, _I, _P, _P, _P, _P, _SZ, _P, _P, _P, _P, _P, _P, _I, _I, _I64,
                               _I64, _I, _P, _P, _I, _I64, _PREP, _P]),
    "csa_attend_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "csa_attend": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I64, _P, _I, _F, _F, _F, _I,
                        _I, _I, _P, _I, _P, _SZ, _P]),
    "csa_attend_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I64, _P, _I, _F, _F, _F,
                                _I, _I, _I, _P, _I, _P]),
    "hca_attend_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I64, _I]),
    "hca_attend": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I64, _P, _I, _F, _F, _F, _I, _I, _I,
                        _P, _I, _P, _SZ, _P]),
    "csa_pack_proj_weights": (_I, [_P, _P, _I, _I, _I, _P]),
    "csa_q_up_proj": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _I, _P]),
    "csa_grouped_out_proj": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "csa_decode_append": (_I, [C.POINTER(AppendJob), _I, C.POINTER(WindowJob), _I, _I, _P, _PG, _I, _P]),
    "csa_append_index_paged": (_I, [C.POINTER(AppendJob), C.POINTER(WindowJob), _I, _P, _P, _P, _P, _P, _PG, _I,
                                    _I, _I, _I64, _P, _I, _I, _P, _I, _P, _P]),
    "csa_index_paged": (_I, [_P, _P, _P, _P, _P, _PG, _I, _I, _I, _I64, _P, _I, _I, _P, _I, _P, _P]),
    "csa_attend_paged": (_I, [_P, _P, _P, _PG, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I64, _P, _I, _F, _F, _F,
                              _I, _I, _I, _P, _I, _P, _SZ, _P]),
    "hca_attend_paged": (_I, [_P, _P, _P, _PG, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I64, _P, _I, _F, _F, _F, _I, _I,
                              _I, _P, _I, _P, _SZ, _P]),
}

_lib = None


class CSAError(RuntimeError):
    pass


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libcsa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise CSAError(f"{path} not found: build it with `python -m long_context_sparse_04_amd.build` "
                       "(there is no fallback implementation)")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int, what: str) -> None:
    if status != 0:
        msg = load().csa_status_string(status).decode()
        raise CSAError(f"{what} failed: {msg}")
