"""ctypes view of libkvq.so (the C ABI declared in include/kvq.h).

Loading fails loudly when the library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK, KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_ENOSPACE, KVQ_EHIP = range(5)
STATUS_NAMES = {0: "KVQ_OK", 1: "KVQ_EINVAL", 2: "KVQ_EUNSUPPORTED", 3: "KVQ_ENOSPACE", 4: "KVQ_EHIP"}
KVQ_INT8_SYM, KVQ_INT4_ASYM, KVQ_INT2_ASYM, KVQ_INT8_CHANNEL, KVQ_FP8_E4M3, KVQ_INT4_INLINE = 0, 1, 2, 3, 4, 5
KVQ_OUT_F32, KVQ_OUT_BF16 = 0, 1


class CacheDesc(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("rot_signs", ctypes.c_void_p),
                ("channel_scales", ctypes.c_void_p)]


class DecodeOptions(ctypes.Structure):
    _fields_ = [("num_workgroups", ctypes.c_int32)]


class Layout(ctypes.Structure):
    _fields_ = [("code_bytes", ctypes.c_uint64), ("meta_bytes", ctypes.c_uint64),
                ("row_code_bytes", ctypes.c_uint32), ("row_meta_floats", ctypes.c_uint32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_DESC = ctypes.POINTER(CacheDesc)
_OPT = ctypes.POINTER(DecodeOptions)

# name -> (restype, argtypes); the symbols include/kvq.h declares
SIGNATURES = {
    "kvq_query_layout": (_I32, [_DESC, ctypes.POINTER(Layout)]),
    "kvq_reshape_and_cache": (_I32, [_DESC, _P, _P, _I64, _I64, _P, _P, _I32, _P, _P, _P, _P, _P]),
    "kvq_calibrate_channel_scales": (_I32, [_DESC, _P, _P, _I64, _I64, _I32, _P, _P]),
    "kvq_decode_workspace_size": (_I32, [_DESC, _I32, _I32, _I32, _OPT, ctypes.POINTER(_SZ)]),
    "kvq_workspace_init": (_I32, [_P, _SZ, _P]),
    "kvq_paged_decode_attention": (_I32, [_DESC, _P, _I32, _P, _I32, _I32, _P, _P, _P, _P, _P, _P,
                                          _I32, _P, _I32, _P, _I32, ctypes.c_float, _OPT, _P, _SZ, _P]),
    "kvq_paged_decode_attention_noalloc": (_I32, [_DESC, _P, _I32, _P, _I32, _I32, _P, _P, _P, _P, _P, _P,
                                                  _I32, _P, _I32, _P, _I32, ctypes.c_float, _P]),
    "kvq_decode_step": (_I32, [_DESC, _P, _I32, _P, _I32, _I32, _P, _P, _I64, _I64, _P, _P, _P, _P, _P, _P,
                               _P, _P, _I32, _P, _I32, _P, _I32, ctypes.c_float, _OPT, _P, _SZ, _P]),
    "kvq_paged_prefill_attention": (_I32, [_DESC, _P, _I32, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P,
                                           _I32, _P, _I32, _P, _I32, ctypes.c_float, _P, _SZ, _P]),
    "kvq_prefill_workspace_size": (_I32, [_DESC, _I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)]),
    "kvq_gather_dequant": (_I32, [_DESC, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _P]),
    "kvq_last_error": (ctypes.c_char_p, []),
    "kvq_version": (_I32, []),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkvq.so once; raise if it is missing (build it with
    ``python -m sub_byte_quantized_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libkvq.so not found at {path}; build it with "
                          "`python -m sub_byte_quantized_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
