"""ctypes declarations of libfsa.so (the C ABI in include/fsa.h).

Loading fails loudly when the library has not been built; there is no
fallback implementation.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfsa.so")

FSA_OK, FSA_ERR_NULL, FSA_ERR_SHAPE, FSA_ERR_DTYPE = 0, -1, -2, -3
FSA_ERR_WORKSPACE, FSA_ERR_NO_DEVICE, FSA_ERR_LAUNCH, FSA_ERR_ARG = -4, -5, -6, -7
FSA_BF16, FSA_F32 = 0, 1
FSA_SEL_ALL, FSA_SEL_INDEX, FSA_SEL_SEGMENT, FSA_SEL_INDEX_KV, FSA_SEL_INDEX_SCORED = 0, 1, 2, 3, 4
FSA_OP_SELECT_BLOCKS, FSA_OP_PREFILL_ATTN, FSA_OP_TOPK, FSA_OP_DECODE_ATTN = 1, 2, 3, 4
FSA_SEG_GLOBAL, FSA_SEG_FOCUS, FSA_SEG_LOCAL, FSA_SEG_STREAMING = 0, 1, 2, 3
FSA_NOALLOC_SCRATCH_BYTES = 16 << 20
FSA_DBG_BLOCK_INDEX, FSA_DBG_TOKEN_INDEX, FSA_DBG_PAGE_ID, FSA_DBG_SEGMENT = 1, 2, 4, 8
FSA_DBG_UNAVAILABLE = 0x80000000

c_int, c_float, c_double, c_size_t, c_void_p = (ctypes.c_int, ctypes.c_float, ctypes.c_double,
                                                 ctypes.c_size_t, ctypes.c_void_p)
c_int32_p = ctypes.POINTER(ctypes.c_int32)


class PrefillShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "S", "Hq", "Hkv", "D", "T")]


class SelectParams(ctypes.Structure):
    _fields_ = [("p_centroid", c_double), ("p_rescue", c_double),
                ("band_blocks", ctypes.c_int32), ("sink_blocks", ctypes.c_int32)]


class DecodeShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "Hq", "Hkv", "D", "page_size", "num_pages", "max_pages", "max_seq_len")]


class KvSelect(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("idx", c_void_p), ("k", ctypes.c_int32),
                ("segments", c_void_p), ("n_seg", c_void_p), ("max_seg", ctypes.c_int32),
                ("n_split", ctypes.c_int32), ("scores", c_void_p)]


# name -> (restype, argtypes)
SIGNATURES = {
    "block_stats": (c_int, [c_int, c_void_p, ctypes.POINTER(PrefillShape), c_void_p, c_void_p,
                            c_void_p]),
    "select_blocks": (c_int, [c_int, c_void_p, c_void_p, c_void_p, ctypes.POINTER(PrefillShape),
                              ctypes.POINTER(SelectParams), c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "sparse_prefill_attn": (c_int, [c_int, c_void_p, c_void_p, c_void_p,
                                    ctypes.POINTER(PrefillShape), c_void_p, c_void_p, c_float,
                                    c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "topk_indices": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                             ctypes.POINTER(DecodeShape), c_int, c_void_p, c_void_p, c_void_p,
                             c_size_t, c_void_p]),
    "topk_indices_scored": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                    ctypes.POINTER(DecodeShape), c_int, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_size_t, c_void_p]),
    "topk_indices_kv": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                ctypes.POINTER(DecodeShape), c_int, c_void_p, c_void_p, c_void_p,
                                c_size_t, c_void_p]),
    "topk_union_kv": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                              c_void_p]),
    "sparse_decode_attn": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   ctypes.POINTER(DecodeShape), ctypes.POINTER(KvSelect),
                                   c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "sparse_decode_attn_noalloc": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p, ctypes.POINTER(DecodeShape),
                                           ctypes.POINTER(KvSelect), c_float, c_void_p, c_void_p,
                                           c_void_p]),
    "fsa_workspace_size": (c_size_t, [c_int, c_void_p, c_void_p]),
    "fsa_build_segments": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int32_p,
                                   ctypes.POINTER(c_int)]),
    "fsa_build_segments_nb": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                      c_int32_p, ctypes.POINTER(c_int)]),
    "fsa_status_string": (ctypes.c_char_p, [c_int]),
    "fsa_debug_flags": (c_int, [ctypes.POINTER(ctypes.c_uint32), c_int]),
    "fsa_device_check": (c_int, []),
}

_lib = None


def load():
    """Load libfsa.so once; raises RuntimeError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m free_sparse_attention_head_amd.build` "
            "(the HIP library is required; there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class FsaError(RuntimeError):
    def __init__(self, name, status):
        msg = load().fsa_status_string(status).decode()
        super().__init__(f"{name} failed with status {status}: {msg}")
        self.status = status


def check(name, status):
    if status != FSA_OK:
        raise FsaError(name, status)
