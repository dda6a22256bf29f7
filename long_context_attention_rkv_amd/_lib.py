"""ctypes declarations of librkv's C ABI (include/rkv.h)."""

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librkv.so")

RKV_OK = 0
RKV_ERR_INVALID_ARG = 1
RKV_ERR_UNSUPPORTED = 2
RKV_ERR_WORKSPACE = 3
RKV_ERR_HIP = 4
RKV_ERR_RANGE = 5

RKV_SCRATCH_BYTES = 32 << 20   # the fixed scratch of rkv_decode_attn_noalloc

RKV_F32 = 0
RKV_BF16 = 1


class RkvStride(C.Structure):
    _fields_ = [("base", C.c_int32), ("double_after", C.c_int64)]


class RkvCache(C.Structure):
    _fields_ = [
        ("dtype", C.c_int32),
        ("n_inst", C.c_int64),
        ("n_kv_heads", C.c_int32),
        ("seq_len", C.c_int64),
        ("head_dim", C.c_int32),
        ("stride", RkvStride),
        ("k", C.c_int32),
        ("bits", C.c_int32),
        ("group", C.c_int32),
        ("n_refs", C.c_int64),
        ("ref_idx", C.c_void_p),
        ("codes_k", C.c_void_p),
        ("codes_v", C.c_void_p),
        ("scales", C.c_void_p),
        ("ref_kv", C.c_void_p),
        ("ref_bits", C.c_int32),
        ("ref_scales", C.c_void_p),
        ("latent", C.c_int32),
        ("latent_seed", C.c_uint64),
    ]


# name -> (restype, argtypes)
SIGNATURES = {
    "rkv_num_refs": (C.c_int64, [C.c_int64, RkvStride]),
    "rkv_ref_position": (C.c_int64, [C.c_int64, RkvStride]),
    "rkv_cache_init": (C.c_int, [C.POINTER(RkvCache)]),
    "rkv_cache_sizes": (C.c_int, [C.POINTER(RkvCache), C.POINTER(C.c_size_t)]),
    "rkv_encode_workspace": (C.c_int, [C.POINTER(RkvCache), C.POINTER(C.c_size_t)]),
    "rkv_encode": (C.c_int, [C.c_void_p, C.c_void_p, C.POINTER(RkvCache), C.c_void_p,
                             C.c_size_t, C.c_void_p]),
    "rkv_select_refs": (C.c_int, [C.c_void_p, C.c_void_p, C.POINTER(RkvCache), C.c_void_p,
                                  C.c_size_t, C.c_void_p]),
    "rkv_quantize": (C.c_int, [C.c_void_p, C.c_void_p, C.POINTER(RkvCache), C.c_void_p,
                               C.c_size_t, C.c_void_p]),
    "rkv_reconstruct": (C.c_int, [C.POINTER(RkvCache), C.c_void_p, C.c_void_p, C.c_void_p]),
    "rkv_decode_workspace": (C.c_int, [C.POINTER(RkvCache), C.c_int32, C.c_int32,
                                       C.POINTER(C.c_size_t)]),
    "rkv_decode_split_hint": (C.c_int, [C.POINTER(RkvCache), C.c_int32, C.POINTER(C.c_int32)]),
    "rkv_decode_attn": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(RkvCache), C.c_float,
                                  C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p]),
    "rkv_decode_attn_tiles": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(RkvCache), C.c_float,
                                        C.c_void_p, C.c_int32, C.c_void_p, C.c_int32,
                                        C.c_void_p, C.c_size_t, C.c_void_p]),
    "rkv_append": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.POINTER(RkvCache), C.c_int64,
                             C.c_void_p, C.c_size_t, C.c_void_p]),
    "rkv_decode_attn_len": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(RkvCache), C.c_int64,
                                      C.c_float, C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t,
                                      C.c_void_p]),
    "rkv_decode_attn_noalloc": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(RkvCache), C.c_float,
                                          C.c_void_p, C.c_int32, C.c_void_p]),
    "rkv_status_string": (C.c_char_p, [C.c_int]),
    "rkv_last_hip_error": (C.c_int32, []),
    "rkv_version": (C.c_int32, []),
}

_lib = None


def load():
    """Load librkv.so from the package directory; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m long_context_attention_rkv_amd.build` (needs hipcc, gfx950)")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
