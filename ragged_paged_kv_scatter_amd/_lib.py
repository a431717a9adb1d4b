"""ctypes view of librpa.so (the C ABI declared in include/rpa.h).

Only argument marshalling lives here.  There is no fallback: if the library
is missing or fails to load, every call raises."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librpa.so")

RPA_F32, RPA_BF16, RPA_FP8_E4M3 = 0, 1, 2
STATUS = {0: "RPA_OK", 1: "RPA_ERR_NULL_POINTER", 2: "RPA_ERR_INVALID_SHAPE",
          3: "RPA_ERR_UNSUPPORTED", 4: "RPA_ERR_INVALID_OPTION", 5: "RPA_ERR_WORKSPACE",
          6: "RPA_ERR_HIP"}
EXPORTS = ("rpa_update_kv_cache", "rpa_workspace_bytes", "rpa_forward", "rpa_error_string",
           "rpa_profile_enable", "rpa_profile_read", "rpa_slot_mapping",
           "rpa_reshape_and_cache", "rpa_copy_blocks", "rpa_swap_blocks",
           "rpa_validate_metadata", "rpa_trace_format", "rpa_forward_noalloc")
NOALLOC_SCRATCH_BYTES = 32 << 20      # RPA_NOALLOC_SCRATCH_BYTES in include/rpa.h


class RpaDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "total_tokens", "max_num_seqs", "pages_per_seq", "num_pages", "page_size",
        "num_q_heads", "num_kv_heads", "head_dim", "head_dim_padded", "q_dtype",
        "kv_in_dtype", "cache_dtype")]


class RpaOptions(ctypes.Structure):
    _fields_ = [
        ("softmax_scale", ctypes.c_float),
        ("sliding_window", ctypes.c_int32),
        ("logits_soft_cap", ctypes.c_float),
        ("q_scale", ctypes.c_float),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("chunk_prefill_size", ctypes.c_int32),
        ("num_kv_pages_per_block", ctypes.c_int32),
        ("num_queries_per_block", ctypes.c_int32),
        ("lds_limit_bytes", ctypes.c_int64),
    ]


class RpaKernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double)]


_lib = None


class RpaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def load():
    """Load librpa.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m ragged_paged_kv_scatter_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I32P = ctypes.POINTER(ctypes.c_int32)
    lib.rpa_update_kv_cache.argtypes = [ctypes.POINTER(RpaDesc), P, P, P, P, P, P, P,
                                        ctypes.c_float, ctypes.c_float, P]
    lib.rpa_update_kv_cache.restype = ctypes.c_int
    lib.rpa_workspace_bytes.argtypes = [ctypes.POINTER(RpaDesc), ctypes.POINTER(RpaOptions),
                                        ctypes.POINTER(ctypes.c_size_t)]
    lib.rpa_workspace_bytes.restype = ctypes.c_int
    lib.rpa_forward.argtypes = [ctypes.POINTER(RpaDesc), ctypes.POINTER(RpaOptions), P, P, P, P,
                                P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.rpa_forward.restype = ctypes.c_int
    lib.rpa_error_string.argtypes = [ctypes.c_int]
    lib.rpa_error_string.restype = ctypes.c_char_p
    lib.rpa_profile_enable.argtypes = [ctypes.c_int]
    lib.rpa_profile_enable.restype = ctypes.c_int
    lib.rpa_profile_read.argtypes = [ctypes.POINTER(RpaKernelStat), ctypes.c_int]
    lib.rpa_profile_read.restype = ctypes.c_int
    lib.rpa_slot_mapping.argtypes = [ctypes.POINTER(RpaDesc), P, P, P, P, P, P]
    lib.rpa_slot_mapping.restype = ctypes.c_int
    lib.rpa_reshape_and_cache.argtypes = [ctypes.POINTER(RpaDesc), P, P, P, P, P,
                                          ctypes.c_float, ctypes.c_float, P]
    lib.rpa_reshape_and_cache.restype = ctypes.c_int
    PP = ctypes.POINTER(ctypes.c_void_p)
    lib.rpa_copy_blocks.argtypes = [PP, PP, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, P,
                                    ctypes.c_int32, P]
    lib.rpa_copy_blocks.restype = ctypes.c_int
    lib.rpa_swap_blocks.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P,
                                    ctypes.c_int32, P]
    lib.rpa_swap_blocks.restype = ctypes.c_int
    lib.rpa_validate_metadata.argtypes = [ctypes.POINTER(RpaDesc), P, P, P, P, P, P, P]
    lib.rpa_validate_metadata.restype = ctypes.c_int
    lib.rpa_trace_format.argtypes = [ctypes.POINTER(RpaDesc), ctypes.POINTER(RpaOptions),
                                     ctypes.c_int, ctypes.c_char_p, ctypes.c_size_t,
                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.rpa_trace_format.restype = ctypes.c_int
    lib.rpa_forward_noalloc.argtypes = [ctypes.POINTER(RpaDesc), ctypes.POINTER(RpaOptions), P,
                                        P, P, P, P, P, P, P, P, P, P]
    lib.rpa_forward_noalloc.restype = ctypes.c_int
    del I32P
    _lib = lib
    return lib


def check(code):
    if code != 0:
        raise RpaError(code, load().rpa_error_string(code).decode())
