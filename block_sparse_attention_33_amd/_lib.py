"""ctypes view of libmsa.so (the C ABI declared in include/msa.h)."""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa.so")

MSA_OK = 0
MSA_ERR_INVALID_ARG = -1
MSA_ERR_UNSUPPORTED = -2
MSA_ERR_WORKSPACE = -3
MSA_ERR_HIP = -4
MSA_ERR_SCRATCH = -5
MSA_DECODE_SCRATCH_BYTES = 16 << 20

MSA_OP_POOL = 0
MSA_OP_INDEX = 1
MSA_OP_PREFILL = 2
MSA_OP_DECODE = 3
MSA_OP_BACKWARD = 4
MSA_OP_PREFILL_VARLEN = 5


class MsaDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


class MsaKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_float)]


_P = ctypes.c_void_p
_DIMS = ctypes.POINTER(MsaDims)
_SIZE_P = ctypes.POINTER(ctypes.c_size_t)

# name -> (restype, argtypes); mirrors include/msa.h
SIGNATURES = {
    "msa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "msa_version": (ctypes.c_int, []),
    "msa_workspace_bytes": (ctypes.c_int, [ctypes.c_int, _DIMS, _SIZE_P, _SIZE_P]),
    "msa_backward_pass_rows": (ctypes.c_int, [_DIMS, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int32)]),
    "msa_plan_check": (ctypes.c_int, [ctypes.c_int, _DIMS, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int32)]),
    "msa_pool_block_keys": (ctypes.c_int, [_DIMS, _P, _P, _P]),
    "msa_index_select": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "msa_prefill": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "msa_prefill_varlen": (ctypes.c_int, [_DIMS, ctypes.POINTER(ctypes.c_int32), _P, _P, _P, _P, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "msa_prefill_switched": (ctypes.c_int, [_DIMS, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                            _P, ctypes.POINTER(ctypes.c_int32)]),
    "msa_decode": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "msa_decode_noalloc": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P]),
    "msa_prefill_lse": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "msa_prefill_backward": (ctypes.c_int, [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                            _P]),
    "msa_prefill_chunk_workspace_bytes": (ctypes.c_int, [_DIMS, ctypes.c_int32, _SIZE_P, _SIZE_P]),
    "msa_prefill_chunk": (ctypes.c_int, [_DIMS, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                         ctypes.c_size_t, _P]),
    "msa_prefill_chunk_varlen": (ctypes.c_int, [_DIMS, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                                _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "msa_decode_init": (ctypes.c_int, [_DIMS, ctypes.c_int32, _P, _P, _P, _P]),
    "msa_decode_step": (ctypes.c_int, [_DIMS, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]),
    "msa_decode_varlen": (ctypes.c_int, [_DIMS, ctypes.POINTER(ctypes.c_int32), _P, _P, _P, _P, _P, _P, _P, _P,
                                         ctypes.c_size_t, _P]),
    "msa_decode_init_varlen": (ctypes.c_int, [_DIMS, ctypes.POINTER(ctypes.c_int32), _P, _P, _P, _P]),
    "msa_decode_step_varlen": (ctypes.c_int, [_DIMS, ctypes.POINTER(ctypes.c_int32), _P, _P, _P, _P, _P, _P, _P, _P,
                                              _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "msa_decode_varlen_device": (ctypes.c_int, [_DIMS] + [_P] * 9 + [ctypes.c_size_t, _P]),
    "msa_decode_step_varlen_device": (ctypes.c_int, [_DIMS] + [_P] * 13 + [ctypes.c_size_t, _P]),
    "msa_probe_mfma_bf16": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _P, ctypes.POINTER(ctypes.c_double), _P]),
    "msa_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "msa_profile_read": (ctypes.c_int, [ctypes.POINTER(MsaKernelTime), ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_int)]),
}

_lib = None


def load():
    """Load libmsa.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -m block_sparse_attention_33_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().msa_status_string(code).decode()
