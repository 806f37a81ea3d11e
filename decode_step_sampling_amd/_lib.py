"""ctypes loader for libdss.so (the C ABI declared in include/dss.h and the
measurement / test hooks of include/dss_hooks.h).

The library is built in-tree by ``python -m decode_step_sampling_amd.build``.
There is no fallback: if the library is missing, every op raises.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdss.so")

DSS_OK = 0
DSS_ERR_INVALID_ARG = -1
DSS_ERR_WORKSPACE = -2
DSS_ERR_UNSUPPORTED = -3
DSS_ERR_HIP = -4
DSS_ERR_DEVICE = -5

DSS_MAX_VOCAB = 1 << 20

DSS_FLAG_ORDER_JOINT = 0x1
DSS_FLAG_FROM_ZERO = 0x2
DSS_FLAG_STREAMING = 0x4
DSS_FLAG_SINGLE_PIVOT = 0x8

OP_IDS = {
    "sampling_from_probs": 0,
    "top_k_sampling_from_probs": 1,
    "top_p_sampling_from_probs": 2,
    "min_p_sampling_from_probs": 3,
    "top_k_top_p_sampling_from_probs": 4,
    "top_k_renorm_probs": 5,
    "top_p_renorm_probs": 6,
    "top_k_mask_logits": 7,
    "top_k_top_p_sampling_from_logits": 8,
    "softmax": 9,
    "top_k": 10,
    "chain_speculative_sampling": 11,
}

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_U64 = ctypes.c_uint64
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t

_HEAD = [_P, _I32, _I32, _P, _I32, _P, _U64, _P, _U64]     # probs .. offset
_TAIL = [_P, _P, _P, _U32, _P, _SZ, _P]                     # samples .. stream
_RENORM_TAIL = [_P, _U32, _P, _SZ, _P]                      # row_status .. stream

SIGNATURES = {
    "dss_sampling_from_probs": (_HEAD + _TAIL, ctypes.c_int),
    "dss_top_k_sampling_from_probs": (_HEAD + [_P, _I32] + _TAIL, ctypes.c_int),
    "dss_top_p_sampling_from_probs": (_HEAD + [_P, _F32] + _TAIL, ctypes.c_int),
    "dss_min_p_sampling_from_probs": (_HEAD + [_P, _F32] + _TAIL, ctypes.c_int),
    "dss_top_k_top_p_sampling_from_probs": (_HEAD + [_P, _I32, _P, _F32] + _TAIL, ctypes.c_int),
    "dss_top_k_top_p_sampling_from_probs_noalloc": (_HEAD + [_P, _I32, _P, _F32, _P, _P, _P,
                                                             _U32, _P], ctypes.c_int),
    "dss_top_k_renorm_probs": ([_P, _P, _I32, _I32, _P, _I32] + _RENORM_TAIL, ctypes.c_int),
    "dss_top_p_renorm_probs": ([_P, _P, _I32, _I32, _P, _F32] + _RENORM_TAIL, ctypes.c_int),
    "dss_top_k_mask_logits": ([_P, _P, _I32, _I32, _P, _I32] + _RENORM_TAIL, ctypes.c_int),
    "dss_softmax": ([_P, _P, _I32, _I32, _P, _F32] + _RENORM_TAIL, ctypes.c_int),
    "dss_top_k": ([_P, _I32, _I32, _I32, _P, _P, _P, _U32, _P, _SZ, _P], ctypes.c_int),
    "dss_top_k_top_p_sampling_from_logits": (_HEAD + [_P, _I32, _P, _F32, _P, _F32] + _TAIL,
                                             ctypes.c_int),
    "dss_chain_speculative_sampling": ([_P, _P, _P, _I32, _I32, _I32, _P, _U64, _P, _U64,
                                        _P, _P, _P, _U32, _P, _SZ, _P], ctypes.c_int),
    "dss_workspace_size": ([_I32, _I32, _I32, _I32, _U32], ctypes.c_size_t),
    "dss_strerror": ([_I32], ctypes.c_char_p),
    "dss_version": ([], ctypes.c_int32),
    "dss_set_timing_events": ([_P, _P], ctypes.c_int32),
    "dss_stream_read_reference": ([_P, ctypes.c_int64, _P, _P], ctypes.c_int32),
    "dss_set_spin_limit": ([_U64], ctypes.c_int32),
    "dss_set_split_slices": ([_I32], ctypes.c_int32),
    "dss_set_handoff_test": ([_I32], ctypes.c_int32),
    "dss_workspace_status": ([_P, _SZ, _P, _P], ctypes.c_int32),
}

_lib = None


class DssError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def load():
    """Load libdss.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m decode_step_sampling_amd.build` (there is no CPU fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def strerror(status):
    return load().dss_strerror(int(status)).decode()


def check(status, where):
    if status != DSS_OK:
        raise DssError(status, where)
