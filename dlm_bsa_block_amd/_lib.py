"""ctypes view of libbsa.so (the C ABI declared in include/bsa.h)."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_uint8, c_void_p, c_char_p

HERE = os.path.dirname(os.path.abspath(__file__))
# BSA_LIBRARY names another build of the same library (the sanitizer build of sanitize_check.py)
LIB_PATH = os.environ.get("BSA_LIBRARY") or os.path.join(HERE, "libbsa.so")

BSA_OK, BSA_ERR_INVALID, BSA_ERR_UNSUPPORTED, BSA_ERR_CAPACITY, BSA_ERR_WORKSPACE, BSA_ERR_HIP = range(6)
BSA_BF16, BSA_F32 = 0, 1
BSA_ROPE_HALF, BSA_ROPE_INTERLEAVED = 0, 1

# every function the header declares, with its ctypes signature
EXPORTS = {}


class BsaTensor(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("dtype", c_int32), ("B", c_int32), ("H", c_int32), ("L", c_int32),
                ("D", c_int32), ("stride_b", c_int64), ("stride_h", c_int64), ("stride_l", c_int64)]


class BsaSelectParams(ctypes.Structure):
    _fields_ = [("kv_block", c_int32), ("q_block", c_int32), ("q_pos0", c_int32), ("q_len", c_int32),
                ("causal", c_int32), ("pooled_q", c_int32), ("topk", c_int32), ("topk_num", c_int32),
                ("topk_den", c_int32), ("n_first", c_int32), ("n_last", c_int32), ("dual_band", c_int32),
                ("layout", c_int32), ("scale", c_float), ("cap", c_int32)]


class BsaAttnParams(ctypes.Structure):
    _fields_ = [("scale", c_float), ("kv_block", c_int32), ("q_block", c_int32), ("q_pos0", c_int32),
                ("causal", c_int32), ("cap", c_int32)]


class BsaThreshParams(ctypes.Structure):
    _fields_ = [("scale", c_float), ("lambda_", c_float), ("tile", c_int32), ("causal", c_int32)]


_T = POINTER(BsaTensor)
_PF = POINTER(c_float)
_PI = POINTER(c_int32)
_PU8 = POINTER(c_uint8)

_SIGS = {
    "bsa_build_block_summaries": (c_int32, [_T, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "bsa_select_workspace_bytes": (c_size_t, [_T, c_int32, c_int32, POINTER(BsaSelectParams)]),
    "bsa_select_blocks": (c_int32, [_T, c_void_p, c_void_p, c_void_p, c_int32, c_int32, POINTER(BsaSelectParams),
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "bsa_active_rows": (c_int32, [_T, _T, c_float, c_void_p, c_void_p, c_void_p]),
    "bsa_merge_attention_states": (c_int32, [_T, c_void_p, _T, c_void_p, _T, c_void_p, c_void_p]),
    "bsa_block_attention_merge": (c_int32, [_T, _T, _T, c_float, _T, c_void_p, _T, c_void_p, c_void_p]),
    "bsa_attention_workspace_bytes": (c_size_t, [_T, _T, POINTER(BsaAttnParams)]),
    "bsa_window_decode_workspace_bytes": (c_size_t, [_T, _T, POINTER(BsaAttnParams), c_int32]),
    "bsa_select_blocks_refresh": (c_int32, [_T, c_int32, _T, c_void_p, c_void_p, c_int32, c_int32,
                                            POINTER(BsaSelectParams), c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_size_t, c_void_p]),
    "bsa_token_select_workspace_bytes": (c_size_t, [_T, _T, c_int32]),
    "bsa_token_select": (c_int32, [_T, _T, c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_size_t,
                                   c_void_p]),
    "bsa_token_attention_workspace_bytes": (c_size_t, [_T, _T, c_int32]),
    "bsa_token_attention_fwd": (c_int32, [_T, _T, _T, c_void_p, c_void_p, c_int32, c_float, _T, c_void_p, c_void_p,
                                          c_size_t, c_void_p]),
    "bsa_window_decode_fwd": (c_int32, [_T, _T, _T, c_void_p, c_void_p, POINTER(BsaAttnParams), c_int32, c_void_p,
                                        _T, c_void_p, c_void_p, c_size_t, c_void_p]),
    "bsa_sparse_attention_fwd": (c_int32, [_T, _T, _T, c_void_p, c_void_p, POINTER(BsaAttnParams), c_void_p, _T,
                                           c_void_p, c_void_p, c_size_t, c_void_p]),
    "bsa_decode_step_workspace_bytes": (c_size_t, [_T, _T, POINTER(BsaSelectParams)]),
    "bsa_decode_step": (c_int32, [_T, _T, _T, c_void_p, c_void_p, c_int32, POINTER(BsaSelectParams), c_void_p,
                                  c_void_p, _T, c_void_p, c_void_p, c_size_t, c_void_p]),
    "bsa_denoise_step_workspace_bytes": (c_size_t, [_T, _T, POINTER(BsaSelectParams)]),
    "bsa_denoise_step": (c_int32, [_T, _T, c_float, c_void_p, _T, _T, _T, _T, POINTER(BsaSelectParams), _T,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, _T, c_void_p, c_void_p,
                                   c_size_t, c_void_p]),
    "bsa_noalloc_scratch_bytes": (c_size_t, []),
    "bsa_sparse_attention_fwd_noalloc": (c_int32, [_T, _T, _T, c_void_p, c_void_p, POINTER(BsaAttnParams), c_void_p,
                                                   _T, c_void_p, c_void_p]),
    "bsa_threshold_attention_fwd": (c_int32, [_T, _T, _T, POINTER(BsaThreshParams), _T, c_void_p, c_void_p,
                                              c_void_p, c_void_p]),
    "bsa_threshold_decode_workspace_bytes": (c_size_t, [_T, _T, c_int32]),
    "bsa_threshold_decode_fwd": (c_int32, [_T, _T, _T, c_float, c_float, c_int32, _T, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_size_t, c_void_p]),
    "bsa_status_string": (c_char_p, [c_int32]),
    "bsa_last_error": (c_char_p, []),
    "bsa_version": (c_int32, []),
}

_lib = None


class BsaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({_status_name(status)}): {detail}")
        self.status = status


def _status_name(s):
    return ["ok", "invalid", "unsupported", "capacity", "workspace", "hip"][s] if 0 <= s < 6 else "unknown"


def lib() -> ctypes.CDLL:
    """Load libbsa.so (built in-tree).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m dlm_bsa_block_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def check(status: int, where: str):
    if status != BSA_OK:
        raise BsaError(status, where, lib().bsa_last_error().decode())
