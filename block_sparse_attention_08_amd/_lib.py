"""ctypes binding of libsparse_attn.so (argument marshalling only).

The library is loaded on first use, after torch, so that it binds to the HIP
runtime torch already holds.  If the library has not been built the call
raises; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libsparse_attn.so")
PEAKS_PATH = os.path.join(PKG, "lib", "libsa_peaks.so")

SA_DTYPE_F32, SA_DTYPE_BF16 = 0, 1
SA_SELECT_ALPHA, SA_SELECT_DENSITY = 0, 1

STATUS_NAMES = {
    0: "SA_OK", 1: "SA_ERR_NULL", 2: "SA_ERR_SHAPE", 3: "SA_ERR_DTYPE", 4: "SA_ERR_PARAM",
    5: "SA_ERR_ALIGN", 6: "SA_ERR_UNSUPPORTED", 7: "SA_ERR_HIP", 8: "SA_ERR_SCRATCH",
}


class SaDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("select_mode", ctypes.c_int32),
        ("alpha", ctypes.c_double),
        ("density", ctypes.c_double),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("approx", ctypes.c_int32),
    ]


class SaSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("q_bar", "k_bar", "v_sum", "tail", "blk_idx", "blk_cnt")]


class SaBwdSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("lse", "delta", "sel_bits", "col_idx", "col_cnt", "dk_bar",
                                               "dv_bar")]


LIST_FLAGS = {1: "count", 2: "range", 4: "order", 8: "ineligible", 16: "no_diagonal"}


class SparseAttnError(ValueError):
    def __init__(self, status: int, what: str, text: str):
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({text})")
        self.status = status


_lib = None
_peaks = None
_lock = threading.Lock()

_P = ctypes.c_void_p
_SIGS = {
    "sparse_attn_buffer_sizes": [ctypes.POINTER(SaDesc), ctypes.POINTER(SaSizes)],
    "sparse_attn_block_pool": [ctypes.POINTER(SaDesc), _P, _P, _P, _P, _P, _P, _P, _P],
    "sparse_attn_select": [ctypes.POINTER(SaDesc), _P, _P, _P, _P, _P],
    "sparse_attn_route": [ctypes.POINTER(SaDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "sparse_attn_fwd_lse": [ctypes.POINTER(SaDesc)] + [_P] * 11,
    "sparse_attn_bwd_buffer_sizes": [ctypes.POINTER(SaDesc), ctypes.POINTER(SaBwdSizes)],
    "sparse_attn_bwd": [ctypes.POINTER(SaDesc)] + [_P] * 19,
    "sparse_attn_bwd_noalloc": [ctypes.POINTER(SaDesc)] + [_P] * 13,
    "sparse_attn_check_lists": [ctypes.POINTER(SaDesc), _P, _P, _P, _P],
    "sparse_attn_bwd_noalloc_scratch": [ctypes.POINTER(SaDesc), ctypes.POINTER(ctypes.c_size_t),
                                        ctypes.POINTER(ctypes.c_size_t)],
    "sparse_attn_fwd": [ctypes.POINTER(SaDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "sparse_attn_status_string": [ctypes.c_int],
    "sparse_attn_abi_version": [],
}


def lib() -> ctypes.CDLL:
    """The loaded library (loads it on first call)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build the HIP library first "
                    "(python -m block_sparse_attention_08_amd.build)")
            import torch  # noqa: F401  (load torch's HIP runtime first)
            h = ctypes.CDLL(LIB_PATH)
            for name, args in _SIGS.items():
                fn = getattr(h, name)
                fn.argtypes = args
                fn.restype = ctypes.c_int
            h.sparse_attn_status_string.restype = ctypes.c_char_p
            h.sparse_attn_abi_version.restype = ctypes.c_int32
            _lib = h
    return _lib


def peaks_lib() -> ctypes.CDLL:
    """libsa_peaks.so: the achievable-rate kernels (measurement only)."""
    global _peaks
    if _peaks is not None:
        return _peaks
    with _lock:
        if _peaks is None:
            if not os.path.exists(PEAKS_PATH):
                raise RuntimeError(f"{PEAKS_PATH} is missing: build the HIP libraries first")
            import torch  # noqa: F401
            h = ctypes.CDLL(PEAKS_PATH)
            h.sa_peak_read.argtypes = [_P, ctypes.c_size_t, _P, _P, ctypes.POINTER(ctypes.c_size_t)]
            h.sa_peak_read.restype = ctypes.c_int
            h.sa_peak_mfma_bf16.argtypes = [ctypes.c_int, _P, _P, ctypes.POINTER(ctypes.c_double)]
            h.sa_peak_mfma_bf16.restype = ctypes.c_int
            h.sa_peak_mfma_bf16_data.argtypes = [ctypes.c_int, _P, _P, ctypes.POINTER(ctypes.c_double)]
            h.sa_peak_mfma_bf16_data.restype = ctypes.c_int
            h.sa_peak_lds_read.argtypes = [ctypes.c_int, _P, _P, ctypes.POINTER(ctypes.c_double)]
            h.sa_peak_lds_read.restype = ctypes.c_int
            _peaks = h
    return _peaks


def check(status: int, what: str) -> None:
    if status != 0:
        text = lib().sparse_attn_status_string(status).decode()
        raise SparseAttnError(status, what, text)
