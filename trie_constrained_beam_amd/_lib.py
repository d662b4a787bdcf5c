"""ctypes declarations of libtcb.so (include/tcb.h). Argument marshalling only.

The library is loaded from this package directory. If it is missing the import
fails loudly: there is no fallback implementation of any step.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtcb.so")

TCB_OK = 0
ERRORS = {-1: "TCB_E_ARG", -2: "TCB_E_RANGE", -3: "TCB_E_BUDGET", -4: "TCB_E_STATE",
          -5: "TCB_E_WORKSPACE", -6: "TCB_E_HIP", -7: "TCB_E_NONFINITE", -8: "TCB_E_DEVICE"}
TCB_F32, TCB_BF16 = 0, 1
TCB_NORM_CHILDREN, TCB_NORM_LEVEL, TCB_NORM_OPEN = 0, 1, 2
TCB_READ_AUTO, TCB_READ_DENSE, TCB_READ_GATHER = 0, 1, 2
TCB_TABLE_LOGPROB, TCB_TABLE_LOGITS = 0, 1
TCB_SCORE_MAX_K = 512
TCB_SCORE_STATIC_SCRATCH = 64 << 20
TCB_MAX_L = 8
TCB_MAX_WIDTH = 4096
TCB_MASK_AUTO = -1
TCB_TRACE_SLOTS = 16
TCB_TRACE_TILE, TCB_TRACE_MERGE = 1, 2


class TrieInfo(C.Structure):
    _fields_ = [("L", C.c_int32), ("V", C.c_int32), ("mask_depths", C.c_int32),
                ("n_items", C.c_int64), ("n_distinct", C.c_int64),
                ("nodes_per_depth", C.c_int64 * (TCB_MAX_L + 1)),
                ("node_offset", C.c_int64 * (TCB_MAX_L + 2)),
                ("device_bytes", C.c_size_t)]


class BeamsStatus(C.Structure):
    _fields_ = [("steps", C.c_int64), ("active", C.c_int32), ("finished", C.c_int32),
                ("free_slots", C.c_int32), ("free_requests", C.c_int32)]


class TcbError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


P = C.c_void_p
I32, I64 = C.c_int32, C.c_int64
# name -> (restype, argtypes); every name is declared in include/tcb.h
SIGNATURES = {
    "tcb_last_error": (C.c_char_p, []),
    "tcb_version": (C.c_char_p, []),
    "tcb_build_trie": (I32, [P, I64, I32, I32, I32, C.POINTER(P)]),
    "tcb_trie_info": (I32, [P, C.POINTER(TrieInfo)]),
    "tcb_trie_host_arrays": (I32, [P, C.POINTER(P), C.POINTER(P), C.POINTER(P)]),
    "tcb_trie_upload": (I32, [P, P, C.c_size_t, P]),
    "tcb_trie_destroy": (None, [P]),
    "tcb_beams_workspace_bytes": (I32, [P, I32, I32, I32, C.POINTER(C.c_size_t)]),
    "tcb_beams_create": (I32, [P, I32, I32, I32, I32, P, C.c_size_t, P, C.POINTER(P)]),
    "tcb_beam_init": (I32, [P, I32, P, P, P, P]),
    "tcb_beam_step": (I32, [P, P, I64, I32, P]),
    "tcb_beam_step_sampled": (I32, [P, P, I64, I32, C.c_float, C.c_uint64, P]),
    "tcb_beam_step_lmhead": (I32, [P, P, I64, I32, P, P]),
    "tcb_beam_export": (I32, [P, P, P, P, P, P, P, P, P]),
    "tcb_beams_status": (I32, [P, C.POINTER(BeamsStatus)]),
    "tcb_request_level": (I32, [P, I32, C.POINTER(I32)]),
    "tcb_beams_set_validate": (I32, [P, I32]),
    "tcb_beams_set_read_mode": (I32, [P, I32]),
    "tcb_beam_check": (I32, [P, P]),
    "tcb_beam_finalize": (I32, [P, I32, P, P, P, P, P, P]),
    "tcb_beam_finalize_device": (I32, [P, I32, P, P, P, P, P, P]),
    "tcb_beams_set_finish_outputs": (I32, [P, P, P, P, P]),
    "tcb_beams_enable_timing": (I32, [P, I32, I32]),
    "tcb_beams_timing": (I32, [P, C.POINTER(C.c_double), C.POINTER(C.c_double), C.POINTER(C.c_double),
                               C.POINTER(I32)]),
    "tcb_beams_set_trace": (I32, [P, P, I64]),
    "tcb_beams_trace_log": (I32, [P, P, I32, C.POINTER(I32)]),
    "tcb_beams_destroy": (None, [P]),
    "tcb_trie_codes_bytes": (I32, [P, C.POINTER(C.c_size_t)]),
    "tcb_trie_upload_codes": (I32, [P, P, C.c_size_t, P]),
    "tcb_score_workspace_bytes": (I32, [P, I32, C.POINTER(C.c_size_t)]),
    "tcb_score_catalog": (I32, [P, I32, P, I32, P, P, I32, C.c_float, I32, P, P, P, P, P, C.c_size_t, P]),
    "tcb_score_catalog_static": (I32, [P, I32, P, I32, P, P, I32, C.c_float, I32, P, P, P, P, P]),
    "tcb_score_enable_timing": (I32, [I32]),
    "tcb_score_timing": (I32, [C.POINTER(C.c_double), C.POINTER(C.c_double), C.POINTER(I32)]),
}

_lib = None


def lib():
    """The loaded libtcb.so (raises ImportError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m trie_constrained_beam_amd.build` (no fallback exists)")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def check(code):
    if code != TCB_OK:
        raise TcbError(code, lib().tcb_last_error().decode())
    return code
