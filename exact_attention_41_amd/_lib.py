"""ctypes loader for libfa.so and the raw C signatures declared in include/fa.h."""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK = 0
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_INVALID_ARG", 2: "FA_ERR_UNSUPPORTED",
                3: "FA_ERR_WORKSPACE", 4: "FA_ERR_HIP"}

EXPORTED = ("fa_status_str", "fa_fwd", "fa_fwd_f32", "fa_bwd_workspace_size", "fa_bwd",
            "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq", "fa_fwd_gqa",
            "fa_bwd_gqa_workspace_size", "fa_bwd_gqa", "fa_decode_workspace_size", "fa_decode",
            "fa_fwd_rect", "fa_fwd_fp8", "fa_bwd_rect_workspace_size", "fa_bwd_rect",
            "fa_clock_probe", "fa_decode_noalloc", "fa_fwd_train", "fa_bwd_train")

_lock = threading.Lock()
_lib = None


class LibraryMissing(RuntimeError):
    pass


def load() -> ctypes.CDLL:
    """Load libfa.so once; raise loudly if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(
                f"{LIB_PATH} is not built; run `python -m exact_attention_41_amd.build` "
                "(or __graft_entry__.build()). There is no fallback path.")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.fa_status_str.argtypes = [i]
        lib.fa_status_str.restype = ctypes.c_char_p
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
        lib.fa_fwd.restype = i
        lib.fa_fwd_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
        lib.fa_fwd_f32.restype = i
        lib.fa_bwd_workspace_size.argtypes = [i, i, i, i]
        lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
        lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                               i, i, i, i, i, f, vp]
        lib.fa_bwd.restype = i
        lib.fa_bwd_preprocess.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                          i, i, i, i, vp]
        lib.fa_bwd_preprocess.restype = i
        lib.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp,
                                    i, i, i, i, i, f, vp]
        lib.fa_bwd_dkdv.restype = i
        lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp,
                                  i, i, i, i, i, f, i, vp]
        lib.fa_bwd_dq.restype = i
        lib.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
        lib.fa_fwd_gqa.restype = i
        lib.fa_bwd_gqa_workspace_size.argtypes = [i, i, i, i, i]
        lib.fa_bwd_gqa_workspace_size.restype = ctypes.c_size_t
        lib.fa_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                   i, i, i, i, i, i, f, vp]
        lib.fa_bwd_gqa.restype = i
        lib.fa_bwd_rect_workspace_size.argtypes = [i, i, i, i, i, i]
        lib.fa_bwd_rect_workspace_size.restype = ctypes.c_size_t
        lib.fa_bwd_rect.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                    i, i, i, i, i, i, i, f, vp]
        lib.fa_bwd_rect.restype = i
        lib.fa_bwd_train.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     ctypes.c_size_t, i, i, i, i, i, i, i, f, vp]
        lib.fa_bwd_train.restype = i
        lib.fa_bwd_rect.restype = i
        lib.fa_fwd_rect.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
        lib.fa_fwd_rect.restype = i
        lib.fa_fwd_train.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
        lib.fa_fwd_train.restype = i
        lib.fa_fwd_rect.restype = i
        lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, f, f, f, vp]
        lib.fa_fwd_fp8.restype = i
        lib.fa_decode_workspace_size.argtypes = [i, i, i, i, i, i]
        lib.fa_decode_workspace_size.restype = ctypes.c_size_t
        lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                  i, i, i, i, i, i, i, f, vp]
        lib.fa_decode.restype = i
        lib.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
        lib.fa_decode_noalloc.restype = i
        lib.fa_clock_probe.argtypes = [vp, i, i, vp]
        lib.fa_clock_probe.restype = i
        _lib = lib
        return lib
