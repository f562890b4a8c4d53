"""ctypes declarations of libstreambp's C ABI (include/streambp.h)."""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libstreambp.so")

SBP_OK, SBP_ERR_INVALID_ARG, SBP_ERR_UNSUPPORTED, SBP_ERR_WORKSPACE, SBP_ERR_HIP = range(5)
SBP_F32, SBP_BF16 = 0, 1
SBP_MEAN_VALID, SBP_SUM = 0, 1

vp = C.c_void_p
i32 = C.c_int32
i64 = C.c_int64
f32 = C.c_float
sz = C.c_size_t


class LayerDesc(C.Structure):
    _fields_ = [("T", i64), ("d", i64), ("Hq", i32), ("Hkv", i32), ("dh", i32),
                ("F", i64), ("eps", f32), ("dtype", i32), ("rope_theta", f32),
                ("qk_norm", i32)]


LAYER_NAMES = ("g1", "Wq", "Wk", "Wv", "Wo", "g2", "W1", "W3", "W2")
QK_NORM_NAMES = ("qn", "kn")  # per-head norm gains, present only with QK-norm


class LayerWeights(C.Structure):
    _fields_ = [(n, vp) for n in LAYER_NAMES + QK_NORM_NAMES]


class LayerGrads(C.Structure):
    _fields_ = [(n, vp) for n in LAYER_NAMES + QK_NORM_NAMES]


# name -> (restype, argtypes); every symbol include/streambp.h declares
SIGNATURES = {
    "sbp_lmhead_ce_workspace_size": (i32, [i64, i64, i64, i32, i32, C.POINTER(sz)]),
    "sbp_lmhead_ce_fwd_bwd": (i32, [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32,
                                    vp, vp, vp, vp, vp, sz, vp]),
    "sbp_lmhead_ce_workspace_size_grouped": (i32, [i64, i64, i64, i32, i32, i32, C.POINTER(sz)]),
    "sbp_lmhead_logprob_workspace_size": (i32, [i64, i64, i64, i32, i32, C.POINTER(sz)]),
    "sbp_lmhead_logprob_fwd": (i32, [vp, vp, vp, i64, i64, i64, i32, i32, vp, vp, vp, sz, vp]),
    "sbp_attn_bwd_workspace_size": (i32, [i64, i64, i32, i32, i32, i32, i32, C.POINTER(sz)]),
    "sbp_attn_bwd_chunked": (i32, [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, f32, i32,
                                   i32, i32, vp, vp, vp, vp, sz, vp]),
    "sbp_attn_bwd_chunked_noalloc": (i32, [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, f32,
                                           i32, i32, i32, vp, vp, vp, vp]),
    "sbp_attn_bwd_packed_workspace_size": (i32, [i64, i32, i32, i32, i32, i32, C.POINTER(sz)]),
    "sbp_attn_bwd_packed": (i32, [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, f32, i32,
                                  i32, i32, vp, vp, vp, vp, sz, vp]),
    "sbp_layer_bwd_workspace_size": (i32, [C.POINTER(LayerDesc), i32, C.POINTER(sz)]),
    "sbp_layer_bwd": (i32, [C.POINTER(LayerDesc), vp, vp, C.POINTER(LayerWeights), i32, i32,
                            vp, C.POINTER(LayerGrads), vp, sz, vp]),
    "sbp_layer_bwd_packed_workspace_size": (i32, [C.POINTER(LayerDesc), i32, C.POINTER(sz)]),
    "sbp_layer_bwd_packed": (i32, [C.POINTER(LayerDesc), vp, i32, vp, vp, C.POINTER(LayerWeights),
                                   i32, i32, vp, C.POINTER(LayerGrads), vp, sz, vp]),
    "sbp_layer_fwd_workspace_size": (i32, [C.POINTER(LayerDesc), i32, C.POINTER(sz)]),
    "sbp_layer_fwd": (i32, [C.POINTER(LayerDesc), vp, i32, vp, C.POINTER(LayerWeights), i32, vp,
                            vp, sz, vp]),
    "sbp_model_bwd_workspace_size": (i32, [C.POINTER(LayerDesc), i32, i32, i64, i32, i32,
                                           C.POINTER(sz)]),
    "sbp_model_bwd": (i32, [C.POINTER(LayerDesc), i32, vp, i32, C.POINTER(vp),
                            C.POINTER(LayerWeights), vp, vp, i64, vp, vp, i32, i32, i32, i32, vp,
                            vp, vp, C.POINTER(LayerGrads), vp, vp, vp, sz, vp]),
    "sbp_status_string": (C.c_char_p, [i32]),
    "sbp_last_error": (C.c_char_p, []),
    "sbp_version": (i32, []),
    "sbp_profile_begin": (i32, [i32]),
    "sbp_profile_end": (i32, [C.POINTER(i32)]),
    "sbp_profile_entry": (i32, [i32, C.POINTER(C.c_char_p), C.POINTER(i64), C.POINTER(C.c_double),
                                C.POINTER(C.c_double), C.POINTER(C.c_double)]),
}

_lib = None


class StreamBPError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{status_name(status)}: {msg}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load the in-tree libstreambp.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libstreambp is not built ({path} missing); run "
                           "`python -m memory_efficient_exact_amd.build`")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_name(s: int) -> str:
    return load().sbp_status_string(s).decode()


def check(status: int):
    if status != SBP_OK:
        raise StreamBPError(status, load().sbp_last_error().decode())
