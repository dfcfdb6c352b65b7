"""ctypes loader for the in-tree gfx950 library ``libkda.so`` (declarations: include/kda.h).

There is no fallback: if the library is missing or does not load, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda.so")

KDA_LAYOUT = {"BNSD": 0, "BSND": 1, "TND": 2}
KDA_QK_L2NORM = 1
KDA_BETA_SIGMOID = 2
KDA_SCALAR_GATE = 4
KDA_RAW_GATE = 8
NOALLOC_SCRATCH_BYTES = 64 << 20   # KDA_NOALLOC_SCRATCH_BYTES in include/kda.h
KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP = range(5)

EXPORTED = ["kda_chunk_fwd_workspace", "kda_chunk_fwd", "kda_chunk_fwd_timed",
            "kda_num_stages", "kda_stage_name", "kda_chunk_fwd_plan", "kda_status_str",
            "kda_version", "kda_chunk_fwd_plan_kernels", "kda_num_kernel_variants",
            "kda_kernel_variant", "kda_chunk_fwd_noalloc", "kda_chunk_fwd_raw_gate",
            "kda_chunk_fwd_raw_gate_timed"]


class KdaShape(ctypes.Structure):
    """Mirror of ``kda_shape`` in include/kda.h."""
    _fields_ = [("layout", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("n_qk", ctypes.c_int32),
                ("n_v", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("scale", ctypes.c_float), ("flags", ctypes.c_uint32)]


class KdaRawGate(ctypes.Structure):
    """Mirror of ``kda_raw_gate`` in include/kda.h."""
    _fields_ = [("a_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("lower_bound", ctypes.c_float)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkda.so once; raise if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m kimi_delta_attention_chunk_amd.build` "
            "(hipcc --offload-arch=gfx950); there is no CPU fallback")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    S = ctypes.POINTER(KdaShape)
    lib.kda_chunk_fwd_workspace.argtypes = [S, ctypes.POINTER(ctypes.c_size_t)]
    lib.kda_chunk_fwd_workspace.restype = ctypes.c_int
    args = [S, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.kda_chunk_fwd.argtypes = args
    lib.kda_chunk_fwd.restype = ctypes.c_int
    G = ctypes.POINTER(KdaRawGate)
    raw = [S, P, P, P, P, P, G, P, P, P, P, P, ctypes.c_size_t, P]
    lib.kda_chunk_fwd_raw_gate.argtypes = raw
    lib.kda_chunk_fwd_raw_gate.restype = ctypes.c_int
    lib.kda_chunk_fwd_raw_gate_timed.argtypes = raw + [ctypes.POINTER(ctypes.c_void_p),
                                                       ctypes.c_int32]
    lib.kda_chunk_fwd_raw_gate_timed.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [S, P, P, P, P, P, P, P, P, P, P]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_chunk_fwd_timed.argtypes = args + [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]
    lib.kda_chunk_fwd_timed.restype = ctypes.c_int
    lib.kda_num_stages.argtypes = []
    lib.kda_num_stages.restype = ctypes.c_int32
    lib.kda_stage_name.argtypes = [ctypes.c_int32]
    lib.kda_stage_name.restype = ctypes.c_char_p
    lib.kda_chunk_fwd_plan.argtypes = [S, ctypes.POINTER(ctypes.c_uint32),
                                       ctypes.POINTER(ctypes.c_int32)]
    lib.kda_chunk_fwd_plan.restype = ctypes.c_int
    lib.kda_status_str.argtypes = [ctypes.c_int]
    lib.kda_status_str.restype = ctypes.c_char_p
    lib.kda_chunk_fwd_plan_kernels.argtypes = [S, ctypes.c_char_p, ctypes.c_size_t]
    lib.kda_chunk_fwd_plan_kernels.restype = ctypes.c_int
    lib.kda_num_kernel_variants.argtypes = []
    lib.kda_num_kernel_variants.restype = ctypes.c_int32
    lib.kda_kernel_variant.argtypes = [ctypes.c_int32]
    lib.kda_kernel_variant.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_int32
    _lib = lib
    return lib
