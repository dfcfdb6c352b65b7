"""ctypes marshalling for the fp64 KDA oracle (test infrastructure only).

``kda_oracle`` takes the same tensors the GPU entry point takes (bf16 q/k/v/beta, fp32 g and
initial state, int32 cu_seqlens) as numpy arrays or CPU torch tensors and returns fp64 numpy
arrays.  Every arithmetic step is in ``kda_oracle.c``; nothing here computes the method.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "liboracle_kda.so")

LAYOUTS = {"BNSD": 0, "BSND": 1, "TND": 2}
QK_L2NORM = 1
BETA_SIGMOID = 2
SCALAR_GATE = 4      # g holds one value per (token, value head), shaped like beta

_loaded: dict = {}


def build_oracle(out_path: str = LIB, mutant: int = 0, openmp: bool = True) -> str:
    """Compile kda_oracle.c with gcc into a shared library (mutant 0 = the real oracle)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           f"-DKDA_ORACLE_MUTANT={int(mutant)}", SRC, "-o", out_path + ".tmp", "-lm"]
    if openmp:
        cmd.insert(1, "-fopenmp")
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def load_oracle(path: str = LIB) -> ctypes.CDLL:
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        if path != LIB:
            raise FileNotFoundError(path)
        build_oracle(path)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_kda_fwd.argtypes = [I, I, I, I, I, I, I, ctypes.c_double, ctypes.c_uint,
                                   P, P, P, P, P, P, P, I, I, P, P]
    lib.oracle_kda_fwd.restype = I
    lib.oracle_kda_fwd_raw_gate.argtypes = [I, I, I, I, I, I, I, ctypes.c_double, ctypes.c_uint,
                                            P, P, P, P, P, P, ctypes.c_double, P, P, P, I, I,
                                            P, P]
    lib.oracle_kda_fwd_raw_gate.restype = I
    lib.oracle_num_threads.restype = I
    lib.oracle_mutant_id.restype = I
    _loaded[path] = lib
    return lib


def oracle_threads(path: str = LIB) -> int:
    return int(load_oracle(path).oracle_num_threads())


def _bits16(x) -> np.ndarray:
    """bf16 tensor (torch) or uint16/int16 bit array (numpy) -> contiguous uint16 bits."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            if x.dtype != torch.bfloat16:
                raise TypeError(f"expected bfloat16 tensor, got {x.dtype}")
            return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy()
                                        .view(np.uint16))
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    if a.dtype not in (np.uint16, np.int16):
        raise TypeError(f"expected bf16 bits as uint16, got {a.dtype}")
    return np.ascontiguousarray(a.view(np.uint16))


def _arr(x, dtype) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(np.asarray(x))
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def kda_oracle(q, k, v, g, beta, scale: float, initial_state=None, cu_seqlens=None,
               layout: str = "BNSD", flags: int = QK_L2NORM | BETA_SIGMOID,
               dv_range: Optional[tuple] = None, want_final: bool = True,
               lib_path: str = LIB, raw_gate: Optional[tuple] = None):
    """Run the oracle.  Returns (out, final_state) as float64 arrays.

    out has v's shape; entries that the recurrence does not define (rows past a sequence's
    valid length, value channels outside dv_range) are NaN.  final_state is
    [batch, n_v, d_v, d_k] (rows outside dv_range are NaN) or None when want_final is False.
    raw_gate = (A_log [n_v] fp32, dt_bias [n_v, d_k] fp32, lower_bound): g is then the raw bf16
    gate (v's shape), activated by the oracle.
    """
    lib = load_oracle(lib_path)
    qb, kb, vb, bb = _bits16(q), _bits16(k), _bits16(v), _bits16(beta)
    ga = _bits16(g) if raw_gate is not None else _arr(g, np.float32)
    lay = LAYOUTS[layout]
    if layout == "BNSD":
        batch, n_qk, seq_len, d_k = qb.shape
        n_v, d_v = vb.shape[1], vb.shape[3]
    elif layout == "BSND":
        batch, seq_len, n_qk, d_k = qb.shape
        n_v, d_v = vb.shape[2], vb.shape[3]
    else:
        seq_len, n_qk, d_k = qb.shape
        n_v, d_v = vb.shape[1], vb.shape[2]
        if cu_seqlens is None:
            raise ValueError("TND needs cu_seqlens")
        batch = int(np.asarray(cu_seqlens).shape[0]) - 1
    want_g = bb.shape if (int(flags) & SCALAR_GATE) else vb.shape
    if ga.shape != want_g:
        raise ValueError(f"g has shape {ga.shape}, expected {want_g}")
    cu = None if cu_seqlens is None else _arr(cu_seqlens, np.int32)
    init = None if initial_state is None else _arr(initial_state, np.float32)
    lo, hi = (0, d_v) if dv_range is None else (int(dv_range[0]), int(dv_range[1]))
    out = np.full(vb.shape, np.nan, dtype=np.float64)
    fin = np.full((batch, n_v, d_v, d_k), np.nan, dtype=np.float64) if want_final else None

    def ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    if raw_gate is not None:
        a_log = _arr(raw_gate[0], np.float32)
        dt_bias = _arr(raw_gate[1], np.float32)
        if a_log.shape != (n_v,) or dt_bias.shape != (n_v, d_k):
            raise ValueError(f"A_log {a_log.shape} / dt_bias {dt_bias.shape}: expected "
                             f"({n_v},) / ({n_v}, {d_k})")
        rc = lib.oracle_kda_fwd_raw_gate(lay, batch, seq_len, n_qk, n_v, d_k, d_v, float(scale),
                                         int(flags), ptr(qb), ptr(kb), ptr(vb), ptr(ga),
                                         ptr(a_log), ptr(dt_bias), float(raw_gate[2]), ptr(bb),
                                         ptr(init), ptr(cu), lo, hi, ptr(out), ptr(fin))
    else:
        rc = lib.oracle_kda_fwd(lay, batch, seq_len, n_qk, n_v, d_k, d_v, float(scale),
                                int(flags), ptr(qb), ptr(kb), ptr(vb), ptr(ga), ptr(bb),
                                ptr(init), ptr(cu), lo, hi, ptr(out), ptr(fin))
    if rc != 0:
        raise ValueError(f"oracle_kda_fwd rejected its arguments (code {rc})")
    return out, fin
