"""Python binding of the C ABI in include/kda.h (argument marshalling only).

``kda_chunk_fwd`` / ``kda_chunk_fwd_workspace`` / ``kda_status_str`` mirror the C entry points;
torch provides device memory and the current HIP stream.  Every step of the computation runs
in the gfx950 kernels of libkda.so.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import KdaShape, KDA_LAYOUT, KDA_QK_L2NORM, KDA_BETA_SIGMOID, KDA_SCALAR_GATE, KDA_OK

D = 128


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {kda_status_str(status)}")


def kda_status_str(status: int) -> str:
    return _lib.load().kda_status_str(int(status)).decode()


def kda_num_stages() -> int:
    return int(_lib.load().kda_num_stages())


def kda_stage_name(i: int) -> str:
    return _lib.load().kda_stage_name(int(i)).decode()


def make_shape(layout: str, batch: int, seq_len: int, n_qk: int, n_v: int, scale: float,
               qk_l2norm: bool = True, beta_sigmoid: bool = True, d_k: int = D,
               d_v: int = D, scalar_gate: bool = False) -> KdaShape:
    if layout not in KDA_LAYOUT:
        raise ValueError(f"unknown layout {layout!r}")
    flags = ((KDA_QK_L2NORM if qk_l2norm else 0) | (KDA_BETA_SIGMOID if beta_sigmoid else 0)
             | (KDA_SCALAR_GATE if scalar_gate else 0))
    return KdaShape(KDA_LAYOUT[layout], int(batch), int(seq_len), int(n_qk), int(n_v),
                    int(d_k), int(d_v), float(scale), flags)


def kda_chunk_fwd_workspace(shape: KdaShape) -> int:
    n = ctypes.c_size_t(0)
    st = _lib.load().kda_chunk_fwd_workspace(ctypes.byref(shape), ctypes.byref(n))
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_fwd_workspace")
    return int(n.value)


def kda_chunk_fwd_plan(shape: KdaShape):
    """(stage mask, segments per sequence) of the plan for `shape` (kda_chunk_fwd_plan)."""
    mask = ctypes.c_uint32(0)
    segs = ctypes.c_int32(0)
    st = _lib.load().kda_chunk_fwd_plan(ctypes.byref(shape), ctypes.byref(mask),
                                        ctypes.byref(segs))
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_fwd_plan")
    return int(mask.value), int(segs.value)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def infer_shape(q: torch.Tensor, v: torch.Tensor, layout: str,
                cu_seqlens: Optional[torch.Tensor]):
    """(batch, seq_len, n_qk, n_v) from tensor shapes, as the FlashKDA README lays them out."""
    if layout == "BNSD":
        return q.shape[0], q.shape[2], q.shape[1], v.shape[1]
    if layout == "BSND":
        return q.shape[0], q.shape[1], q.shape[2], v.shape[2]
    if layout == "TND":
        if cu_seqlens is None:
            raise ValueError("TND needs cu_seqlens")
        return cu_seqlens.shape[0] - 1, q.shape[0], q.shape[1], v.shape[1]
    raise ValueError(f"unknown layout {layout!r}")


def kda_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  beta: torch.Tensor, scale: Optional[float] = None,
                  initial_state: Optional[torch.Tensor] = None,
                  cu_seqlens: Optional[torch.Tensor] = None, layout: str = "BNSD",
                  qk_l2norm: bool = True, beta_sigmoid: bool = True,
                  output_final_state: bool = True, out: Optional[torch.Tensor] = None,
                  final_state: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None,
                  stage_events: Optional[Sequence] = None):
    """KDA chunked forward on the current HIP device and stream.  Returns (out, final_state).

    q, k: bf16; v: bf16; g: fp32 natural-log decay, either v's shape (one gate per key
    channel) or beta's shape (one gate per token and value head, shared by every key channel:
    the library's scalar-gate option); beta: bf16 (logits when beta_sigmoid); initial_state:
    fp32 [batch, n_v, 128, 128] or None; cu_seqlens: int32 [batch+1] (required for TND).  All
    tensors must be contiguous and on one GPU.
    """
    batch, seq_len, n_qk, n_v = infer_shape(q, v, layout, cu_seqlens)
    if scale is None:
        scale = q.shape[-1] ** -0.5
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("g", g, torch.float32),
                        ("beta", beta, torch.bfloat16)):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.shape != q.shape:
        raise ValueError("k must match q")
    if g.shape == v.shape:
        scalar_gate = False
    elif g.shape == beta.shape:
        scalar_gate = True
    else:
        raise ValueError("g must have v's shape (per channel) or beta's shape (scalar gate)")
    if initial_state is not None and (initial_state.dtype != torch.float32
                                      or not initial_state.is_contiguous()
                                      or tuple(initial_state.shape) != (batch, n_v, v.shape[-1],
                                                                         q.shape[-1])):
        raise ValueError("initial_state must be contiguous fp32 [batch, n_v, d_v, d_k]")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda):
        raise ValueError("cu_seqlens must be an int32 GPU tensor")
    shape = make_shape(layout, batch, seq_len, n_qk, n_v, scale, qk_l2norm, beta_sigmoid,
                       q.shape[-1], v.shape[-1], scalar_gate)
    lib = _lib.load()
    if out is None:
        out = torch.empty_like(v)
    if final_state is None and output_final_state:
        final_state = torch.empty((batch, n_v, v.shape[-1], q.shape[-1]), dtype=torch.float32,
                                  device=v.device)
    nbytes = kda_chunk_fwd_workspace(shape)
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=v.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(v.device).cuda_stream)
    args = [ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            _ptr(initial_state), _ptr(cu_seqlens), _ptr(out), _ptr(final_state),
            _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
            stream]
    if stage_events is None:
        st = lib.kda_chunk_fwd(*args)
    else:
        evs = (ctypes.c_void_p * len(stage_events))(*[ctypes.c_void_p(e) for e in stage_events])
        st = lib.kda_chunk_fwd_timed(*args, evs, len(stage_events))
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_fwd")
    return out, final_state


def chunk_fwd(inp, **kw):
    """Convenience: run on a workloads.Inputs bundle already on the GPU."""
    return kda_chunk_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.initial_state,
                         inp.cu_seqlens, inp.layout, inp.qk_l2norm, inp.beta_sigmoid, **kw)
