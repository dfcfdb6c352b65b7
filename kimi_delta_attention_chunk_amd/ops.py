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
from ._lib import (KdaShape, KdaRawGate, KDA_LAYOUT, KDA_QK_L2NORM, KDA_BETA_SIGMOID,
                   KDA_SCALAR_GATE, KDA_RAW_GATE, KDA_OK)

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
               d_v: int = D, scalar_gate: bool = False, raw_gate: bool = False) -> KdaShape:
    if layout not in KDA_LAYOUT:
        raise ValueError(f"unknown layout {layout!r}")
    flags = ((KDA_QK_L2NORM if qk_l2norm else 0) | (KDA_BETA_SIGMOID if beta_sigmoid else 0)
             | (KDA_SCALAR_GATE if scalar_gate else 0) | (KDA_RAW_GATE if raw_gate else 0))
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


def kda_chunk_fwd_plan_kernels(shape: KdaShape) -> list:
    """Names (with template arguments) of the kernels a call with `shape` launches, in order."""
    buf = ctypes.create_string_buffer(1024)
    st = _lib.load().kda_chunk_fwd_plan_kernels(ctypes.byref(shape), buf, len(buf))
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_fwd_plan_kernels")
    return buf.value.decode().split(";")


def kda_kernel_variants() -> list:
    """Every kernel variant compiled into the library."""
    lib = _lib.load()
    return [lib.kda_kernel_variant(i).decode() for i in range(lib.kda_num_kernel_variants())]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def infer_shape(q: torch.Tensor, v: torch.Tensor, layout: str,
                cu_seqlens: Optional[torch.Tensor]):
    """(batch, seq_len, n_qk, n_v) from tensor shapes, as the FlashKDA README lays them out."""
    want = 3 if layout == "TND" else 4
    if layout not in KDA_LAYOUT:
        raise ValueError(f"unknown layout {layout!r}")
    if q.dim() != want or v.dim() != want:
        raise ValueError(f"{layout}: q and v must have {want} dimensions")
    if layout == "BNSD":
        return q.shape[0], q.shape[2], q.shape[1], v.shape[1]
    if layout == "BSND":
        return q.shape[0], q.shape[1], q.shape[2], v.shape[2]
    if cu_seqlens is None:
        raise ValueError("TND needs cu_seqlens")
    if cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 2:
        raise ValueError("cu_seqlens must be a 1-D tensor of batch + 1 >= 2 entries")
    return cu_seqlens.shape[0] - 1, q.shape[0], q.shape[1], v.shape[1]


def _expected_shapes(layout: str, batch: int, seq_len: int, n_qk: int, n_v: int, d_k: int,
                     d_v: int) -> dict:
    """Shapes of every tensor of a call (FlashKDA README, sections 参数说明 and 返回值说明)."""
    if layout == "BNSD":
        qs, vs, bs = (batch, n_qk, seq_len, d_k), (batch, n_v, seq_len, d_v), (batch, n_v, seq_len)
    elif layout == "BSND":
        qs, vs, bs = (batch, seq_len, n_qk, d_k), (batch, seq_len, n_v, d_v), (batch, seq_len, n_v)
    else:
        qs, vs, bs = (seq_len, n_qk, d_k), (seq_len, n_v, d_v), (seq_len, n_v)
    gs = tuple(vs[:-1]) + (d_k,)
    return dict(q=qs, k=qs, v=vs, g=gs, g_scalar=bs, beta=bs, out=vs,
                state=(batch, n_v, d_v, d_k), cu=(batch + 1,))


def check_tensors(tensors: dict, layout: str):
    """Dtype, shape and contiguity of every tensor of a call, then that all of them live on one
    GPU.  `tensors` maps q, k, v, g, beta, initial_state, cu_seqlens, out, final_state,
    workspace to tensors or None.  Returns (batch, seq_len, n_qk, n_v, scalar_gate).  Raises
    ValueError / TypeError, so that no wrong-sized or host buffer reaches the kernels."""
    q, v, g, beta = tensors["q"], tensors["v"], tensors["g"], tensors["beta"]
    cu = tensors.get("cu_seqlens")
    batch, seq_len, n_qk, n_v = infer_shape(q, v, layout, cu)
    exp = _expected_shapes(layout, batch, seq_len, n_qk, n_v, q.shape[-1], v.shape[-1])
    raw = tensors.get("a_log") is not None or tensors.get("dt_bias") is not None
    dtypes = dict(q=torch.bfloat16, k=torch.bfloat16, v=torch.bfloat16,
                  g=torch.bfloat16 if raw else torch.float32,
                  beta=torch.bfloat16, initial_state=torch.float32, cu_seqlens=torch.int32,
                  out=torch.bfloat16, final_state=torch.float32, a_log=torch.float32,
                  dt_bias=torch.float32)
    scalar_gate = not raw and tuple(g.shape) == exp["g_scalar"]
    shapes = dict(q=exp["q"], k=exp["k"], v=exp["v"], g=exp["g_scalar"] if scalar_gate else exp["g"],
                  beta=exp["beta"], initial_state=exp["state"], cu_seqlens=exp["cu"],
                  out=exp["out"], final_state=exp["state"], a_log=(n_v,),
                  dt_bias=(n_v, q.shape[-1]))
    if raw and (tensors.get("a_log") is None or tensors.get("dt_bias") is None):
        raise ValueError("the raw-gate form needs both A_log and dt_bias")
    for name, t in tensors.items():
        if t is None:
            continue
        if name in dtypes and t.dtype != dtypes[name]:
            raise TypeError(f"{name} must be {dtypes[name]}, got {t.dtype}")
        if name in shapes and tuple(t.shape) != tuple(shapes[name]):
            what = " (or beta's shape for one gate per token and head)" if name == "g" else ""
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shapes[name])}{what}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    devices = {(t.device.type, t.device.index) for t in tensors.values() if t is not None}
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if len(devices) != 1:
        raise ValueError(f"all tensors must be on one GPU, got {sorted(devices)}")
    return batch, seq_len, n_qk, n_v, scalar_gate


def kda_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  beta: torch.Tensor, scale: Optional[float] = None,
                  initial_state: Optional[torch.Tensor] = None,
                  cu_seqlens: Optional[torch.Tensor] = None, layout: str = "BNSD",
                  qk_l2norm: bool = True, beta_sigmoid: bool = True,
                  output_final_state: bool = True, out: Optional[torch.Tensor] = None,
                  final_state: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None,
                  stage_events: Optional[Sequence] = None,
                  gate: Optional[tuple] = None):
    """KDA chunked forward on the current HIP device and stream.  Returns (out, final_state).

    q, k: bf16; v: bf16; g: fp32 natural-log decay, either v's shape (one gate per key
    channel) or beta's shape (one gate per token and value head, shared by every key channel:
    the library's scalar-gate option); beta: bf16 (logits when beta_sigmoid); initial_state:
    fp32 [batch, n_v, d_v, d_k] or None; cu_seqlens: int32 [batch+1] (required for TND).
    gate = (A_log fp32 [n_v], dt_bias fp32 [n_v, d_k], lower_bound): g is then the raw bf16
    gate (v's shape), activated in the kernel (kda_chunk_fwd_raw_gate).  All tensors, including
    caller-supplied out, final_state and workspace, must be contiguous and on one GPU; every
    shape and dtype is checked before anything is launched.
    """
    a_log, dt_bias, lower_bound = gate if gate is not None else (None, None, None)
    tensors = dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=initial_state,
                   cu_seqlens=cu_seqlens, out=out, final_state=final_state, workspace=workspace,
                   a_log=a_log, dt_bias=dt_bias)
    if gate is not None and (a_log is None or dt_bias is None):
        raise ValueError("gate needs A_log and dt_bias tensors")
    batch, seq_len, n_qk, n_v, scalar_gate = check_tensors(tensors, layout)
    if scale is None:
        scale = q.shape[-1] ** -0.5
    shape = make_shape(layout, batch, seq_len, n_qk, n_v, scale, qk_l2norm, beta_sigmoid,
                       q.shape[-1], v.shape[-1], scalar_gate, raw_gate=gate is not None)
    lib = _lib.load()
    if out is None:
        out = torch.empty_like(v)
    if final_state is None and output_final_state:
        final_state = torch.empty((batch, n_v, v.shape[-1], q.shape[-1]), dtype=torch.float32,
                                  device=v.device)
    nbytes = kda_chunk_fwd_workspace(shape)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=v.device)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                         f"the call needs {nbytes}")
    stream = ctypes.c_void_p(torch.cuda.current_stream(v.device).cuda_stream)
    args = [ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            _ptr(initial_state), _ptr(cu_seqlens), _ptr(out), _ptr(final_state),
            _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
            stream]
    if gate is not None:
        rg = KdaRawGate(a_log.data_ptr(), dt_bias.data_ptr(), float(lower_bound))
        args[6:6] = [ctypes.byref(rg)]     # after beta
        fn, fn_timed = lib.kda_chunk_fwd_raw_gate, lib.kda_chunk_fwd_raw_gate_timed
    else:
        fn, fn_timed = lib.kda_chunk_fwd, lib.kda_chunk_fwd_timed
    if stage_events is None:
        st = fn(*args)
    else:
        evs = (ctypes.c_void_p * len(stage_events))(*[ctypes.c_void_p(e) for e in stage_events])
        st = fn_timed(*args, evs, len(stage_events))
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_fwd")
    return out, final_state


def kda_chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                          beta: torch.Tensor, scale: Optional[float], initial_state,
                          cu_seqlens, layout: str, out: torch.Tensor,
                          final_state: Optional[torch.Tensor] = None, qk_l2norm: bool = True,
                          beta_sigmoid: bool = True) -> None:
    """kda_chunk_fwd_noalloc: the chunked forward with the library's own device scratch as the
    workspace; allocates nothing (the caller passes out and, optionally, final_state).  Calls
    that overlap in time on one GPU race on that scratch."""
    if out is None:
        raise ValueError("kda_chunk_fwd_noalloc writes into a caller-supplied out")
    tensors = dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=initial_state,
                   cu_seqlens=cu_seqlens, out=out, final_state=final_state)
    batch, seq_len, n_qk, n_v, scalar_gate = check_tensors(tensors, layout)
    if scale is None:
        scale = q.shape[-1] ** -0.5
    shape = make_shape(layout, batch, seq_len, n_qk, n_v, scale, qk_l2norm, beta_sigmoid,
                       q.shape[-1], v.shape[-1], scalar_gate)
    stream = ctypes.c_void_p(torch.cuda.current_stream(v.device).cuda_stream)
    st = _lib.load().kda_chunk_fwd_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
        _ptr(cu_seqlens), _ptr(out), _ptr(final_state), stream)
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_fwd_noalloc")


def chunk_fwd(inp, **kw):
    """Convenience: run on a workloads.Inputs bundle already on the GPU."""
    return kda_chunk_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.initial_state,
                         inp.cu_seqlens, inp.layout, inp.qk_l2norm, inp.beta_sigmoid,
                         gate=inp.gate_args, **kw)
