"""Seeded synthetic inputs for the KDA chunked forward.

This module only draws random tensors with the shapes and value distributions of the
workloads below; it holds none of the method's arithmetic.  The same host tensors feed the GPU
library and the fp64 oracle.

Conventions shared with the library (FlashKDA README, sections 参数说明 and 约束说明):
q/k/v/beta are bf16, g and the states are fp32, cu_seqlens is an int32 prefix sum.
By default q and k are raw N(0,1) rows and beta holds N(0,1) logits; the library is then
called with its fused row L2-normalise and beta-sigmoid options switched on, which yields the
"row L2-normalised q/k" and "beta = sigmoid(N(0,1))" distributions of the workloads.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

D = 128


@dataclass(frozen=True)
class Workload:
    name: str
    layout: str                 # "BNSD" | "BSND" | "TND"
    batch: int                  # B, or the number of packed sequences for TND
    seq_len: int                # stored length S (TND: ignored, lengths are drawn)
    n_qk: int
    n_v: int
    g_kind: str                 # "small" | "strong" | "unit" | "mixed"
    init: bool                  # draw an fp32 N(0, 0.1^2) initial state
    seed: int
    tnd_max_len: int = 0        # TND: lengths uniform in [1, tnd_max_len]
    note: str = ""
    scalar_gate: bool = False   # one gate per (token, value head), shaped like beta
    d: int = D                  # head dim d_k = d_v (128 or 64)
    raw_gate: bool = False      # raw bf16 gate with A_log, dt_bias, lower_bound = -5


WORKLOADS = [
    Workload("tiny_s256", "BNSD", 1, 256, 1, 1, "small", False, 1000,
             note="B=1, Nqk=Nv=1, S=256 (4 chunks); g = -0.05*U(0,1); zero state"),
    Workload("prefill_s8k_n3", "BNSD", 1, 8192, 3, 3, "strong", True, 1001,
             note="B=1, Nqk=Nv=3, S=8192, BNSD; g = -5*sigmoid(N(0,1)); state N(0,0.1^2)"),
    Workload("gqa_tail_s4100", "BSND", 4, 4100, 4, 16, "unit", False, 1002,
             note="B=4, Nqk=4, Nv=16, S=4100 (tail of 4), BSND; g = -sigmoid(N(0,1))"),
    Workload("varlen_tnd_32seq", "TND", 32, 0, 32, 32, "strong", True, 1003, tnd_max_len=4096,
             note="32 packed sequences, lengths U{1..4096}; Nqk=Nv=32; per-sequence states"),
    Workload("long_s128k_n32", "BNSD", 1, 131072, 32, 32, "mixed", False, 1004,
             note="B=1, Nqk=Nv=32, S=131072 (2048 chunks/head); mixed per-channel decay"),
    Workload("gdn_prefill_s8k_n3", "BNSD", 1, 8192, 3, 3, "strong", True, 1005,
             note="the 8K prefill with one gate per (token, head) (the GDN form); "
                  "g = -5*sigmoid(N(0,1))", scalar_gate=True),
    Workload("prefill_s8k_n3_raw_gate", "BNSD", 1, 8192, 3, 3, "raw", True, 1007,
             note="the 8K prefill with the raw bf16 gate activated in the kernel, as in the "
                  "FlashKDA README's quick start: g, A_log, dt_bias ~ N(0,1), lower_bound = -5",
             raw_gate=True),
    Workload("prefill_s8k_n6_d64", "BNSD", 1, 8192, 6, 6, "strong", True, 1006,
             note="the 8K prefill at head dim 64 with six heads (the same q/k/v bytes as three "
                  "128-dim heads); g = -5*sigmoid(N(0,1)); state N(0,0.1^2)", d=64),
    Workload("prefill_s8k_n48", "BNSD", 1, 8192, 48, 48, "strong", True, 1008,
             note="B=1, Nqk=Nv=48, S=8192, BNSD (the largest head count of the FlashKDA README's "
                  "performance shapes); g = -5*sigmoid(N(0,1)); state N(0,0.1^2)"),
]
BY_NAME = {w.name: w for w in WORKLOADS}


@dataclass
class Inputs:
    layout: str
    batch: int
    seq_len: int                # S for BNSD/BSND, T for TND
    n_qk: int
    n_v: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    initial_state: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    scale: float = 1.0 / math.sqrt(D)
    qk_l2norm: bool = True
    beta_sigmoid: bool = True
    meta: dict = field(default_factory=dict)
    # raw-gate form: g is the raw bf16 gate (v's shape) and these activate it
    a_log: Optional[torch.Tensor] = None      # fp32 [n_v]
    dt_bias: Optional[torch.Tensor] = None    # fp32 [n_v, d_k]
    lower_bound: float = -5.0

    @property
    def raw_gate(self) -> bool:
        """g is the raw bf16 gate, activated with a_log, dt_bias and lower_bound."""
        return self.a_log is not None

    @property
    def gate_args(self):
        """(A_log, dt_bias, lower_bound) of the raw-gate form, or None."""
        return (self.a_log, self.dt_bias, self.lower_bound) if self.raw_gate else None

    @property
    def scalar_gate(self) -> bool:
        """g holds one value per (token, value head) (beta's shape) instead of one per channel."""
        return tuple(self.g.shape) == tuple(self.beta.shape)

    @property
    def lengths(self) -> list:
        if self.cu_seqlens is None:
            return [self.seq_len] * self.batch
        c = self.cu_seqlens.tolist()
        return [c[i + 1] - c[i] for i in range(len(c) - 1)]

    @property
    def tokens(self) -> int:
        return int(sum(self.lengths))

    def to(self, device) -> "Inputs":
        def mv(t):
            return None if t is None else t.to(device)
        return Inputs(self.layout, self.batch, self.seq_len, self.n_qk, self.n_v,
                      mv(self.q), mv(self.k), mv(self.v), mv(self.g), mv(self.beta),
                      mv(self.initial_state), mv(self.cu_seqlens), self.scale,
                      self.qk_l2norm, self.beta_sigmoid, dict(self.meta), mv(self.a_log),
                      mv(self.dt_bias), self.lower_bound)


def _gate(kind: str, shape, gen: torch.Generator) -> torch.Tensor:
    """Natural-log decay g <= 0, one draw per element of `shape` ("mixed" splits the last axis)."""
    if kind == "small":
        return -0.05 * torch.rand(shape, generator=gen)
    if kind == "strong":
        return -5.0 * torch.sigmoid(torch.randn(shape, generator=gen))
    if kind == "unit":
        return -1.0 * torch.sigmoid(torch.randn(shape, generator=gen))
    if kind == "mixed":
        half = shape[-1] // 2
        a = -0.01 * torch.rand(tuple(shape[:-1]) + (half,), generator=gen)
        b = -5.0 * torch.sigmoid(torch.randn(tuple(shape[:-1]) + (shape[-1] - half,),
                                             generator=gen))
        return torch.cat([a, b], dim=-1)
    if kind == "zero":
        return torch.zeros(shape)
    if kind == "floor":
        return torch.full(shape, -5.0)
    raise ValueError(kind)


def make_inputs(layout: str, batch: int, seq_len: int, n_qk: int, n_v: int, *,
                g_kind: str = "strong", init: bool = False, seed: int = 0,
                lengths: Optional[list] = None, valid_lengths: Optional[list] = None,
                d: int = D, scalar_gate: bool = False, raw_gate: bool = False,
                lower_bound: float = -5.0) -> Inputs:
    """Draw one seeded input set.

    layout "TND" packs ``lengths`` (a list of sequence lengths) into T tokens; for BNSD/BSND
    ``valid_lengths`` (optional) becomes a cu_seqlens prefix sum of per-row valid lengths.
    ``scalar_gate`` draws g with beta's shape (one gate per token and value head).
    ``raw_gate`` draws, as the FlashKDA README's quick start does, a raw bf16 gate g ~ N(0,1)
    (v's shape), A_log ~ N(0,1) [n_v] and dt_bias ~ N(0,1) [n_v, d] in fp32 (g_kind unused).
    """
    gen = torch.Generator().manual_seed(int(seed))
    if layout == "TND":
        assert lengths is not None and len(lengths) == batch
        T = int(sum(lengths))
        qs, vs, bs = (T, n_qk, d), (T, n_v, d), (T, n_v)
        cu = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0).tolist()),
                          dtype=torch.int32)
        stored = T
    else:
        if layout == "BNSD":
            qs, vs, bs = (batch, n_qk, seq_len, d), (batch, n_v, seq_len, d), (batch, n_v,
                                                                               seq_len)
        elif layout == "BSND":
            qs, vs, bs = (batch, seq_len, n_qk, d), (batch, seq_len, n_v, d), (batch, seq_len,
                                                                               n_v)
        else:
            raise ValueError(layout)
        cu = None
        if valid_lengths is not None:
            cu = torch.tensor([0] + list(torch.tensor(valid_lengths).cumsum(0).tolist()),
                              dtype=torch.int32)
        stored = seq_len
    q = torch.randn(qs, generator=gen).to(torch.bfloat16)
    k = torch.randn(qs, generator=gen).to(torch.bfloat16)
    v = torch.randn(vs, generator=gen).to(torch.bfloat16)
    if raw_gate:
        if scalar_gate:
            raise ValueError("the raw-gate form has one gate per key channel")
        g = torch.randn(vs, generator=gen).to(torch.bfloat16)
    else:
        g = _gate(g_kind, bs if scalar_gate else vs, gen).to(torch.float32).contiguous()
    beta = torch.randn(bs, generator=gen).to(torch.bfloat16)
    st = None
    if init:
        st = (0.1 * torch.randn((batch, n_v, d, d), generator=gen)).to(torch.float32)
    inp = Inputs(layout, batch, stored, n_qk, n_v, q, k, v, g, beta, st, cu)
    if raw_gate:
        inp.a_log = torch.randn((n_v,), generator=gen).to(torch.float32)
        inp.dt_bias = torch.randn((n_v, d), generator=gen).to(torch.float32)
        inp.lower_bound = float(lower_bound)
    return inp


def _tnd_lengths(w: Workload, s: int) -> list:
    gen = torch.Generator().manual_seed(s + 7919)
    return torch.randint(1, w.tnd_max_len + 1, (w.batch,), generator=gen).tolist()


def workload_shape(w) -> dict:
    """make_inputs keyword arguments of a named workload's shape (sequence lengths drawn as
    workload_inputs draws them; no tensors)."""
    if isinstance(w, str):
        w = BY_NAME[w]
    kw = dict(layout=w.layout, batch=w.batch, seq_len=w.seq_len, n_qk=w.n_qk, n_v=w.n_v,
              d=w.d, scalar_gate=w.scalar_gate, raw_gate=w.raw_gate)
    if w.layout == "TND":
        kw.update(seq_len=0, lengths=_tnd_lengths(w, w.seed))
    return kw


def workload_inputs(w, seed: Optional[int] = None) -> Inputs:
    """Inputs of one named workload (seed defaults to the workload's own)."""
    if isinstance(w, str):
        w = BY_NAME[w]
    s = w.seed if seed is None else seed
    if w.layout == "TND":
        lengths = _tnd_lengths(w, s)
        inp = make_inputs("TND", w.batch, 0, w.n_qk, w.n_v, g_kind=w.g_kind, init=w.init,
                          seed=s, lengths=lengths, scalar_gate=w.scalar_gate, d=w.d,
                          raw_gate=w.raw_gate)
    else:
        inp = make_inputs(w.layout, w.batch, w.seq_len, w.n_qk, w.n_v, g_kind=w.g_kind,
                          init=w.init, seed=s, scalar_gate=w.scalar_gate, d=w.d,
                          raw_gate=w.raw_gate)
    inp.meta["workload"] = w.name
    return inp
