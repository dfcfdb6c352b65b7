"""Independent fp64 evaluation of the KDA chunk equations, used only to pin the oracle.

The oracle walks the token recurrence.  This module instead evaluates the chunk form printed
in the FlashKDA README (section 功能说明) literally, with an explicit gamma^-1 and a library
matrix inverse.  The same section only says that the state is carried across chunks and the
output produced there; the vLLM #43195 summary (实现拆解, 关键源码片段) names the per-chunk
products h and v_new and an output kernel o = q h + A v_new.  The plain reading used here:

    G   = running sum of g inside the chunk          gamma = exp(G)
    Kt  = gamma * K      Kb = K / gamma      Qt = scale * gamma * Q
    T   = strictly-lower(diag(beta) Kt Kb^T)         Ainv = (I + T)^-1
    U   = Ainv diag(beta) V                           W = Ainv diag(beta) Kt
    Aqk = lower-with-diagonal(Qt Kb^T)
    Vn  = U - W S^T
    O   = Qt S^T + Aqk Vn
    S   = S diag(gamma_last) + Vn^T (K * exp(G_last - G))

fp64 holds gamma^-1 = e^{320} for a 64-token chunk at the g >= -5 floor, so the literal form is
exact up to rounding for every chunk size used here.
"""
from __future__ import annotations

import numpy as np


def _bf16_to_f64(x) -> np.ndarray:
    import torch
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _f64(x) -> np.ndarray:
    import torch
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def chunk_stream(q, k, v, g, beta, scale, S0, C):
    """One (sequence, head) stream.  q,k,g: [n, Dk]; v: [n, Dv]; beta: [n]; S0: [Dv, Dk]."""
    n, dk = q.shape
    dv = v.shape[1]
    S = S0.copy()
    out = np.zeros((n, dv))
    for s in range(0, n, C):
        e = min(n, s + C)
        Q, K, V, gg, b = q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e]
        m = e - s
        G = np.cumsum(gg, axis=0)
        gam = np.exp(G)
        Kt = gam * K
        Kb = K / gam
        Qt = scale * gam * Q
        T = np.tril(np.diag(b) @ Kt @ Kb.T, -1)
        Ainv = np.linalg.inv(np.eye(m) + T)
        U = Ainv @ np.diag(b) @ V
        W = Ainv @ np.diag(b) @ Kt
        Aqk = np.tril(Qt @ Kb.T)
        Vn = U - W @ S.T
        out[s:e] = Qt @ S.T + Aqk @ Vn
        S = S * gam[-1][None, :] + Vn.T @ (K * np.exp(G[-1][None, :] - G))
    return out, S


def bruteforce(inp, C: int):
    """Whole-tensor brute force for an ``Inputs`` bundle (any layout); fp64 numpy results."""
    q = _bf16_to_f64(inp.q)
    k = _bf16_to_f64(inp.k)
    v = _bf16_to_f64(inp.v)
    g = _f64(inp.g)
    beta = _bf16_to_f64(inp.beta)
    if inp.qk_l2norm:
        q = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
        k = k / np.sqrt((k * k).sum(-1, keepdims=True) + 1e-6)
    if inp.beta_sigmoid:
        beta = 1.0 / (1.0 + np.exp(-beta))
    grp = inp.n_v // inp.n_qk
    dv = v.shape[-1]
    dk = q.shape[-1]
    out = np.full(v.shape, np.nan)
    fin = np.zeros((inp.batch, inp.n_v, dv, dk))
    lengths = inp.lengths
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.tolist()
    for b in range(inp.batch):
        L = lengths[b]
        for h in range(inp.n_v):
            hq = h // grp
            if inp.layout == "BNSD":
                qq, kk = q[b, hq, :L], k[b, hq, :L]
                vv, gg, bb = v[b, h, :L], g[b, h, :L], beta[b, h, :L]
            elif inp.layout == "BSND":
                qq, kk = q[b, :L, hq], k[b, :L, hq]
                vv, gg, bb = v[b, :L, h], g[b, :L, h], beta[b, :L, h]
            else:
                t0 = cu[b]
                qq, kk = q[t0:t0 + L, hq], k[t0:t0 + L, hq]
                vv, gg, bb = v[t0:t0 + L, h], g[t0:t0 + L, h], beta[t0:t0 + L, h]
            S0 = (np.zeros((dv, dk)) if inp.initial_state is None
                  else _f64(inp.initial_state)[b, h])
            o, S = chunk_stream(qq, kk, vv, gg, bb, inp.scale, S0, C)
            if inp.layout == "BNSD":
                out[b, h, :L] = o
            elif inp.layout == "BSND":
                out[b, :L, h] = o
            else:
                out[cu[b]:cu[b] + L, h] = o
            fin[b, h] = S
    return out, fin
