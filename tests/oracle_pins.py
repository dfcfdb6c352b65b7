"""Pins that tie the fp64 oracle to something other than itself.

Each ``pin_*`` function takes the path of an oracle shared library and raises AssertionError
when that library disagrees with the pages or with mathematics:

  hand example      values worked out by hand for two tokens at D=4 (tests/golden)
  brute force       the chunk equations of the FlashKDA README evaluated literally in fp64
                    (explicit gamma^-1, numpy matrix inverse), chunk sizes 1, 2, 3, 7, 16, 64
  beta = 0          closed form: pure per-channel decay of the initial state
  g = 0             the plain delta rule S <- S (I - beta k k^T) + beta v k^T
  retrieval         beta = 1 and unit keys make S_t k_t = v_t, so q_t = k_t reads back scale*v_t
  linearity         (V, S0) -> (O, S_T) is linear
  resume            splitting a sequence and carrying the state equals one run
  layouts/packing   BNSD, BSND and TND hold the same numbers; packed sequences are independent
  GQA               Nqk < Nv equals repeating each q/k head over its group
  fused options     sigmoid(0) = 1/2; L2-normalising c*u equals u for a unit u
  valid lengths     cu_seqlens with BNSD truncates each batch row
  row subsets       computing a subset of state rows equals the full run
  scalar gate       one gate per (token, head): the gated delta rule in the form
                    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T, and the per-channel
                    form with the gate repeated over the channels, in every layout
  raw gate          the activation g = lower_bound * sigmoid(exp(A_log[h]) (g_raw + dt_bias[h]))
                    at closed-form points: a raw gate cancelling dt_bias gives lower_bound / 2,
                    a large one lower_bound, exp(A_log) = 3 or 1/2 per value head gives
                    lower_bound * sigmoid(3) or sigmoid(1/2), lower_bound = 0 gives no decay;
                    with beta = 0 every activated gate lies in [lower_bound, 0]

The same functions run against compile-time planted mistakes in the oracle
(tests/test_oracle_mutants.py) to show that each mistake is caught by at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from oracle import kda_oracle, QK_L2NORM, BETA_SIGMOID, SCALAR_GATE
from bruteforce_chunked import bruteforce
from kimi_delta_attention_chunk_amd.workloads import make_inputs, Inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _run(lib, inp: Inputs, **kw):
    flags = ((QK_L2NORM if inp.qk_l2norm else 0) | (BETA_SIGMOID if inp.beta_sigmoid else 0)
             | (SCALAR_GATE if inp.scalar_gate else 0))
    return kda_oracle(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.initial_state,
                      inp.cu_seqlens, inp.layout, flags, lib_path=lib, raw_gate=inp.gate_args,
                      **kw)


def _close(a, b, atol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    m = ~np.isnan(b)
    assert np.array_equal(np.isnan(a), np.isnan(b)), f"{what}: NaN pattern differs"
    err = float(np.max(np.abs(a[m] - b[m]))) if m.any() else 0.0
    assert err <= atol, f"{what}: max |diff| {err:.3e} > {atol:.1e}"


def _bf(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def pin_hand_example(lib):
    ex = json.load(open(os.path.join(GOLDEN, "hand_example_d4.json")))
    g = np.array([[0, 0, 0, 0], [math.log(0.5), 0, 0, 0]], dtype=np.float32)
    inp = Inputs("TND", 1, 2, 1, 1,
                 _bf(ex["q"]).reshape(2, 1, 4), _bf(ex["k"]).reshape(2, 1, 4),
                 _bf(ex["v"]).reshape(2, 1, 4), torch.from_numpy(g).reshape(2, 1, 4),
                 _bf(ex["beta"]).reshape(2, 1), None,
                 torch.tensor([0, 2], dtype=torch.int32), scale=ex["scale"],
                 qk_l2norm=False, beta_sigmoid=False)
    out, fin = _run(lib, inp)
    _close(out.reshape(2, 4), np.array(ex["out"]), 1e-8, "hand example out")
    _close(fin[0, 0], np.array(ex["final_state"]), 1e-8, "hand example final_state")


def pin_bruteforce_chunked(lib):
    cases = [
        make_inputs("BNSD", 2, 70, 1, 2, g_kind="strong", init=True, seed=11, d=16),
        make_inputs("BSND", 1, 67, 2, 4, g_kind="floor", init=True, seed=12, d=8),
        make_inputs("TND", 3, 0, 1, 1, g_kind="unit", init=True, seed=13,
                    lengths=[5, 64, 33], d=16),
    ]
    for i, inp in enumerate(cases):
        out, fin = _run(lib, inp)
        for C in (1, 2, 3, 7, 16, 64):
            bo, bf = bruteforce(inp, C)
            _close(out, bo, 1e-9, f"case {i} C={C} out")
            _close(fin, bf, 1e-9, f"case {i} C={C} final_state")
    # full head size, one 64-token chunk plus a tail, every gate at the -5 floor
    inp = make_inputs("BNSD", 1, 100, 1, 1, g_kind="floor", init=True, seed=14)
    out, fin = _run(lib, inp)
    bo, bf = bruteforce(inp, 64)
    _close(out, bo, 1e-9, "D=128 floor out")
    _close(fin, bf, 1e-9, "D=128 floor final_state")


def pin_beta_zero(lib):
    d, n = 8, 23
    inp = make_inputs("BNSD", 1, n, 1, 1, g_kind="strong", init=True, seed=21, d=d)
    inp.beta = torch.zeros_like(inp.beta)
    inp.qk_l2norm = False
    inp.beta_sigmoid = False
    out, fin = _run(lib, inp)
    S0 = inp.initial_state[0, 0].double().numpy()
    G = np.cumsum(inp.g[0, 0].double().numpy(), axis=0)
    q = inp.q[0, 0].double().numpy()
    expect_o = np.stack([inp.scale * (S0 * np.exp(G[t])[None, :]) @ q[t] for t in range(n)])
    _close(out[0, 0], expect_o, 1e-10, "beta=0 out")
    _close(fin[0, 0], S0 * np.exp(G[-1])[None, :], 1e-10, "beta=0 final_state")


def pin_plain_delta_rule(lib):
    d, n = 8, 31
    inp = make_inputs("BNSD", 1, n, 1, 1, g_kind="zero", init=True, seed=31, d=d)
    out, fin = _run(lib, inp)
    q = inp.q[0, 0].double().numpy()
    k = inp.k[0, 0].double().numpy()
    q = q / np.sqrt((q * q).sum(1, keepdims=True) + 1e-6)
    k = k / np.sqrt((k * k).sum(1, keepdims=True) + 1e-6)
    v = inp.v[0, 0].double().numpy()
    b = 1 / (1 + np.exp(-inp.beta[0, 0].double().numpy()))
    S = inp.initial_state[0, 0].double().numpy()
    eo = np.zeros((n, d))
    for t in range(n):
        # S (I - b k k^T) + b v k^T : the Householder-like form of the delta rule
        S = S @ (np.eye(d) - b[t] * np.outer(k[t], k[t])) + b[t] * np.outer(v[t], k[t])
        eo[t] = inp.scale * S @ q[t]
    _close(out[0, 0], eo, 1e-10, "g=0 out")
    _close(fin[0, 0], S, 1e-10, "g=0 final_state")


def pin_perfect_retrieval(lib):
    d, n = 16, 40
    rng = np.random.default_rng(41)
    keys = np.zeros((n, d), dtype=np.float32)
    for t in range(n):
        idx = rng.choice(d, 4, replace=False)
        keys[t, idx] = rng.choice([-0.5, 0.5], 4)
    inp = make_inputs("BNSD", 1, n, 1, 1, g_kind="strong", init=True, seed=42, d=d)
    inp.k = _bf(keys).reshape(1, 1, n, d)
    inp.q = inp.k.clone()
    inp.beta = torch.ones_like(inp.beta)
    inp.qk_l2norm = False
    inp.beta_sigmoid = False
    out, _ = _run(lib, inp)
    _close(out[0, 0], inp.scale * inp.v[0, 0].double().numpy(), 1e-10, "retrieval out")


def pin_linearity(lib):
    d, n = 8, 29
    base = make_inputs("BNSD", 1, n, 1, 1, g_kind="unit", init=True, seed=51, d=d)
    mask = (torch.arange(d) % 2 == 0)
    v1 = torch.where(mask, base.v, torch.zeros_like(base.v))
    v2 = base.v - v1
    s1 = torch.where(mask[:, None], base.initial_state, torch.zeros_like(base.initial_state))
    s2 = base.initial_state - s1
    outs = []
    for vv, ss in ((base.v, base.initial_state), (v1, s1), (v2, s2), (2 * base.v,
                                                                    2 * base.initial_state)):
        inp = make_inputs("BNSD", 1, n, 1, 1, g_kind="unit", init=True, seed=51, d=d)
        inp.v, inp.initial_state = vv, ss
        outs.append(_run(lib, inp))
    (o, f), (o1, f1), (o2, f2), (o3, f3) = outs
    _close(o1 + o2, o, 1e-10, "additivity out")
    _close(f1 + f2, f, 1e-10, "additivity final_state")
    _close(o3, 2 * o, 1e-10, "homogeneity out")
    _close(f3, 2 * f, 1e-10, "homogeneity final_state")


def pin_resume_split(lib):
    d, n = 16, 150
    full = make_inputs("BNSD", 1, n, 1, 2, g_kind="strong", init=True, seed=61, d=d)
    out, fin = _run(lib, full)
    for cut in (1, 37, 64, 100):
        a = make_inputs("BNSD", 1, n, 1, 2, g_kind="strong", init=True, seed=61, d=d)
        b = make_inputs("BNSD", 1, n, 1, 2, g_kind="strong", init=True, seed=61, d=d)
        for x, sl in ((a, slice(0, cut)), (b, slice(cut, n))):
            x.q, x.k, x.v = x.q[:, :, sl].contiguous(), x.k[:, :, sl].contiguous(), \
                x.v[:, :, sl].contiguous()
            x.g, x.beta = x.g[:, :, sl].contiguous(), x.beta[:, :, sl].contiguous()
            x.seq_len = sl.stop - sl.start
        oa, fa = _run(lib, a)
        b.initial_state = torch.from_numpy(fa.astype(np.float32))
        ob, fb = _run(lib, b)
        # the carried state passes through fp32 (the boundary's state dtype)
        _close(np.concatenate([oa, ob], axis=2), out, 2e-6, f"resume at {cut} out")
        _close(fb, fin, 2e-6, f"resume at {cut} final_state")


def _permute_layouts(inp: Inputs):
    """Same numbers as BSND and as TND (B=1 per sequence row) from a BNSD bundle."""
    def bsnd(x):
        return x.permute(0, 2, 1, 3).contiguous() if x.dim() == 4 else \
            x.permute(0, 2, 1).contiguous()

    def tnd(x):
        y = bsnd(x)
        return y.reshape((-1,) + tuple(y.shape[2:]))
    cu = torch.tensor([inp.seq_len * i for i in range(inp.batch + 1)], dtype=torch.int32)
    b = Inputs("BSND", inp.batch, inp.seq_len, inp.n_qk, inp.n_v, bsnd(inp.q), bsnd(inp.k),
               bsnd(inp.v), bsnd(inp.g), bsnd(inp.beta), inp.initial_state, None, inp.scale)
    t = Inputs("TND", inp.batch, inp.seq_len * inp.batch, inp.n_qk, inp.n_v, tnd(inp.q),
               tnd(inp.k), tnd(inp.v), tnd(inp.g), tnd(inp.beta), inp.initial_state, cu,
               inp.scale)
    return b, t


def pin_layout_invariance(lib):
    inp = make_inputs("BNSD", 2, 45, 2, 4, g_kind="strong", init=True, seed=71, d=8)
    out, fin = _run(lib, inp)
    b, t = _permute_layouts(inp)
    ob, fb = _run(lib, b)
    ot, ft = _run(lib, t)
    _close(ob.transpose(0, 2, 1, 3), out, 0.0, "BSND vs BNSD out")
    _close(fb, fin, 0.0, "BSND vs BNSD final_state")
    _close(ot.reshape(2, 45, 4, 8).transpose(0, 2, 1, 3), out, 0.0, "TND vs BNSD out")
    _close(ft, fin, 0.0, "TND vs BNSD final_state")


def pin_packing_invariance(lib):
    lengths = [7, 64, 1, 90]
    inp = make_inputs("TND", 4, 0, 1, 2, g_kind="strong", init=True, seed=81,
                      lengths=lengths, d=8)
    out, fin = _run(lib, inp)
    cu = inp.cu_seqlens.tolist()
    for s in range(4):
        sl = slice(cu[s], cu[s + 1])
        one = Inputs("TND", 1, lengths[s], 1, 2, inp.q[sl], inp.k[sl], inp.v[sl], inp.g[sl],
                     inp.beta[sl], inp.initial_state[s:s + 1].contiguous(),
                     torch.tensor([0, lengths[s]], dtype=torch.int32), inp.scale)
        o1, f1 = _run(lib, one)
        _close(o1, out[sl], 0.0, f"packed sequence {s} out")
        _close(f1[0], fin[s], 0.0, f"packed sequence {s} final_state")


def pin_gqa(lib):
    inp = make_inputs("BNSD", 1, 50, 2, 4, g_kind="strong", init=True, seed=91, d=8)
    out, fin = _run(lib, inp)
    rep = Inputs("BNSD", 1, 50, 4, 4, inp.q[:, [0, 0, 1, 1]].contiguous(),
                 inp.k[:, [0, 0, 1, 1]].contiguous(), inp.v, inp.g, inp.beta,
                 inp.initial_state, None, inp.scale)
    o2, f2 = _run(lib, rep)
    _close(o2, out, 0.0, "GQA vs repeated heads out")
    _close(f2, fin, 0.0, "GQA vs repeated heads final_state")


def pin_fused_options(lib):
    d, n = 16, 20
    rng = np.random.default_rng(101)
    units = np.zeros((2, n, d), dtype=np.float32)
    for a in range(2):
        for t in range(n):
            idx = rng.choice(d, 4, replace=False)
            units[a, t, idx] = rng.choice([-0.5, 0.5], 4)
    plain = make_inputs("BNSD", 1, n, 1, 1, g_kind="strong", init=True, seed=102, d=d)
    plain.q = _bf(units[0]).reshape(1, 1, n, d)
    plain.k = _bf(units[1]).reshape(1, 1, n, d)
    plain.beta = torch.full_like(plain.beta, 0.5)
    plain.qk_l2norm = False
    plain.beta_sigmoid = False
    fused = make_inputs("BNSD", 1, n, 1, 1, g_kind="strong", init=True, seed=102, d=d)
    fused.q = _bf(3 * units[0]).reshape(1, 1, n, d)     # |3u| = 3: normalises back to ~u
    fused.k = _bf(2 * units[1]).reshape(1, 1, n, d)
    fused.beta = torch.zeros_like(fused.beta)            # sigmoid(0) = 1/2
    po, pf = _run(lib, plain)
    fo, ff = _run(lib, fused)
    # the 1e-6 inside the norm's square root moves |u|=1 by about 1e-7
    _close(fo, po, 1e-6, "fused options out")
    _close(ff, pf, 1e-6, "fused options final_state")


def pin_valid_lengths(lib):
    lens = [30, 64, 1]
    inp = make_inputs("BNSD", 3, 70, 1, 2, g_kind="strong", init=True, seed=111,
                      valid_lengths=lens, d=8)
    out, fin = _run(lib, inp)
    for b, L in enumerate(lens):
        one = Inputs("BNSD", 1, L, 1, 2, inp.q[b:b + 1, :, :L].contiguous(),
                     inp.k[b:b + 1, :, :L].contiguous(), inp.v[b:b + 1, :, :L].contiguous(),
                     inp.g[b:b + 1, :, :L].contiguous(), inp.beta[b:b + 1, :, :L].contiguous(),
                     inp.initial_state[b:b + 1].contiguous(), None, inp.scale)
        o1, f1 = _run(lib, one)
        _close(out[b:b + 1, :, :L], o1, 0.0, f"valid length row {b} out")
        _close(fin[b:b + 1], f1, 0.0, f"valid length row {b} final_state")
        assert np.isnan(out[b, :, L:]).all(), "rows past the valid length must stay undefined"


def pin_row_subset(lib):
    inp = make_inputs("BNSD", 1, 40, 1, 2, g_kind="strong", init=True, seed=121, d=32)
    out, fin = _run(lib, inp)
    so, sf = _run(lib, inp, dv_range=(5, 21))
    _close(so[..., 5:21], out[..., 5:21], 0.0, "row subset out")
    _close(sf[:, :, 5:21], fin[:, :, 5:21], 0.0, "row subset final_state")
    assert np.isnan(so[..., :5]).all() and np.isnan(sf[:, :, 21:]).all()


def pin_scalar_gate(lib):
    """One gate per (token, value head), shared by every key channel (the GDN form).

    (a) Two value heads reading one q/k head, against the gated delta rule written as
        S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T with a_t = exp(g_t), token by token
        in numpy fp64.
    (b) In BNSD, BSND and TND, the same numbers as the per-channel form with each token's gate
        repeated over the channels.
    """
    d, n = 16, 37
    inp = make_inputs("BNSD", 1, n, 1, 2, g_kind="unit", init=True, seed=131, d=d,
                      scalar_gate=True)
    assert inp.scalar_gate and tuple(inp.g.shape) == (1, 2, n)
    out, fin = _run(lib, inp)
    q = inp.q[0, 0].double().numpy()
    k = inp.k[0, 0].double().numpy()
    q = q / np.sqrt((q * q).sum(1, keepdims=True) + 1e-6)
    k = k / np.sqrt((k * k).sum(1, keepdims=True) + 1e-6)
    for h in range(2):
        v = inp.v[0, h].double().numpy()
        b = 1 / (1 + np.exp(-inp.beta[0, h].double().numpy()))
        a = np.exp(inp.g[0, h].double().numpy())
        S = inp.initial_state[0, h].double().numpy()
        eo = np.zeros((n, d))
        for t in range(n):
            S = a[t] * S @ (np.eye(d) - b[t] * np.outer(k[t], k[t])) + b[t] * np.outer(v[t], k[t])
            eo[t] = inp.scale * S @ q[t]
        _close(out[0, h], eo, 1e-10, f"scalar gate out, head {h}")
        _close(fin[0, h], S, 1e-10, f"scalar gate final_state, head {h}")
    for layout, kw in (("BNSD", {}), ("BSND", {}), ("TND", dict(lengths=[13, 24]))):
        sc = make_inputs(layout, 2, 19, 1, 2, g_kind="strong", init=True, seed=132, d=d,
                         scalar_gate=True, **kw)
        pc = make_inputs(layout, 2, 19, 1, 2, g_kind="strong", init=True, seed=132, d=d, **kw)
        pc.q, pc.k, pc.v, pc.beta, pc.initial_state = sc.q, sc.k, sc.v, sc.beta, sc.initial_state
        pc.g = sc.g[..., None].expand(*sc.g.shape, d).contiguous()
        so, sf = _run(lib, sc)
        po, pf = _run(lib, pc)
        _close(so, po, 0.0, f"scalar vs repeated gate out ({layout})")
        _close(sf, pf, 0.0, f"scalar vs repeated gate final_state ({layout})")


def _raw_and_fp32(layout, seed, d=16, n=37, n_qk=1, n_v=2):
    """A raw-gate input set and a copy with an fp32 gate in its place (same other tensors)."""
    raw = make_inputs(layout, 1, n, n_qk, n_v, init=True, seed=seed, d=d, raw_gate=True)
    f32 = make_inputs(layout, 1, n, n_qk, n_v, g_kind="zero", init=True, seed=seed, d=d)
    f32.q, f32.k, f32.v, f32.beta, f32.initial_state = raw.q, raw.k, raw.v, raw.beta, \
        raw.initial_state
    return raw, f32


def _per_head(x, layout, vals):
    """A tensor shaped like v whose value head h holds vals[h] (broadcast over tokens and channels)."""
    ax = 1 if layout == "BNSD" else 2
    shape = [1] * x.dim()
    shape[ax] = len(vals)
    return torch.as_tensor(vals, dtype=torch.float32).reshape(shape).expand(x.shape)


def pin_raw_gate(lib):
    """The raw-gate activation at points where it has a closed form."""
    lb = -5.0
    for layout in ("BNSD", "BSND"):
        # (a) g_raw = -dt_bias (dt_bias rounded to bf16 so that -dt_bias is a bf16 value):
        #     sigmoid(0) = 1/2 for any A_log, so g = lb / 2 everywhere
        raw, f32 = _raw_and_fp32(layout, 141)
        raw.dt_bias = raw.dt_bias.to(torch.bfloat16).float()
        db = raw.dt_bias[None, :, None, :] if layout == "BNSD" else raw.dt_bias[None, None]
        raw.g = (-db).expand(raw.v.shape).contiguous().to(torch.bfloat16)
        f32.g = torch.full(raw.v.shape, lb / 2, dtype=torch.float32)
        for (o1, f1), (o2, f2) in [(_run(lib, raw), _run(lib, f32))]:
            _close(o1, o2, 0.0, f"raw gate at -dt_bias out ({layout})")
            _close(f1, f2, 0.0, f"raw gate at -dt_bias final_state ({layout})")
        # (b) g_raw = 64, |dt_bias| < 6, A_log = 0: sigmoid(58..70) is 1 in fp64, so g = lb
        raw, f32 = _raw_and_fp32(layout, 142)
        raw.g = torch.full(raw.v.shape, 64.0).to(torch.bfloat16)
        raw.dt_bias = raw.dt_bias.clamp(-5.9, 5.9)
        raw.a_log = torch.zeros_like(raw.a_log)
        f32.g = torch.full(raw.v.shape, lb, dtype=torch.float32)
        (o1, f1), (o2, f2) = _run(lib, raw), _run(lib, f32)
        _close(o1, o2, 0.0, f"saturated raw gate out ({layout})")
        _close(f1, f2, 0.0, f"saturated raw gate final_state ({layout})")
        # (c) g_raw = 1, dt_bias = 0, exp(A_log) = 3 for value head 0 and 1/2 for head 1 (both
        #     read the one q/k head): g = lb sigmoid(3) and lb sigmoid(1/2); the fp32 copy holds
        #     those constants rounded to fp32, and A_log is itself an fp32 value
        raw, f32 = _raw_and_fp32(layout, 143)
        raw.g = torch.ones(raw.v.shape).to(torch.bfloat16)
        raw.dt_bias = torch.zeros_like(raw.dt_bias)
        raw.a_log = torch.tensor([math.log(3.0), math.log(0.5)], dtype=torch.float32)
        s3, sh = 1.0 / (1.0 + math.exp(-3.0)), 1.0 / (1.0 + math.exp(-0.5))
        f32.g = _per_head(raw.v, layout, [lb * s3, lb * sh]).contiguous()
        (o1, f1), (o2, f2) = _run(lib, raw), _run(lib, f32)
        _close(o1, o2, 1e-5, f"time scale exp(A_log) out ({layout})")
        _close(f1, f2, 1e-5, f"time scale exp(A_log) final_state ({layout})")
    # (d) lower_bound = 0: no decay at all, whatever the raw gate
    raw, f32 = _raw_and_fp32("BNSD", 144)
    raw.lower_bound = 0.0
    (o1, f1), (o2, f2) = _run(lib, raw), _run(lib, f32)
    _close(o1, o2, 0.0, "lower_bound 0 out")
    _close(f1, f2, 0.0, "lower_bound 0 final_state")
    # (e) beta = 0: S_T = S_0 Diag(exp(sum_t g_t)), so log(S_T / S_0) per key channel is the sum
    #     of the activated gates over the T tokens, which must lie in [T lb, 0] (and strictly
    #     inside for finite raw gates)
    raw, _ = _raw_and_fp32("BNSD", 145, n=23)
    raw.g = (3.0 * raw.g.float()).to(torch.bfloat16)
    raw.beta = torch.zeros_like(raw.beta)
    raw.beta_sigmoid = False
    raw.qk_l2norm = False
    _, fin = _run(lib, raw)
    s0 = raw.initial_state.double().numpy()
    with np.errstate(invalid="ignore", divide="ignore"):
        tot = np.log(fin / s0)   # [1, h, dv, dk], equal along dv
    assert np.all(tot < 0) and np.all(tot > 23 * lb), "activated gates outside (lb, 0)"
    assert np.allclose(tot, tot[:, :, :1, :], atol=1e-9), "decay must depend on the key channel only"


ALL_PINS = [pin_hand_example, pin_bruteforce_chunked, pin_beta_zero, pin_plain_delta_rule,
            pin_perfect_retrieval, pin_linearity, pin_resume_split, pin_layout_invariance,
            pin_packing_invariance, pin_gqa, pin_fused_options, pin_valid_lengths,
            pin_row_subset, pin_scalar_gate, pin_raw_gate]
