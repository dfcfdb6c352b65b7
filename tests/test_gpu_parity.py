"""GPU parity: the gfx950 library against the fp64 oracle, through the C ABI.

Small cases (several chunks, ragged tails, every layout, GQA, both fused-option settings) are
compared in full, for the per-channel gate and the scalar (GDN) gate, with cases that make the
plan select every kernel variant the library holds.  The named workloads run at their full
sizes in the launch configuration the benchmark times, and every output and final-state element
is compared with the oracle (head by head, to bound host memory).  Further tests check
invariants that hold at any size.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import kda_oracle, QK_L2NORM, BETA_SIGMOID, SCALAR_GATE
from parity import assert_parity
from kimi_delta_attention_chunk_amd import kda_chunk_fwd, chunk_fwd
from kimi_delta_attention_chunk_amd.workloads import (Inputs, make_inputs, workload_inputs,
                                                      WORKLOADS)
from gpu_cases import (SMALL, SCALAR_GATE_CASES, D64_CASES, TWO_LEVEL, VARIANT_CASES,
                       RAW_GATE_CASES, NO_DECAY_CASES, case_shape)
from kimi_delta_attention_chunk_amd.ops import kda_chunk_fwd_plan_kernels

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kimi_delta_attention_chunk_amd import _lib
    _lib.load()   # raises if libkda.so is missing: there is no fallback


def oracle_of(inp: Inputs, dv_range=None):
    flags = ((QK_L2NORM if inp.qk_l2norm else 0) | (BETA_SIGMOID if inp.beta_sigmoid else 0)
             | (SCALAR_GATE if inp.scalar_gate else 0))
    return kda_oracle(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.initial_state,
                      inp.cu_seqlens, inp.layout, flags, dv_range=dv_range,
                      raw_gate=inp.gate_args)


def run_gpu(inp: Inputs, **kw):
    d = inp.to("cuda")
    out, fin = chunk_fwd(d, **kw)
    torch.cuda.synchronize()
    return out, fin


def compare(inp: Inputs, what: str, dv_range=None):
    print(f"[case] {what}", flush=True)
    out, fin = run_gpu(inp)
    ro, rf = oracle_of(inp, dv_range)
    assert_parity(out, ro, f"{what} out")
    assert_parity(fin, rf, f"{what} final_state")
    return out, fin


def test_hand_example_zero_padded():
    ex = json.load(open(os.path.join(GOLDEN, "hand_example_d4.json")))
    D = 128
    q = torch.zeros(1, 1, 2, D)
    k = torch.zeros(1, 1, 2, D)
    v = torch.zeros(1, 1, 2, D)
    g = torch.zeros(1, 1, 2, D)
    q[0, 0, :, :4] = torch.tensor(ex["q"], dtype=torch.float32)
    k[0, 0, :, :4] = torch.tensor(ex["k"], dtype=torch.float32)
    v[0, 0, :, :4] = torch.tensor(ex["v"], dtype=torch.float32)
    g[0, 0, 1, 0] = math.log(0.5)
    beta = torch.tensor(ex["beta"]).reshape(1, 1, 2)
    inp = Inputs("BNSD", 1, 2, 1, 1, q.bfloat16(), k.bfloat16(), v.bfloat16(), g,
                 beta.bfloat16(), None, None, scale=ex["scale"], qk_l2norm=False,
                 beta_sigmoid=False)
    out, fin = run_gpu(inp)
    exp_out = np.zeros((2, D))
    exp_out[:, :4] = ex["out"]
    exp_fin = np.zeros((D, D))
    exp_fin[:4, :4] = ex["final_state"]
    assert_parity(out[0, 0], exp_out, "hand example out")
    assert_parity(fin[0, 0], exp_fin, "hand example final_state")


@pytest.mark.parametrize("name,kw", D64_CASES, ids=[s[0] for s in D64_CASES])
def test_head_dim_64(name, kw):
    inp = make_inputs(**kw)
    assert inp.q.shape[-1] == 64
    compare(inp, name)


@pytest.mark.parametrize("name,kw", SCALAR_GATE_CASES, ids=[s[0] for s in SCALAR_GATE_CASES])
def test_scalar_gate(name, kw):
    inp = make_inputs(**kw)
    assert inp.scalar_gate
    compare(inp, name)


@pytest.mark.parametrize("name,kw", TWO_LEVEL, ids=[s[0] for s in TWO_LEVEL])
def test_two_level_scan(name, kw):
    inp = make_inputs(**kw)
    compare(inp, name)


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_cases(name, kw):
    inp = make_inputs(**kw)
    compare(inp, name)


@pytest.mark.parametrize("name,kw", NO_DECAY_CASES, ids=[s[0] for s in NO_DECAY_CASES])
def test_no_decay_final_state(name, kw):
    compare(make_inputs(**kw), name)


def test_flags_off_prenormalised_inputs():
    inp = make_inputs("BNSD", 1, 160, 1, 2, g_kind="strong", init=True, seed=12)
    q = inp.q.double()
    k = inp.k.double()
    inp.q = (q / q.norm(dim=-1, keepdim=True)).bfloat16()
    inp.k = (k / k.norm(dim=-1, keepdim=True)).bfloat16()
    inp.beta = torch.sigmoid(inp.beta.double()).bfloat16()
    inp.qk_l2norm = False
    inp.beta_sigmoid = False
    compare(inp, "flags off")


@pytest.mark.parametrize("name,kw", VARIANT_CASES, ids=[s[0] for s in VARIANT_CASES])
def test_kernel_variants(name, kw):
    kernels = kda_chunk_fwd_plan_kernels(case_shape(kw))
    compare(make_inputs(**kw), f"{name} {kernels}")


@pytest.mark.parametrize("name,kw", RAW_GATE_CASES, ids=[s[0] for s in RAW_GATE_CASES])
def test_raw_gate(name, kw):
    inp = make_inputs(**kw)
    assert inp.raw_gate and inp.g.dtype == torch.bfloat16
    compare(inp, f"{name} {kda_chunk_fwd_plan_kernels(case_shape(kw))}")


HEAD_AXIS = {"BNSD": 1, "BSND": 2, "TND": 1}


@pytest.mark.parametrize("name", [w.name for w in WORKLOADS])
def test_workload(name):
    """Full size, every element: outputs compared one value head at a time (each head's slice
    meets the bar on its own, which implies it for the whole tensor)."""
    inp = workload_inputs(name)
    print(f"[case] workload {name}", flush=True)
    out, fin = run_gpu(inp)
    out = out.cpu()
    ro, rf = oracle_of(inp)
    ax = HEAD_AXIS[inp.layout]
    for h in range(inp.n_v):
        assert_parity(out.select(ax, h), np.take(ro, h, axis=ax), f"workload {name} out head {h}")
    assert_parity(fin, rf, f"workload {name} final_state")


# Range of the fp16 intermediates (U, the innovation v - S k, the combine's state operand):
# v and the initial state scaled by c.  The recurrence is linear in (v, S_0), so out and
# final_state scale by c as well; both sides are divided by c (a power of two, exact) and held
# to the same bar as unscaled inputs.  One-level and two-level forms, both head dims.
RANGE_CASES = [
    (c, kw) for c in (64.0, 512.0, 2048.0) for kw in (
        dict(layout="BNSD", batch=1, seq_len=300, n_qk=1, n_v=2, g_kind="unit", init=True,
             seed=71),
        dict(layout="BNSD", batch=1, seq_len=64 * 40 + 17, n_qk=1, n_v=1, g_kind="small",
             init=True, seed=72),
        dict(layout="BSND", batch=1, seq_len=64 * 24 + 3, n_qk=1, n_v=1, g_kind="zero",
             init=True, seed=73, d=64),
    )
]


@pytest.mark.parametrize("c,kw", RANGE_CASES,
                         ids=[f"v_x{int(c)}_{kw['layout']}_s{kw['seq_len']}_d{kw.get('d', 128)}"
                              for c, kw in RANGE_CASES])
def test_value_range(c, kw):
    inp = make_inputs(**kw)
    inp.v = (inp.v.float() * c).bfloat16()
    inp.initial_state = inp.initial_state * c
    print(f"[case] v and initial state x{c} {kw}", flush=True)
    out, fin = run_gpu(inp)
    ro, rf = oracle_of(inp)
    assert_parity(out.double() / c, ro / c, f"x{c} out / {c}")
    assert_parity(fin.double() / c, rf / c, f"x{c} final_state / {c}")


def test_layout_invariance_bitwise():
    inp = make_inputs("BNSD", 2, 130, 2, 4, g_kind="strong", init=True, seed=21)
    o1, f1 = run_gpu(inp)

    def bsnd(x):
        return x.permute(0, 2, 1, 3).contiguous() if x.dim() == 4 else \
            x.permute(0, 2, 1).contiguous()
    b = Inputs("BSND", 2, 130, 2, 4, bsnd(inp.q), bsnd(inp.k), bsnd(inp.v), bsnd(inp.g),
               bsnd(inp.beta), inp.initial_state, None, inp.scale)
    o2, f2 = run_gpu(b)
    def tnd(x):
        y = bsnd(x)
        return y.reshape((-1,) + tuple(y.shape[2:]))
    t = Inputs("TND", 2, 260, 2, 4, tnd(inp.q), tnd(inp.k), tnd(inp.v), tnd(inp.g),
               tnd(inp.beta), inp.initial_state, torch.tensor([0, 130, 260], dtype=torch.int32),
               inp.scale)
    o3, f3 = run_gpu(t)
    assert torch.equal(o2.permute(0, 2, 1, 3), o1)
    assert torch.equal(f2, f1)
    assert torch.equal(o3.reshape(2, 130, 4, 128).permute(0, 2, 1, 3), o1)
    assert torch.equal(f3, f1)


def test_packing_invariance_bitwise():
    lengths = [5, 64, 129, 1, 70]
    inp = make_inputs("TND", 5, 0, 1, 2, g_kind="strong", init=True, seed=22, lengths=lengths)
    o, f = run_gpu(inp)
    cu = inp.cu_seqlens.tolist()
    for s, L in enumerate(lengths):
        sl = slice(cu[s], cu[s + 1])
        one = Inputs("TND", 1, L, 1, 2, inp.q[sl].contiguous(), inp.k[sl].contiguous(),
                     inp.v[sl].contiguous(), inp.g[sl].contiguous(), inp.beta[sl].contiguous(),
                     inp.initial_state[s:s + 1].contiguous(),
                     torch.tensor([0, L], dtype=torch.int32), inp.scale)
        o1, f1 = run_gpu(one)
        assert torch.equal(o1, o[sl]), f"sequence {s} out"
        assert torch.equal(f1[0], f[s]), f"sequence {s} final_state"


def test_gqa_equals_repeated_heads_bitwise():
    inp = make_inputs("BNSD", 1, 100, 2, 6, g_kind="unit", init=True, seed=23)
    o, f = run_gpu(inp)
    idx = [0, 0, 0, 1, 1, 1]
    rep = Inputs("BNSD", 1, 100, 6, 6, inp.q[:, idx].contiguous(), inp.k[:, idx].contiguous(),
                 inp.v, inp.g, inp.beta, inp.initial_state, None, inp.scale)
    o2, f2 = run_gpu(rep)
    assert torch.equal(o, o2) and torch.equal(f, f2)


def test_run_to_run_determinism():
    inp = make_inputs("BSND", 2, 300, 2, 4, g_kind="strong", init=True, seed=24)
    o1, f1 = run_gpu(inp)
    o2, f2 = run_gpu(inp)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_concurrent_streams_bitwise():
    """Calls on two streams at once, each with its own workspace (the library keeps no state),
    give the results of the same calls made one after the other: a two-level call beside a
    one-level call, three rounds."""
    a = make_inputs("BNSD", 1, 64 * 40 + 9, 1, 2, g_kind="strong", init=True, seed=28).to("cuda")
    b = make_inputs("BSND", 2, 300, 2, 4, g_kind="unit", init=False, seed=29).to("cuda")
    oa, fa = chunk_fwd(a)
    ob, fb = chunk_fwd(b)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(s1):
            oa2, fa2 = chunk_fwd(a)
        with torch.cuda.stream(s2):
            ob2, fb2 = chunk_fwd(b)
        torch.cuda.synchronize()
        assert torch.equal(oa, oa2) and torch.equal(fa, fa2)
        assert torch.equal(ob, ob2) and torch.equal(fb, fb2)


def test_resume_split():
    full = make_inputs("BNSD", 1, 300, 1, 2, g_kind="strong", init=True, seed=25)
    o, f = run_gpu(full)
    for cut in (128, 100):
        parts = []
        for sl in (slice(0, cut), slice(cut, 300)):
            x = make_inputs("BNSD", 1, 300, 1, 2, g_kind="strong", init=True, seed=25)
            x.q, x.k, x.v = x.q[:, :, sl].contiguous(), x.k[:, :, sl].contiguous(), \
                x.v[:, :, sl].contiguous()
            x.g, x.beta = x.g[:, :, sl].contiguous(), x.beta[:, :, sl].contiguous()
            x.seq_len = sl.stop - sl.start
            parts.append(x)
        oa, fa = run_gpu(parts[0])
        parts[1].initial_state = fa.cpu()
        ob, fb = run_gpu(parts[1])
        oc = torch.cat([oa, ob], dim=2)
        if cut % 64 == 0:   # same chunk boundaries: identical arithmetic
            assert torch.equal(oc, o) and torch.equal(fb, f)
        else:
            ref_o, ref_f = oracle_of(full)
            assert_parity(oc, ref_o, f"resume at {cut} out")
            assert_parity(fb, ref_f, f"resume at {cut} final_state")


def test_output_guard_bands_and_padding_rows():
    """NaN-poisoned output with canary bands: every valid row is written, rows past a valid
    length are zero, nothing outside the tensor is touched, and the state is finite."""
    inp = make_inputs("BNSD", 2, 150, 1, 2, g_kind="floor", init=True, seed=26,
                      valid_lengths=[150, 77])
    d = inp.to("cuda")
    n = d.v.numel()
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    canary = torch.randn(guard, device="cuda").bfloat16()
    buf[:guard] = canary
    buf[-guard:] = canary
    out = buf[guard:guard + n].view(d.v.shape)
    fbuf = torch.full((d.initial_state.numel() + 2 * guard,), float("nan"), device="cuda")
    fin = fbuf[guard:guard + d.initial_state.numel()].view(d.initial_state.shape)
    chunk_fwd(d, out=out, final_state=fin)
    torch.cuda.synchronize()
    assert torch.equal(buf[:guard], canary) and torch.equal(buf[-guard:], canary)
    assert torch.isnan(fbuf[:guard]).all() and torch.isnan(fbuf[-guard:]).all()
    assert torch.isfinite(out[0]).all() and torch.isfinite(out[1, :, :77]).all()
    assert (out[1, :, 77:] == 0).all()
    assert torch.isfinite(fin).all()
    ro, rf = oracle_of(inp)
    assert_parity(out, ro, "guarded out")
    assert_parity(fin, rf, "guarded final_state")


@pytest.mark.parametrize("seq_len,init", [(100, False), (64 * 40 + 9, False), (64 * 40 + 9, True)],
                         ids=["one_level", "two_level", "two_level_init"])
def test_null_states(seq_len, init):
    """No final state requested (and no initial state), on both scan forms: the two-level
    combine then stops one step early."""
    inp = make_inputs("BNSD", 1, seq_len, 1, 1, g_kind="strong", init=init, seed=27)
    d = inp.to("cuda")
    out, fin = kda_chunk_fwd(d.q, d.k, d.v, d.g, d.beta, d.scale, d.initial_state, None, "BNSD",
                             output_final_state=False)
    torch.cuda.synchronize()
    assert fin is None
    ro, _ = oracle_of(inp)
    assert_parity(out, ro, "no final_state out")


@pytest.mark.parametrize("raw,n_v", [(False, 2), (True, 2), (False, 40)],
                         ids=["activated_gate", "raw_gate", "one_level_2tile_8wave"])
def test_timed_entry_points_bitwise(raw, n_v):
    """kda_chunk_fwd_timed and kda_chunk_fwd_raw_gate_timed run the same kernels as the untimed
    calls (their dispatches only record HIP events): bitwise equal outputs, and every event of a
    launched stage completes with a non-negative duration.  Two value heads take the two-level
    scan; forty the one-level two-tile scan on eight waves with the prefetch wave."""
    from kimi_delta_attention_chunk_amd import kda_num_stages
    inp = make_inputs("BNSD", 1, 64 * 40 + 9, 1, n_v, g_kind="strong", init=True, seed=29,
                      raw_gate=raw).to("cuda")
    o1, f1 = chunk_fwd(inp)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * kda_num_stages())]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    o2, f2 = chunk_fwd(inp, stage_events=[e.cuda_event for e in evs])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    for s in range(kda_num_stages()):
        assert evs[2 * s].elapsed_time(evs[2 * s + 1]) >= 0.0
