"""Seeded random sweep: GPU against the fp64 oracle on shapes that mix the options.

The fixed cases in test_gpu_parity.py each vary one thing; here every case draws all of them
at once from a fixed seed: layout (BNSD, BSND, packed TND), head dim 64 or 128, GQA group 1, 2
or 4, sequence lengths from 1 token to several chunks (ragged tails), per-row valid lengths,
the gate's distribution (including no decay and the -5 floor), the scalar (GDN) gate, an
initial state or none, and the fused q/k L2 norm and beta sigmoid on or off (off with inputs
normalised beforehand).  About a third of the cases have one or two heads and sequences of
1,100 to 2,600 tokens, which the plan runs as the two-level scan.  Every output and final state
is compared, to the same bar as every other parity test.
"""
from __future__ import annotations

import random

import pytest
import torch

from oracle import kda_oracle, QK_L2NORM, BETA_SIGMOID, SCALAR_GATE
from parity import assert_parity
from kimi_delta_attention_chunk_amd import chunk_fwd
from kimi_delta_attention_chunk_amd.ops import make_shape, kda_chunk_fwd_plan
from kimi_delta_attention_chunk_amd.workloads import make_inputs

N_CASES = 24
SEED = 20261203


def draw_cases(n: int = N_CASES, seed: int = SEED) -> list:
    rng = random.Random(seed)
    cases = []
    for i in range(n):
        layout = rng.choice(["BNSD", "BSND", "TND"])
        d = rng.choice([64, 128])
        long = rng.random() < 0.35
        if long:
            n_qk, n_v = 1, rng.choice([1, 2])
        else:
            n_qk = rng.choice([1, 2])
            n_v = n_qk * rng.choice([1, 2, 4])
        kw = dict(layout=layout, n_qk=n_qk, n_v=n_v, d=d, seed=1000 + i,
                  g_kind=rng.choice(["strong", "unit", "small", "mixed", "floor", "zero"]),
                  init=rng.random() < 0.6, scalar_gate=rng.random() < 0.3)
        if layout == "TND":
            batch = rng.randint(1, 3) if long else rng.randint(1, 5)
            kw.update(batch=batch, seq_len=0,
                      lengths=[rng.randint(1, 2600 if long else 300) for _ in range(batch)])
        else:
            batch = 1 if long else rng.randint(1, 3)
            seq_len = rng.randint(1100, 2600) if long else rng.randint(1, 400)
            kw.update(batch=batch, seq_len=seq_len)
            if rng.random() < 0.4:
                kw["valid_lengths"] = [rng.randint(1, seq_len) for _ in range(batch)]
        flags_on = rng.random() >= 0.2
        cases.append((f"sweep{i:02d}", kw, flags_on))
    return cases


CASES = draw_cases()


def build(kw: dict, flags_on: bool):
    inp = make_inputs(**kw)
    if not flags_on:   # the fused options off: inputs normalised and beta in (0, 1) already
        q = inp.q.double()
        k = inp.k.double()
        inp.q = (q / q.norm(dim=-1, keepdim=True).clamp_min(1e-30)).bfloat16()
        inp.k = (k / k.norm(dim=-1, keepdim=True).clamp_min(1e-30)).bfloat16()
        inp.beta = torch.sigmoid(inp.beta.double()).bfloat16()
        inp.qk_l2norm = False
        inp.beta_sigmoid = False
    return inp


def plan_of(inp, d: int):
    shape = make_shape(inp.layout, inp.batch, inp.seq_len, inp.n_qk, inp.n_v, inp.scale,
                       inp.qk_l2norm, inp.beta_sigmoid, d, d, inp.scalar_gate)
    return kda_chunk_fwd_plan(shape)


def test_sweep_covers_the_options():
    """The drawn set (host only) reaches both scan forms, both head dims and every option."""
    two_level = d64 = gqa = sg = off = tnd = vl = 0
    for _, kw, flags_on in CASES:
        inp = build(kw, flags_on)
        _, segs = plan_of(inp, kw["d"])
        two_level += segs > 1
        d64 += kw["d"] == 64
        gqa += kw["n_v"] > kw["n_qk"]
        sg += kw["scalar_gate"]
        off += not flags_on
        tnd += kw["layout"] == "TND"
        vl += "valid_lengths" in kw
    assert min(two_level, d64, gqa, sg, off, tnd, vl) >= 2, (two_level, d64, gqa, sg, off, tnd, vl)
    assert two_level < len(CASES)


@pytest.mark.gpu
@pytest.mark.parametrize("name,kw,flags_on", CASES, ids=[c[0] for c in CASES])
def test_sweep(name, kw, flags_on):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    inp = build(kw, flags_on)
    mask, segs = plan_of(inp, kw["d"])
    what = (f"{name} {kw['layout']} D={kw['d']} B={kw['batch']} S={kw['seq_len']} "
            f"lens={kw.get('lengths') or kw.get('valid_lengths')} heads={kw['n_qk']}/{kw['n_v']} "
            f"g={kw['g_kind']} init={kw['init']} sg={kw['scalar_gate']} flags={flags_on} "
            f"segments={segs}")
    print(f"[case] {what}", flush=True)
    out, fin = chunk_fwd(inp.to("cuda"))
    torch.cuda.synchronize()
    flags = ((QK_L2NORM if inp.qk_l2norm else 0) | (BETA_SIGMOID if inp.beta_sigmoid else 0)
             | (SCALAR_GATE if inp.scalar_gate else 0))
    ro, rf = kda_oracle(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.initial_state,
                        inp.cu_seqlens, inp.layout, flags)
    assert_parity(out, ro, f"{name} out")
    assert_parity(fin, rf, f"{name} final_state")
