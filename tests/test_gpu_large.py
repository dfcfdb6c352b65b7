"""GPU parity at a size where element offsets need 64 bits.

B=1, 8 heads, 2^21 tokens, head dim 128, BNSD: q, k, v and out hold 2^31 elements each (g,
in fp32, 8 GiB), the workspace 30 GB.  Every index into them past 2^31 - 1 must be computed
in 64 bits, in the kernels and in the host plan.  The inputs repeat one seeded 65,536-token
block 32 times along the sequence (any input is valid; the recurrence runs over all 2^21
tokens).  With 8 heads the plan takes the two-level scan, two segments of 16,384 chunks.  The
oracle checks one 16-row Dv tile of every head over all tokens, and those final-state rows
(state rows evolve independently in the recurrence).
"""
import time

import numpy as np
import pytest
import torch

from oracle import kda_oracle, QK_L2NORM, BETA_SIGMOID
from parity import assert_parity
from kimi_delta_attention_chunk_amd import chunk_fwd
from kimi_delta_attention_chunk_amd.workloads import Inputs, make_inputs

pytestmark = pytest.mark.gpu

S_BLOCK = 65536
REPS = 32
HEADS = 8
DV_TILE = (48, 64)


def log(msg: str, t0: float):
    print(f"[large] {msg} ({time.time() - t0:.1f} s)", flush=True)


def test_offsets_past_2_31_elements():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    t0 = time.time()
    base = make_inputs("BNSD", 1, S_BLOCK, HEADS, HEADS, g_kind="strong", init=True, seed=77)
    rep = lambda x: x.repeat(1, 1, REPS, 1) if x.dim() == 4 else x.repeat(1, 1, REPS)
    inp = Inputs("BNSD", 1, S_BLOCK * REPS, HEADS, HEADS, rep(base.q), rep(base.k),
                 rep(base.v), rep(base.g), rep(base.beta), base.initial_state, None)
    assert inp.q.numel() >= 2 ** 31 and inp.v.numel() >= 2 ** 31
    log(f"inputs {tuple(inp.q.shape)}", t0)
    d = inp.to("cuda")
    out, fin = chunk_fwd(d)
    torch.cuda.synchronize()
    lo, hi = DV_TILE
    out_t = out[..., lo:hi].float().cpu()
    fin_t = fin[:, :, lo:hi, :].cpu()
    del d, out, fin
    torch.cuda.empty_cache()
    log("GPU call done", t0)
    ro, rf = kda_oracle(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale, inp.initial_state,
                        None, "BNSD", QK_L2NORM | BETA_SIGMOID, dv_range=DV_TILE)
    log("oracle done", t0)
    assert_parity(out_t, np.ascontiguousarray(ro[..., lo:hi]), "2^31-element call out (Dv tile)")
    assert_parity(fin_t, np.ascontiguousarray(rf[:, :, lo:hi, :]),
                  "2^31-element call final_state (Dv tile)")
    log("compared", t0)
