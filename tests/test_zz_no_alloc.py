"""The allocation-free entry point (kda_chunk_fwd_noalloc) against kda_chunk_fwd, through the C
ABI: the same kernels on the same inputs, so out and final_state must be bitwise equal.  Two
calls in a row, the second with a smaller input (the scratch keeps the first call's contents),
on a two-level and a one-level shape, then a shape past the scratch limit, rejected on the
host before any launch."""
import ctypes

import pytest
import torch

from kimi_delta_attention_chunk_amd import _lib, chunk_fwd
from kimi_delta_attention_chunk_amd.ops import (kda_chunk_fwd_workspace, make_shape)
from kimi_delta_attention_chunk_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def noalloc(lib, d, out, fin):
    shape = make_shape(d.layout, d.batch, d.seq_len, d.n_qk, d.n_v, d.scale, d.qk_l2norm,
                       d.beta_sigmoid, d.q.shape[-1], d.v.shape[-1], d.scalar_gate)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.kda_chunk_fwd_noalloc(ctypes.byref(shape), ptr(d.q), ptr(d.k), ptr(d.v),
                                     ptr(d.g), ptr(d.beta), ptr(d.initial_state),
                                     ptr(d.cu_seqlens), ptr(out), ptr(fin), stream)


CASES = [
    # first call, then a smaller one: the two-level scan (8K tokens, 3 heads), then one head
    (dict(layout="BNSD", batch=1, seq_len=8192, n_qk=3, n_v=3, g_kind="strong", init=True,
          seed=81),
     dict(layout="TND", batch=3, seq_len=0, n_qk=1, n_v=2, g_kind="unit", init=True, seed=82,
          lengths=[700, 5, 130])),
    (dict(layout="BSND", batch=2, seq_len=1000, n_qk=2, n_v=8, g_kind="small", init=False,
          seed=83),
     dict(layout="BNSD", batch=1, seq_len=77, n_qk=1, n_v=1, g_kind="strong", init=True,
          seed=84, d=64)),
]


@pytest.mark.parametrize("first,second", CASES, ids=["two_level_then_tnd", "gqa_then_d64"])
def test_noalloc_matches_kda_chunk_fwd(first, second):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = _lib.load()
    for kw in (first, second):
        print(f"[case] noalloc {kw}", flush=True)
        d = make_inputs(**kw).to("cuda")
        ref_out, ref_fin = chunk_fwd(d)
        out = torch.full_like(d.v, float("nan"))
        fin = torch.full_like(ref_fin, float("nan"))
        assert noalloc(lib, d, out, fin) == 0
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), "out differs from kda_chunk_fwd"
        assert torch.equal(fin, ref_fin), "final_state differs from kda_chunk_fwd"


def test_noalloc_rejects_shapes_past_the_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = _lib.load()
    shape = make_shape("BNSD", 1, 65536, 4, 4, 0.088)
    assert kda_chunk_fwd_workspace(shape) > _lib.NOALLOC_SCRATCH_BYTES
    P = ctypes.c_void_p
    # rejected from the shape alone: the (fake, never dereferenced) pointers are not used
    st = lib.kda_chunk_fwd_noalloc(ctypes.byref(shape), P(0x10000), P(0x20000), P(0x30000),
                                   P(0x40000), P(0x50000), P(None), P(None), P(0x60000),
                                   P(None), P(None))
    assert st == 3   # KDA_ERR_WORKSPACE
