"""The Python binding's argument checks, on the CPU: every tensor's dtype, shape, contiguity and
device is checked before a pointer reaches the library, so a short, wrongly shaped or host
buffer raises instead of reaching a kernel."""
import pytest
import torch

from kimi_delta_attention_chunk_amd import kda_chunk_fwd
from kimi_delta_attention_chunk_amd.ops import check_tensors

B, NQK, NV, S, D = 2, 1, 2, 70, 128


def tensors(layout="BNSD", **over):
    if layout == "BNSD":
        qs, vs, bs = (B, NQK, S, D), (B, NV, S, D), (B, NV, S)
    elif layout == "BSND":
        qs, vs, bs = (B, S, NQK, D), (B, S, NV, D), (B, S, NV)
    else:
        qs, vs, bs = (S, NQK, D), (S, NV, D), (S, NV)
    t = dict(q=torch.zeros(qs, dtype=torch.bfloat16), k=torch.zeros(qs, dtype=torch.bfloat16),
             v=torch.zeros(vs, dtype=torch.bfloat16), g=torch.zeros(vs),
             beta=torch.zeros(bs, dtype=torch.bfloat16),
             initial_state=torch.zeros(B, NV, D, D),
             cu_seqlens=torch.tensor([0, 30, S], dtype=torch.int32) if layout == "TND" else None,
             out=None, final_state=None, workspace=None)
    t.update(over)
    return t


@pytest.mark.parametrize("layout", ["BNSD", "BSND", "TND"])
def test_valid_host_tensors_are_refused_as_host(layout):
    t = tensors(layout)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        check_tensors(t, layout)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], None, t["initial_state"],
                      t["cu_seqlens"], layout)


def test_scalar_gate_shape_is_recognised():
    t = tensors("BSND", g=torch.zeros(B, S, NV))
    with pytest.raises(ValueError, match="GPU"):
        check_tensors(t, "BSND")


BAD = [
    ("v short in S", dict(v=torch.zeros(B, NV, S - 1, D, dtype=torch.bfloat16)), ValueError),
    ("v short in batch", dict(v=torch.zeros(B - 1, NV, S, D, dtype=torch.bfloat16)), ValueError),
    ("g short", dict(g=torch.zeros(B, NV, S - 1, D)), ValueError),
    ("g wrong dtype", dict(g=torch.zeros(B, NV, S, D, dtype=torch.bfloat16)), TypeError),
    ("beta short", dict(beta=torch.zeros(B, NV, S - 1, dtype=torch.bfloat16)), ValueError),
    ("k differs", dict(k=torch.zeros(B, NQK, S, 64, dtype=torch.bfloat16)), ValueError),
    ("state shape", dict(initial_state=torch.zeros(B, NV, D, D - 1)), ValueError),
    ("state dtype", dict(initial_state=torch.zeros(B, NV, D, D, dtype=torch.float64)), TypeError),
    ("state not contiguous", dict(initial_state=torch.zeros(B, NV, D, D).transpose(2, 3)),
     ValueError),
    ("out shape", dict(out=torch.zeros(B, NV, S, D - 8, dtype=torch.bfloat16)), ValueError),
    ("out dtype", dict(out=torch.zeros(B, NV, S, D)), TypeError),
    ("final_state shape", dict(final_state=torch.zeros(B, NV, D, 64)), ValueError),
    ("cu_seqlens too few entries", dict(cu_seqlens=torch.tensor([0, 30], dtype=torch.int32)),
     ValueError),
    ("cu_seqlens dtype", dict(cu_seqlens=torch.tensor([0, 30, 60], dtype=torch.int64)),
     TypeError),
    ("q not contiguous", dict(q=torch.zeros(B, S, NQK, D, dtype=torch.bfloat16).transpose(1, 2)),
     ValueError),
    ("q wrong rank", dict(q=torch.zeros(NQK, S, D, dtype=torch.bfloat16)), ValueError),
]


@pytest.mark.parametrize("what,over,exc", BAD, ids=[b[0] for b in BAD])
def test_bad_tensors(what, over, exc):
    with pytest.raises(exc):
        check_tensors(tensors("BNSD", **over), "BNSD")


def test_tnd_cu_seqlens_checks():
    with pytest.raises(ValueError, match="cu_seqlens"):
        check_tensors(tensors("TND", cu_seqlens=None), "TND")
    with pytest.raises(ValueError, match="cu_seqlens"):
        check_tensors(tensors("TND", cu_seqlens=torch.tensor([0], dtype=torch.int32)), "TND")
    with pytest.raises(ValueError, match="shape"):   # batch + 1 entries: initial_state disagrees
        check_tensors(tensors("TND", cu_seqlens=torch.tensor([0, 10, 20, S], dtype=torch.int32)),
                      "TND")


def test_unknown_layout():
    with pytest.raises(ValueError, match="layout"):
        check_tensors(tensors("BNSD"), "NSD")


def test_raw_gate_tensor_checks():
    base = tensors("BNSD", g=torch.zeros(B, NV, S, D, dtype=torch.bfloat16))
    ok = dict(base, a_log=torch.zeros(NV), dt_bias=torch.zeros(NV, D))
    with pytest.raises(ValueError, match="GPU"):
        check_tensors(ok, "BNSD")
    with pytest.raises(TypeError):   # the raw gate is bf16
        check_tensors(dict(ok, g=torch.zeros(B, NV, S, D)), "BNSD")
    with pytest.raises(ValueError, match="shape"):
        check_tensors(dict(ok, dt_bias=torch.zeros(NV, D - 1)), "BNSD")
    with pytest.raises(ValueError, match="shape"):
        check_tensors(dict(ok, a_log=torch.zeros(NV + 1)), "BNSD")
    with pytest.raises(ValueError, match="both"):
        check_tensors(dict(base, a_log=torch.zeros(NV)), "BNSD")
