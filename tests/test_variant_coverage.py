"""Every kernel variant compiled into the library is launched by at least one GPU parity case.

The plan picks one kernel variant per stage from the shape (head dim, number of (sequence,
head) chains and of chunk records, gate form); the library reports that choice through
kda_chunk_fwd_plan_kernels without launching anything.  Replaying it over the shapes of every
GPU parity case (fixed cases, named workloads, the seeded sweep) must reach every variant that
kda_kernel_variant lists, so no kernel is left without a comparison against the oracle.
"""
import pytest

from kimi_delta_attention_chunk_amd import _lib
from kimi_delta_attention_chunk_amd.ops import kda_chunk_fwd_plan_kernels, kda_kernel_variants
from gpu_cases import all_case_shapes


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(_lib.LIB_PATH):
        from kimi_delta_attention_chunk_amd.build import build_library
        build_library()
    return _lib.load()


def test_every_variant_has_a_gpu_case(lib):
    reached = {}
    for name, shape in all_case_shapes():
        for k in kda_chunk_fwd_plan_kernels(shape):
            reached.setdefault(k, name)
    variants = kda_kernel_variants()
    assert len(set(variants)) == len(variants)
    missing = [v for v in variants if v not in reached]
    assert not missing, f"kernel variants no GPU case launches: {missing}"
    assert set(reached) <= set(variants)


def test_plan_kernels_buffer_checks(lib):
    import ctypes
    from kimi_delta_attention_chunk_amd.ops import make_shape
    shape = make_shape("BNSD", 1, 8192, 3, 3, 0.088)
    names = kda_chunk_fwd_plan_kernels(shape)
    assert names == ["kda_intra_kernel<0,128,2>", "kda_seg_kernel<128>",
                     "kda_combine_kernel<128>", "kda_out_kernel<128>"]
    need = len(";".join(names)) + 1
    buf = ctypes.create_string_buffer(b"x" * 8, need)
    assert lib.kda_chunk_fwd_plan_kernels(ctypes.byref(shape), buf, need - 1) == 1
    assert buf.raw[:8] == b"x" * 8   # nothing written on error
    assert lib.kda_chunk_fwd_plan_kernels(ctypes.byref(shape), buf, need) == 0
    assert lib.kda_chunk_fwd_plan_kernels(ctypes.byref(shape), None, 64) == 1
    bad = make_shape("BNSD", 1, 8192, 3, 3, 0.088, d_k=256, d_v=256)
    assert lib.kda_chunk_fwd_plan_kernels(ctypes.byref(bad), buf, need) == 2
    assert lib.kda_kernel_variant(-1) is None
    assert lib.kda_kernel_variant(lib.kda_num_kernel_variants()) is None
