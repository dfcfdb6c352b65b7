"""The C ABI on the CPU: the library loads, exports every declared symbol, and rejects bad
arguments on the host before touching a device (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

from kimi_delta_attention_chunk_amd import _lib
from kimi_delta_attention_chunk_amd.ops import make_shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from kimi_delta_attention_chunk_amd.build import build_library
        build_library()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("kda_chunk_fwd", "kda_chunk_fwd_workspace", "kda_status_str"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in kda.h but not exported"
    assert set(declared_functions()) == set(_lib.EXPORTED)


def test_status_strings(lib):
    assert lib.kda_status_str(0) == b"KDA_OK"
    assert lib.kda_status_str(3) == b"KDA_ERR_WORKSPACE"
    assert lib.kda_status_str(99) == b"unknown kda_status"
    assert lib.kda_num_stages() == 5
    names = [lib.kda_stage_name(i) for i in range(5)]
    assert names == [b"kda_intra_kernel", b"kda_seg_kernel", b"kda_combine_kernel",
                     b"kda_out_kernel", b"kda_scan_kernel"]
    assert lib.kda_stage_name(5) == b"unknown stage"
    assert lib.kda_version() >= 100


def ws(lib, shape):
    n = ctypes.c_size_t(0)
    st = lib.kda_chunk_fwd_workspace(ctypes.byref(shape), ctypes.byref(n))
    return st, n.value


def test_workspace_sizes(lib):
    st, n1 = ws(lib, make_shape("BNSD", 1, 8192, 3, 3, 0.088))
    assert st == 0
    # 128 chunks x 3 heads x (W, K_dec fp16, U fp16, Q', O_intra bf16, gamma), plus the
    # two-level scan (3 x (2 x 5 - 1) x 8 = 216 segment-pass workgroups -> 5 segments): per
    # segment P_s (fp16 128x128), N_s (fp32 128x128) and S_in (bf16 128x128), per record O0 and R (bf16
    # 64x128)
    rec = 16384 + 16384 + 16384 + 16384 + 16384 + 512
    assert rec == 82432
    two = 3 * 5 * (32768 + 65536 + 32768) + 384 * 2 * 16384
    assert n1 >= 128 * 3 * rec + two
    assert n1 < 128 * 3 * rec + two + 16 * 256
    # many heads: one-level scan, no matrices
    st, n4 = ws(lib, make_shape("BNSD", 1, 8192, 32, 32, 0.088))
    assert st == 0 and n4 < 128 * 32 * rec + 16 * 256
    st, n2 = ws(lib, make_shape("TND", 32, 65536, 32, 32, 0.088))
    assert st == 0 and n2 >= (65536 // 64 + 32) * 32 * 82432
    # a ragged tail adds one chunk slot per batch row
    st, n3 = ws(lib, make_shape("BSND", 4, 4100, 4, 16, 0.088))
    assert st == 0 and n3 >= 4 * 65 * 16 * 82432
    # head dim 64: a record of 64 x 64 x 10 + 64 x 4 bytes; six heads at 8K use the two-level
    # scan (6 x (2 x 5 - 1) x 4 = 216 workgroups -> 5 segments) with 64 x 64 fp32 matrices
    rec64 = 64 * 64 * 10 + 64 * 4
    assert rec64 == 41216
    st, n5 = ws(lib, make_shape("BNSD", 1, 8192, 6, 6, 0.125, d_k=64, d_v=64))
    assert st == 0
    two64 = 6 * 5 * 4 * 64 * 64 * 2 + 768 * 2 * 64 * 64 * 2
    assert n5 >= 128 * 6 * rec64 + two64
    assert n5 < 128 * 6 * rec64 + two64 + 16 * 256


def plan(lib, shape):
    mask, segs = ctypes.c_uint32(99), ctypes.c_int32(99)
    st = lib.kda_chunk_fwd_plan(ctypes.byref(shape), ctypes.byref(mask), ctypes.byref(segs))
    return st, mask.value, segs.value


def test_plan_query(lib):
    """Stage mask and segment count: the two-level scan when few chains would idle the GPU."""
    two = 0b01111    # intra, segment pass, combine, completion
    one = 0b10001    # intra, one-level scan
    # 3 heads x 8 tiles: (2P - 1) x 24 <= 256 -> P = 5
    assert plan(lib, make_shape("BNSD", 1, 8192, 3, 3, 0.088)) == (0, two, 5)
    # head dim 64: 6 heads x 4 tiles -> P = 5
    assert plan(lib, make_shape("BNSD", 1, 8192, 6, 6, 0.125, d_k=64, d_v=64)) == (0, two, 5)
    # 32 heads fill 256 workgroups: one level
    assert plan(lib, make_shape("BNSD", 1, 131072, 32, 32, 0.088)) == (0, one, 1)
    # 4 chunks cannot be cut into segments of at least 8 chunks
    assert plan(lib, make_shape("BNSD", 1, 256, 1, 1, 0.088)) == (0, one, 1)
    # 41 chunks of one head: 256 / 8 tiles -> 16, capped by 41 / 8
    assert plan(lib, make_shape("BNSD", 1, 64 * 40 + 9, 1, 1, 0.088)) == (0, two, 5)
    # an invalid shape: the workspace query's status, outputs untouched
    assert plan(lib, make_shape("BNSD", 1, 8192, 3, 3, 0.088, d_k=256, d_v=256)) == (2, 99, 99)
    assert lib.kda_chunk_fwd_plan(ctypes.byref(make_shape("BNSD", 1, 8192, 3, 3, 0.088)),
                                  None, None) == 0


@pytest.mark.parametrize("layout, batch, heads, d, scan", [
    # 32 chains fill the compute units with one-tile workgroups and the prefetch wave
    ("BNSD", 1, 32, 128, "kda_scan_kernel<1,128,true>"),
    # 33..64 chains at head dim 128: two tiles a workgroup, eight waves and the prefetch wave
    ("BNSD", 1, 33, 128, "kda_scan_kernel<2,128,true>"),
    ("BNSD", 1, 48, 128, "kda_scan_kernel<2,128,true>"),
    ("BSND", 4, 16, 128, "kda_scan_kernel<2,128,true>"),
    # 65..127 chains: two tiles on four waves, two workgroups a compute unit
    ("BNSD", 2, 48, 128, "kda_scan_kernel<2,128,false>"),
    ("BNSD", 1, 128, 128, "kda_scan_kernel<4,128,false>"),
    # head dim 64 keeps one tile up to 64 chains (with the prefetch wave up to 64)
    ("BNSD", 1, 48, 64, "kda_scan_kernel<1,64,true>"),
])
def test_plan_scan_kernel(layout, batch, heads, d, scan):
    """The one-level scan form the plan picks for a long sequence, by chains and head dim."""
    from kimi_delta_attention_chunk_amd import kda_chunk_fwd_plan_kernels
    shape = make_shape(layout, batch, 8192, heads, heads, 0.1, d_k=d, d_v=d)
    assert kda_chunk_fwd_plan_kernels(shape)[-1] == scan


@pytest.mark.parametrize("bad, code", [
    (dict(layout=7), 1), (dict(batch=0), 1), (dict(seq_len=0), 1), (dict(n_qk=0), 1),
    (dict(n_qk=4, n_v=2), 1), (dict(n_qk=3, n_v=4), 1), (dict(d_k=64), 2), (dict(d_v=256), 2),
    (dict(d_k=64, d_v=64), 0), (dict(d_k=32, d_v=32), 2), (dict(d_k=256, d_v=256), 2),
    (dict(scale=float("nan")), 1), (dict(flags=8), 0), (dict(flags=12), 2), (dict(flags=16), 1),
    (dict(flags=7), 0), (dict(flags=4), 0),
    (dict(layout=1, n_v=1 << 17), 2), (dict(layout=1, n_v=(1 << 17) - 2), 0),
])
def test_shape_rejections(lib, bad, code):
    kw = dict(layout="BNSD", batch=1, seq_len=100, n_qk=1, n_v=2, scale=0.1)
    shape = make_shape(**kw)
    for key, val in bad.items():
        setattr(shape, key, val)
    st, _ = ws(lib, shape)
    assert st == code


def call(lib, shape, **ptrs):
    base = dict(q=0x10000, k=0x20000, v=0x30000, g=0x40000, beta=0x50000, init=None, cu=None,
                out=0x60000, fin=0x70000, ws=0x100000, ws_bytes=1 << 40)
    base.update(ptrs)
    P = ctypes.c_void_p
    return lib.kda_chunk_fwd(ctypes.byref(shape), P(base["q"]), P(base["k"]), P(base["v"]),
                             P(base["g"]), P(base["beta"]), P(base["init"]), P(base["cu"]),
                             P(base["out"]), P(base["fin"]), P(base["ws"]),
                             ctypes.c_size_t(base["ws_bytes"]), P(None))


@pytest.mark.parametrize("ptrs, code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(g=None), 1),
    (dict(beta=None), 1), (dict(out=None), 1), (dict(q=0x10008), 1), (dict(g=0x40004), 1),
    (dict(out=0x60002), 1), (dict(init=0x80000, fin=0x80000), 1),
    (dict(init=0x80000, fin=0x80000 + 4096), 1), (dict(ws=None), 3), (dict(ws_bytes=1024), 3),
    (dict(ws=0x100010), 3),
    # what the call writes may overlap nothing else: out over v, out over the workspace, the
    # final state over q, the workspace over g
    (dict(out=0x30000 + 256), 1), (dict(out=0x100000 - 512), 1), (dict(fin=0x10000), 1),
    (dict(ws=0x40000, ws_bytes=1 << 20), 1),
])
def test_call_rejections(lib, ptrs, code):
    shape = make_shape("BNSD", 1, 100, 1, 2, 0.1)
    assert call(lib, shape, **ptrs) == code


def test_tnd_needs_cu_seqlens(lib):
    shape = make_shape("TND", 2, 100, 1, 1, 0.1)
    assert call(lib, shape, cu=None) == 1
    shape = make_shape("TND", 5, 3, 1, 1, 0.1)   # fewer tokens than sequences
    assert ws(lib, shape)[0] == 1


def test_timed_needs_events(lib):
    """Two events per stage; fewer is rejected before any launch (so fake pointers are safe)."""
    shape = make_shape("BNSD", 1, 100, 1, 1, 0.1)
    P = ctypes.c_void_p
    n = 2 * lib.kda_num_stages() - 1
    evs = (ctypes.c_void_p * n)()
    st = lib.kda_chunk_fwd_timed(ctypes.byref(shape), P(0x10000), P(0x20000), P(0x30000),
                                 P(0x40000), P(0x50000), P(None), P(None), P(0x60000),
                                 P(None), P(0x100000), ctypes.c_size_t(1 << 40), P(None), evs, n)
    assert st == 1
    st = lib.kda_chunk_fwd_timed(ctypes.byref(shape), P(0x10000), P(0x20000), P(0x30000),
                                 P(0x40000), P(0x50000), P(None), P(None), P(0x60000),
                                 P(None), P(0x100000), ctypes.c_size_t(1 << 40), P(None), None, 6)
    assert st == 1


def test_bench_record_model_matches_workspace(lib):
    """The benchmark's compulsory-byte model uses the library's record size: a one-level shape's
    workspace is chunk slots x value heads x that record, plus 256-byte alignment per array."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    for d, nv in ((128, 32), (64, 64)):
        st, n = ws(lib, make_shape("BNSD", 1, 64 * 300, nv, nv, 0.1, d_k=d, d_v=d))
        assert st == 0
        body = 300 * nv * bench.record_bytes(d)
        assert body <= n < body + 8 * 256, (d, n, body)


def call_raw(lib, shape, gate, timed_events=None, **ptrs):
    base = dict(q=0x10000, k=0x20000, v=0x30000, g=0x40000, beta=0x50000, init=None, cu=None,
                out=0x60000, fin=0x70000, ws=0x100000, ws_bytes=1 << 40)
    base.update(ptrs)
    P = ctypes.c_void_p
    args = [ctypes.byref(shape), P(base["q"]), P(base["k"]), P(base["v"]), P(base["g"]),
            P(base["beta"]), None if gate is None else ctypes.byref(gate), P(base["init"]),
            P(base["cu"]), P(base["out"]), P(base["fin"]), P(base["ws"]),
            ctypes.c_size_t(base["ws_bytes"]), P(None)]
    if timed_events is not None:
        return lib.kda_chunk_fwd_raw_gate_timed(*args, timed_events, 10)
    return lib.kda_chunk_fwd_raw_gate(*args)


@pytest.mark.parametrize("what, gate_kw, flags, ptrs, code", [
    ("no KDA_RAW_GATE flag", {}, 3, {}, 1),
    ("NULL gate", None, 11, {}, 1),
    ("NULL A_log", dict(a_log=None), 11, {}, 1),
    ("NULL dt_bias", dict(dt_bias=None), 11, {}, 1),
    ("misaligned dt_bias", dict(dt_bias=0x90004), 11, {}, 1),
    ("lower_bound below -5", dict(lower_bound=-5.5), 11, {}, 1),
    ("lower_bound above 0", dict(lower_bound=0.25), 11, {}, 1),
    ("lower_bound NaN", dict(lower_bound=float("nan")), 11, {}, 1),
    ("with the scalar gate", {}, 15, {}, 2),
    ("out over dt_bias", {}, 11, dict(out=0x90000 - 256), 1),
])
def test_raw_gate_rejections(lib, what, gate_kw, flags, ptrs, code):
    """The raw-gate entry point checks its activation parameters on the host, before any launch
    (so the fake pointers are never dereferenced)."""
    shape = make_shape("BNSD", 1, 100, 1, 2, 0.1)
    shape.flags = flags
    gate = None
    if gate_kw is not None:
        kw = dict(a_log=0x80000, dt_bias=0x90000, lower_bound=-5.0)
        kw.update(gate_kw)
        gate = _lib.KdaRawGate(kw["a_log"], kw["dt_bias"], kw["lower_bound"])
    assert call_raw(lib, shape, gate, **ptrs) == code, what
    if gate is not None:
        evs = (ctypes.c_void_p * 10)()
        assert call_raw(lib, shape, gate, timed_events=evs, **ptrs) == code, what


def test_raw_gate_flag_refused_by_plain_entry(lib):
    shape = make_shape("BNSD", 1, 100, 1, 2, 0.1, raw_gate=True)
    assert call(lib, shape) == 1
    assert ws(lib, shape)[0] == 0   # the workspace query accepts it (same size)
    assert ws(lib, shape)[1] == ws(lib, make_shape("BNSD", 1, 100, 1, 2, 0.1))[1]
