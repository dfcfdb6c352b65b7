"""Shapes of the GPU parity cases, shared by the GPU tests and by the CPU check that every kernel
variant the plan can select is reached by at least one of them.

Each case is (name, keyword arguments of workloads.make_inputs).  This module draws no tensors.
"""
from __future__ import annotations

from kimi_delta_attention_chunk_amd.ops import make_shape
from kimi_delta_attention_chunk_amd.workloads import WORKLOADS, workload_shape

SMALL = [
    ("bnsd_b2_n2_s200_strong_init", dict(layout="BNSD", batch=2, seq_len=200, n_qk=2, n_v=2,
                                         g_kind="strong", init=True, seed=5)),
    ("bsnd_gqa_b2_s150", dict(layout="BSND", batch=2, seq_len=150, n_qk=1, n_v=4,
                              g_kind="unit", init=False, seed=6)),
    ("tnd_ragged", dict(layout="TND", batch=6, seq_len=0, n_qk=2, n_v=2, g_kind="strong",
                        init=True, seed=7, lengths=[1, 63, 64, 65, 130, 17])),
    ("bnsd_valid_lengths", dict(layout="BNSD", batch=3, seq_len=140, n_qk=1, n_v=1,
                                g_kind="small", init=True, seed=8, valid_lengths=[140, 65, 3])),
    ("bnsd_floor_decay", dict(layout="BNSD", batch=1, seq_len=256, n_qk=1, n_v=2,
                              g_kind="floor", init=True, seed=9)),
    ("bnsd_no_decay", dict(layout="BNSD", batch=1, seq_len=192, n_qk=1, n_v=1,
                           g_kind="zero", init=True, seed=10)),
    # no decay over 64 chunks: the state never forgets, so rounding accumulates longest here
    ("bnsd_no_decay_s4096", dict(layout="BNSD", batch=1, seq_len=4096, n_qk=1, n_v=1,
                                 g_kind="zero", init=True, seed=11)),
    # the scan walks sequences longest first: equal lengths (ties broken by index) and more
    # sequences than it ranks (index order)
    ("tnd_equal_lengths", dict(layout="TND", batch=6, seq_len=0, n_qk=1, n_v=2,
                               g_kind="strong", init=True, seed=12,
                               lengths=[100, 3, 100, 100, 64, 100])),
    ("tnd_300_short_seqs", dict(layout="TND", batch=300, seq_len=0, n_qk=1, n_v=1,
                                g_kind="strong", init=True, seed=13,
                                lengths=[1 + (37 * i) % 90 for i in range(300)])),
]

# One gate per (token, value head) (KDA_SCALAR_GATE, the GDN form): every layout, GQA, ragged
# tails, valid lengths, and a sequence long enough for the two-level scan.
SCALAR_GATE_CASES = [
    ("gdn_bnsd_gqa_tail", dict(layout="BNSD", batch=2, seq_len=300, n_qk=1, n_v=2,
                               g_kind="strong", init=True, seed=41, scalar_gate=True)),
    ("gdn_bsnd_valid_lengths", dict(layout="BSND", batch=2, seq_len=200, n_qk=2, n_v=2,
                                    g_kind="unit", init=False, seed=42, valid_lengths=[200, 77],
                                    scalar_gate=True)),
    ("gdn_tnd_ragged", dict(layout="TND", batch=4, seq_len=0, n_qk=2, n_v=4, g_kind="strong",
                            init=True, seed=43, lengths=[150, 64, 1, 90], scalar_gate=True)),
    ("gdn_bnsd_two_level", dict(layout="BNSD", batch=1, seq_len=64 * 40 + 5, n_qk=1, n_v=1,
                                g_kind="small", init=True, seed=44, scalar_gate=True)),
]


# No decay: the state never forgets, so the final state is the case nearest the bound.  These
# are the worst of 150 seeded random no-decay draws (at up to 0.95 of the bound before the
# T/Aqk operands of the intra kernel were made more precise, about 0.56-0.69 after), kept as
# fixed cases so that a loss of precision shows here first.
NO_DECAY_CASES = [
    ("nd_d64_bsnd_b2_init", dict(layout="BSND", batch=2, seq_len=604, n_qk=4, n_v=4, d=64,
                                 g_kind="zero", init=True, seed=9015)),
    ("nd_d64_bsnd_gqa16", dict(layout="BSND", batch=1, seq_len=1102, n_qk=8, n_v=16, d=64,
                               g_kind="zero", init=False, seed=9011)),
    ("nd_d64_bnsd_scalar_gate", dict(layout="BNSD", batch=1, seq_len=712, n_qk=8, n_v=16, d=64,
                                     g_kind="zero", init=True, seed=9107, scalar_gate=True)),
    ("nd_d128_tnd_ragged", dict(layout="TND", batch=3, seq_len=0, n_qk=4, n_v=8, d=128,
                                g_kind="zero", init=False, seed=9146, lengths=[23, 867, 1145])),
]

# Head dim 64 (d_k = d_v = 64): every layout, GQA, ragged tails, valid lengths, no decay, the
# scalar gate, and a sequence long enough for the two-level scan.
D64_CASES = [
    ("d64_bnsd_b2_s200", dict(layout="BNSD", batch=2, seq_len=200, n_qk=2, n_v=2,
                              g_kind="strong", init=True, seed=51, d=64)),
    ("d64_bsnd_gqa_tail", dict(layout="BSND", batch=2, seq_len=150, n_qk=1, n_v=4,
                               g_kind="unit", init=False, seed=52, d=64)),
    ("d64_tnd_ragged", dict(layout="TND", batch=5, seq_len=0, n_qk=2, n_v=2, g_kind="strong",
                            init=True, seed=53, lengths=[1, 63, 65, 130, 17], d=64)),
    ("d64_bnsd_valid_lengths", dict(layout="BNSD", batch=3, seq_len=140, n_qk=1, n_v=1,
                                    g_kind="small", init=True, seed=54,
                                    valid_lengths=[140, 65, 3], d=64)),
    ("d64_bnsd_no_decay", dict(layout="BNSD", batch=1, seq_len=1024, n_qk=1, n_v=1,
                               g_kind="zero", init=True, seed=55, d=64)),
    ("d64_two_level", dict(layout="BNSD", batch=1, seq_len=64 * 40 + 17, n_qk=1, n_v=1,
                           g_kind="strong", init=True, seed=56, d=64)),
    ("d64_gdn_tnd", dict(layout="TND", batch=3, seq_len=0, n_qk=1, n_v=2, g_kind="strong",
                         init=True, seed=57, lengths=[100, 64, 33], scalar_gate=True, d=64)),
]


# Few (sequence, head) chains and long enough sequences: the library runs the two-level scan
# (segments from zero and from the identity, then an affine combine); see kda_plan.cpp.
TWO_LEVEL = [
    ("bnsd_1head_41chunks_tail", dict(layout="BNSD", batch=1, seq_len=64 * 40 + 17, n_qk=1,
                                      n_v=1, g_kind="strong", init=True, seed=31)),
    ("bnsd_valid_lengths", dict(layout="BNSD", batch=2, seq_len=3000, n_qk=1, n_v=1,
                                g_kind="unit", init=True, seed=32, valid_lengths=[3000, 1300])),
    ("tnd_two_seqs", dict(layout="TND", batch=2, seq_len=0, n_qk=1, n_v=1, g_kind="small",
                          init=True, seed=33, lengths=[2100, 700])),
    ("bsnd_gqa", dict(layout="BSND", batch=1, seq_len=1600, n_qk=1, n_v=2, g_kind="mixed",
                      init=False, seed=34)),
    # the most segments (16: one head, 128 chunks) and two heads (8 segments)
    ("bnsd_1head_16seg", dict(layout="BNSD", batch=1, seq_len=8192, n_qk=1, n_v=1,
                              g_kind="strong", init=True, seed=35)),
    ("bnsd_2head_8seg", dict(layout="BNSD", batch=1, seq_len=4096 + 30, n_qk=2, n_v=2,
                             g_kind="small", init=True, seed=36)),
    # packed sequences of very different lengths: the short ones leave later segments empty
    # (their walks return at once, the combine meets identity transfers and zero end states)
    ("tnd_length_mix", dict(layout="TND", batch=5, seq_len=0, n_qk=1, n_v=1, g_kind="strong",
                            init=True, seed=37, lengths=[1, 5000, 64, 65, 700])),
]



# Shapes that make the plan select each kernel variant no other case reaches (the selection
# depends on the head dim, the number of (sequence, head) chains and of chunk records): the
# one-level scan at head dim 128 with two Dv tiles per workgroup, on the eight-wave walk with
# the prefetch wave (33-64 chains; the FlashKDA README's performance shapes have 24-48 heads)
# and on four waves without it (65-127 chains), the head-dim-64 scans above 64 chains, and the
# scalar-gate intra kernel in its four-wave form (more than 512 chunk records).  Each is
# compared in full.
VARIANT_CASES = [
    ("scan_2x128_pf8w_n48_gqa", dict(layout="BNSD", batch=1, seq_len=1100, n_qk=12, n_v=48,
                                g_kind="strong", init=True, seed=61)),
    ("scan_2x128_pf8w_b2_valid", dict(layout="BSND", batch=2, seq_len=700, n_qk=10, n_v=20,
                                      g_kind="strong", init=True, seed=69,
                                      valid_lengths=[700, 333])),
    ("scan_2x128_pf8w_tnd_40", dict(layout="TND", batch=4, seq_len=0, n_qk=5, n_v=10,
                                    g_kind="mixed", init=True, seed=70,
                                    lengths=[500, 64, 1, 300])),
    ("scan_2x128_b2_n48", dict(layout="BSND", batch=2, seq_len=600, n_qk=48, n_v=48,
                               g_kind="unit", init=True, seed=62)),
    ("scan_1x64_n96", dict(layout="BNSD", batch=1, seq_len=300, n_qk=96, n_v=96,
                           g_kind="strong", init=True, seed=63, d=64)),
    ("scan_2x64_pf_b2_n64", dict(layout="BNSD", batch=2, seq_len=200, n_qk=16, n_v=64,
                                 g_kind="mixed", init=False, seed=64, d=64)),
    ("scan_2x64_n160", dict(layout="TND", batch=2, seq_len=0, n_qk=40, n_v=80,
                            g_kind="strong", init=True, seed=65, lengths=[150, 77], d=64)),
    ("scan_4x64_b2_n128", dict(layout="BSND", batch=2, seq_len=130, n_qk=128, n_v=128,
                               g_kind="unit", init=True, seed=66, d=64)),
    ("intra4w_gdn_d128", dict(layout="BNSD", batch=1, seq_len=4160, n_qk=8, n_v=8,
                              g_kind="strong", init=True, seed=67, scalar_gate=True)),
    ("intra4w_gdn_d64", dict(layout="BSND", batch=1, seq_len=4160, n_qk=4, n_v=8,
                             g_kind="small", init=False, seed=68, scalar_gate=True, d=64)),
]


# The raw bf16 gate activated in the kernel (KDA_RAW_GATE; g, A_log, dt_bias ~ N(0,1) as in the
# FlashKDA README's quick start): every layout, GQA, ragged tails, valid lengths, head dim 64,
# the two-level scan, a lower bound other than -5, and the four-wave intra kernel (more than 512
# chunk records) at both head dims.
RAW_GATE_CASES = [
    ("raw_bnsd_b2_tail", dict(layout="BNSD", batch=2, seq_len=200, n_qk=2, n_v=2, init=True,
                              seed=91, raw_gate=True)),
    ("raw_bsnd_gqa_valid", dict(layout="BSND", batch=2, seq_len=150, n_qk=1, n_v=4, init=False,
                                seed=92, valid_lengths=[150, 61], raw_gate=True)),
    ("raw_tnd_ragged", dict(layout="TND", batch=4, seq_len=0, n_qk=2, n_v=2, init=True, seed=93,
                            lengths=[1, 64, 130, 17], raw_gate=True, lower_bound=-1.5)),
    ("raw_two_level", dict(layout="BNSD", batch=1, seq_len=64 * 40 + 5, n_qk=1, n_v=1,
                           init=True, seed=94, raw_gate=True)),
    ("raw_d64_bsnd", dict(layout="BSND", batch=2, seq_len=100, n_qk=2, n_v=4, init=True,
                          seed=95, raw_gate=True, d=64)),
    ("raw_intra4w_d128", dict(layout="BNSD", batch=1, seq_len=4160, n_qk=8, n_v=8, init=True,
                              seed=96, raw_gate=True)),
    ("raw_intra4w_d64", dict(layout="TND", batch=2, seq_len=0, n_qk=4, n_v=8, init=False,
                             seed=97, lengths=[2100, 2060], raw_gate=True, d=64)),
]


def case_shape(kw: dict, flags_on: bool = True):
    """The library shape of a make_inputs case (no tensors drawn)."""
    layout = kw["layout"]
    seq_len = sum(kw["lengths"]) if layout == "TND" else kw["seq_len"]
    d = kw.get("d", 128)
    return make_shape(layout, kw["batch"], seq_len, kw["n_qk"], kw["n_v"], d ** -0.5,
                      flags_on, flags_on, d, d, kw.get("scalar_gate", False),
                      raw_gate=kw.get("raw_gate", False))


def all_case_shapes() -> list:
    """(name, shape) of every fixed GPU parity case, the named workloads and the sweep."""
    from test_gpu_sweep import CASES as SWEEP
    out = []
    for group in (SMALL, SCALAR_GATE_CASES, D64_CASES, TWO_LEVEL, VARIANT_CASES, RAW_GATE_CASES,
                  NO_DECAY_CASES):
        out += [(name, case_shape(kw)) for name, kw in group]
    out += [(name, case_shape(kw, flags_on)) for name, kw, flags_on in SWEEP]
    for w in WORKLOADS:
        out.append((w.name, case_shape(workload_shape(w))))
    return out
