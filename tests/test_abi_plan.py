"""CPU tests of the C ABI: the library loads, exports every declared entry
point, rejects every malformed problem, and its host plan agrees bit-exactly
with the oracle's visibility rules and split rule.  No kernel is launched."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import speculative_decode_verify_amd as va
from speculative_decode_verify_amd import _binding
from oracle import masks
from oracle.masks import Problem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)) - {"sizeof"})


# declared in include/verify_probe.h for the trace build of the library only
TRACE_ONLY = {"va_trace_read"}


def test_library_exports_every_declared_symbol():
    lib = va.load_library()
    names = declared_functions()
    assert set(names) >= {"verify_attn_plan", "verify_attn_split", "verify_attn_combine", "swa_ring_write", "verify_kv_write",
                          "verify_attn_split_state", "verify_attn_combine_state",
                          "va_sample", "va_accept", "va_sample_accept", "va_sample_workspace_bytes", "va_read_probe",
                          "verify_attn_plan_query", "verify_attn_plan_split_range", "va_status_string"}
    assert TRACE_ONLY <= set(names)
    for n in names:
        if n in TRACE_ONLY:
            assert not hasattr(lib, n), f"{n}: the product library carries no trace code"
            continue
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_trace_build_exports_every_declared_symbol():
    path = _binding.trace_library_path()
    assert os.path.exists(path), "build() makes the trace library beside the product one"
    lib = ctypes.CDLL(path)
    for n in declared_functions():
        assert hasattr(lib, n), n
    lib.va_trace_read.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
    buf = (ctypes.c_uint64 * 8)()
    assert lib.va_trace_read(2, buf, 1) == 1          # which must be 0 or 1
    assert lib.va_trace_read(0, None, 1) == 1         # no destination
    assert lib.va_trace_read(0, buf, 8193) == 1       # more records than kept


def test_status_strings():
    lib = va.load_library()
    for s in range(6):
        assert lib.va_status_string(s)
    assert b"unknown" in lib.va_status_string(99)


def test_struct_sizes_match_c_layout():
    # va_problem: eleven int32, int32[16], (pad), three int64, float, int32
    assert ctypes.sizeof(_binding.va_problem) == 144
    assert ctypes.sizeof(_binding.va_plan) == 2048
    # va_plan_info: two int32, four int64, int64[16] x 2, uint32[16], size_t,
    # int32 (+ tail padding)
    assert ctypes.sizeof(_binding.va_plan_info) == 8 + 32 + 256 + 64 + 8 + 8


def _status(**kw):
    try:
        va.Plan(**kw)
    except va.VAError as e:
        return _binding.STATUS[e.status]
    return "VA_OK"


BASE = dict(rows=8, live_rows=5, q_heads=6, kv_heads=1, head_dim=64, first_pos=1019, kv_capacity=1032)


@pytest.mark.parametrize("change,expect", [
    (dict(), "VA_OK"),
    (dict(rows=0), "VA_ERR_INVALID"),
    (dict(rows=17), "VA_ERR_INVALID"),
    (dict(live_rows=9), "VA_ERR_INVALID"),
    (dict(live_rows=-1), "VA_ERR_INVALID"),
    (dict(q_heads=6, kv_heads=4), "VA_ERR_INVALID"),                     # 6 % 4 != 0
    (dict(q_heads=7), "VA_OK"),                                           # G = 7, 56 matrix rows
    (dict(kv_heads=0), "VA_ERR_INVALID"),
    (dict(head_dim=96), "VA_ERR_UNSUPPORTED"),
    (dict(q_heads=13, kv_heads=1, rows=8), "VA_ERR_UNSUPPORTED"),          # 8 * 13 > 96 rows
    (dict(kv_fmt="e4m3_wht_i8"), "VA_ERR_UNSUPPORTED"),                  # quantised needs D = 128
    (dict(scale=0.0), "VA_ERR_INVALID"),
    (dict(scale=float("nan")), "VA_ERR_INVALID"),
    (dict(scale=float("inf")), "VA_ERR_INVALID"),
    (dict(first_pos=-1), "VA_ERR_INVALID"),
    (dict(kv_capacity=1023), "VA_ERR_CAPACITY"),                          # live rows read up to 1023
    (dict(kv_capacity=1024), "VA_OK"),
    (dict(splits=-2), "VA_ERR_INVALID"),
    (dict(mask=7), "VA_ERR_INVALID"),
    (dict(ring_slots=4160), "VA_ERR_INVALID"),                            # ring only in window mode
    (dict(mask="window", window=4096, ring_slots=4160), "VA_OK"),
    (dict(mask="window", window=4096, ring_slots=4096), "VA_ERR_INVALID"),  # the rows' writes would evict
    (dict(mask="window", window=4096, ring_slots=4100), "VA_ERR_INVALID"),  # not a multiple of 64
    (dict(mask="window", window=0, ring_slots=4160), "VA_ERR_INVALID"),
    (dict(mask="window", window=57, ring_slots=64), "VA_OK"),             # 57 + 8 - 1 = 64
    (dict(mask="window", window=58, ring_slots=64), "VA_ERR_INVALID"),
    (dict(mask="tree", prefix_len=100, parent=[-1, 0, 5], rows=3, live_rows=3), "VA_ERR_INVALID"),
    (dict(mask="tree", prefix_len=100, parent=[-1, 0, -2], rows=3, live_rows=3), "VA_ERR_INVALID"),
    (dict(mask="tree", prefix_len=100, parent=[0, 0, 1], rows=3, live_rows=3), "VA_ERR_INVALID"),
    (dict(mask="tree", prefix_len=100, parent=[-1, 0, 1], rows=3, live_rows=3, kv_capacity=103), "VA_OK"),
    (dict(mask="tree", prefix_len=100, parent=[-1, 0, 1], rows=3, live_rows=3, kv_capacity=102), "VA_ERR_CAPACITY"),
    (dict(mask="tree", prefix_len=-1, parent=[-1], rows=1, live_rows=1), "VA_ERR_INVALID"),
])
def test_plan_validation(change, expect):
    kw = dict(BASE)
    kw.update(change)
    assert _status(**kw) == expect


def test_reserved_must_be_zero():
    lib = va.load_library()
    p = _binding.va_problem()
    p.rows, p.live_rows, p.q_heads, p.kv_heads, p.head_dim, p.kv_capacity, p.scale = 8, 1, 6, 1, 64, 100, 1.0
    plan = _binding.va_plan()
    assert lib.verify_attn_plan(ctypes.byref(p), ctypes.byref(plan), None) == 0
    p.reserved = 1
    assert lib.verify_attn_plan(ctypes.byref(p), ctypes.byref(plan), None) == 1
    assert lib.verify_attn_plan(None, ctypes.byref(plan), None) == 1


def test_query_rejects_garbage_plan():
    lib = va.load_library()
    plan = _binding.va_plan()
    info = _binding.va_plan_info()
    assert lib.verify_attn_plan_query(ctypes.byref(plan), ctypes.byref(info)) == 1


def test_append_refusals_before_any_launch():
    """verify_attn_split_append checks its plan and buffers on the host: a
    quantised cache is unsupported, missing new rows are invalid, and a
    linear cache (or tree) without room for every row is a capacity error;
    none of these reaches the GPU."""
    lib = va.load_library()
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every case fails before use

    def call(plan, k_new=fake):
        return lib.verify_attn_split_append(ctypes.byref(plan.plan), fake, k_new, fake, fake, fake, 0, 128,
                                            fake, plan.workspace_bytes, None)

    quant = va.Plan(rows=8, live_rows=8, q_heads=6, kv_heads=1, head_dim=128, kv_fmt="e4m3_wht_i8",
                    first_pos=500, kv_capacity=600)
    assert call(quant) == 2
    ok = va.Plan(rows=8, live_rows=8, q_heads=6, kv_heads=1, head_dim=128, first_pos=500, kv_capacity=600)
    assert call(ok, k_new=None) == 1
    short = va.Plan(rows=8, live_rows=4, q_heads=6, kv_heads=1, head_dim=128, first_pos=500, kv_capacity=506)
    assert call(short) == 3
    tree = va.Plan(rows=16, live_rows=8, q_heads=6, kv_heads=1, head_dim=128, mask="tree", prefix_len=500,
                   parent=[-1] * 16, kv_capacity=510)
    assert call(tree) == 3


def _oracle_problem(kw):
    return Problem(kw.get("mask", "causal"), kw["rows"], kw["live_rows"], first_pos=kw.get("first_pos", 0),
                   prefix_len=kw.get("prefix_len", 0), parent=kw.get("parent"), window=kw.get("window", 0),
                   ring_slots=kw.get("ring_slots", 0))


def _cases():
    rng = np.random.default_rng(7)
    out = []
    for P in (0, 1, 63, 64, 1019, 5000, 65536 + 17):
        for live in (0, 1, 5, 8):
            out.append(dict(rows=8, live_rows=live, q_heads=6, kv_heads=1, head_dim=128, first_pos=P,
                            kv_capacity=P + 8))
    for t0 in (0, 5, 4095, 5120, 51200, 194560):
        for live in (1, 5, 8):
            out.append(dict(rows=8, live_rows=live, q_heads=6, kv_heads=1, head_dim=64, mask="window",
                            window=4096, ring_slots=4160, first_pos=t0))
    for P in (0, 10, 2048, 8192, 32768):
        for _ in range(3):
            par = [-1] + [int(rng.integers(-1, i)) for i in range(1, 16)]
            out.append(dict(rows=16, live_rows=16, q_heads=24, kv_heads=4, head_dim=128, mask="tree",
                            prefix_len=P, parent=par, kv_capacity=P + 16))
    return out


@pytest.mark.parametrize("kw", _cases())
def test_plan_matches_oracle_geometry(kw):
    plan = va.Plan(**kw)
    info = plan.info
    p = _oracle_problem(kw)
    lo, hi = masks.union_extent_fast(p)
    assert (info["lo"], info["hi"]) == (lo, hi)
    if hi - lo < 20000:
        assert masks.union_extent(p) == (lo, hi)
    if kw.get("mask") == "tree":
        anc = masks.tree_ancestors(p.parent)
        for r in range(16):
            assert info["anc"][r] == (anc[r] if r < p.live_rows else 0)
    # per-row visible sets from the plan equal the oracle's, position by position
    span_lo = max(0, lo - 70)
    span_hi = hi + 70
    vm = masks.visible_matrix(p, span_lo, span_hi)
    j = np.arange(span_lo, span_hi)
    for r in range(kw["rows"]):
        mine = (j >= info["row_lo"][r]) & (j < info["row_hi"][r])
        if kw.get("mask") == "tree":
            i = j - kw["prefix_len"]
            mine |= (i >= 0) & (i < 16) & ((np.int64(info["anc"][r]) >> np.clip(i, 0, 15)) & 1 == 1)
        if r >= kw["live_rows"]:
            assert not mine.any()
        assert np.array_equal(mine, vm[r]), r
    # split table equals the oracle's rule for the plan's own count and for others
    for S in sorted({plan.splits, 1, 3, 8, 64}):
        kw2 = dict(kw)
        kw2["splits"] = S
        plan2 = va.Plan(**kw2)
        got = [va.verify_attn_plan_split_range(plan2, s) for s in range(S)]
        exp = masks.split_key_ranges(lo, hi, S)
        exp = [(a, b) if b > a else None for a, b in exp]
        got = [(a, b) if b > a else None for a, b in got]
        assert got == exp


def test_workspace_size_formula():
    plan = va.Plan(rows=16, live_rows=16, q_heads=24, kv_heads=4, head_dim=128, mask="tree", prefix_len=2048,
                   parent=[-1] * 16, kv_capacity=2064, splits=10)
    units = 10 * 4 * 96
    ml = (units * 8 + 255) // 256 * 256
    assert plan.workspace_bytes == ml + units * 128 * 4


def test_chosen_splits_are_sane():
    """The plan's split count: about 6.9 * sqrt(C * B_granule / (B_partial *
    Hkv)) rounded to a multiple of 8, or one 32-key granule per split where
    that comes within a quarter of the granule count; at most one workgroup
    per CU over the KV heads (a multiple of 8) and at most one split per
    granule.  The counts are written out for the measured shapes and the
    rule is recomputed here in floating point for the sweep."""
    want = {1024: 33, 4096: 64, 16384: 128, 32768: 176, 65536: 256, 131072: 256, 196608: 256}
    for P, S_want in want.items():
        plan = va.Plan(rows=8, live_rows=8, q_heads=6, kv_heads=1, head_dim=128, first_pos=P,
                       kv_capacity=262144, num_cus=256)
        S, C = plan.splits, plan.info["chunks"]
        assert S == S_want, (P, S)
        assert 1 <= S <= min(C, 256) and (S == C or S % 8 == 0)
        fit = round(6.9 * math.sqrt(C * (32 * 4 * 128) / (48 * 130 * 4)))
        expect = C if 4 * fit >= 3 * C else ((fit + 4) // 8) * 8
        assert S == min(expect, 256, C), (P, S, expect)
    for t0 in (5120, 51200, 194560):  # window ring, D 64: 129 granules
        plan = va.Plan(rows=8, live_rows=5, q_heads=6, kv_heads=1, head_dim=64, mask="window", first_pos=t0,
                       window=4096, ring_slots=4160, num_cus=256)
        assert plan.info["chunks"] == 129 and plan.splits == 64, (t0, plan.splits)
    for P, S_want in {2048: 16, 8192: 32, 32768: 64}.items():
        plan = va.Plan(rows=16, live_rows=16, q_heads=24, kv_heads=4, head_dim=128, mask="tree", prefix_len=P,
                       parent=[-1] * 16, kv_capacity=P + 100, num_cus=256)
        assert plan.splits == S_want, (P, plan.splits)
    plan = va.Plan(rows=16, live_rows=16, q_heads=24, kv_heads=4, head_dim=128, mask="tree", prefix_len=65536,
                   parent=[-1] * 16, kv_capacity=65536 + 100, kv_fmt="e4m3_wht_i8", num_cus=256)
    assert plan.splits == 64
    # a few granules: one split each; the CU cap over KV heads
    plan = va.Plan(rows=1, live_rows=1, q_heads=1, kv_heads=1, head_dim=64, first_pos=40, kv_capacity=64,
                   num_cus=256)
    assert plan.splits == plan.info["chunks"] == 2
    plan = va.Plan(rows=16, live_rows=16, q_heads=24, kv_heads=4, head_dim=128, mask="tree", prefix_len=200000,
                   parent=[-1] * 16, kv_capacity=200100, num_cus=40)
    assert plan.splits == 8


def test_row_groups_rule():
    """Two workgroups per (split, KV head) exactly when the matrix rows fill
    more than four 16-row blocks and twice the workgroups fit one per CU:
    the 16-node tree over four KV heads at 2K and 8K keys (16 and 32
    splits), not at 32K (64 splits) or for the 48-row sweep."""
    def tree(P, num_cus=256, live=16, rows=16, q_heads=24, fmt="bf16"):
        return va.Plan(rows=rows, live_rows=live, q_heads=q_heads, kv_heads=4, head_dim=128, mask="tree",
                       prefix_len=P, parent=[-1] * rows, kv_capacity=P + 100, num_cus=num_cus, kv_fmt=fmt)
    for P, want in ((2048, 2), (8192, 2), (32768, 1)):
        plan = tree(P)
        assert plan.info["row_groups"] == want, (P, plan.splits, plan.info["row_groups"])
        assert (2 * plan.splits * 4 <= 256) == (want == 2)
    assert tree(8192, num_cus=128).info["row_groups"] == 1  # 2 * 32 * 4 > 128
    assert tree(2048, fmt="e4m3_wht_i8").info["row_groups"] == 2
    # 80 matrix rows (five blocks) qualify, 64 (four blocks) do not
    assert tree(2048, rows=16, q_heads=20).info["row_groups"] == 2
    assert tree(2048, rows=16, q_heads=16).info["row_groups"] == 1
    for P in (1024, 16384, 196608):
        plan = va.Plan(rows=8, live_rows=8, q_heads=6, kv_heads=1, head_dim=128, first_pos=P,
                       kv_capacity=262144, num_cus=256)
        assert plan.info["row_groups"] == 1
    # the workspace does not depend on the row groups
    plan = tree(2048)
    units = plan.splits * 4 * 96
    assert plan.workspace_bytes == (units * 8 + 255) // 256 * 256 + units * 128 * 4
