"""The trace build of the library (lib/libverify_attn_trace.so, the same
sources with per-workgroup phase stamps; include/verify_probe.h).

Gates: its outputs, lse and partials equal the product library's bit for bit
on the same inputs (the stamps change no arithmetic), and every record of
the launch is ordered as the phases run: split entry <= arguments <= chunk 0
in LDS <= last step <= partials written, the first DMA issued (by another
wave) before chunk 0 is in LDS, each workgroup's chunk count equal to the
plan's split table and its barrier time within its steps' span, every
role's waits (consumers at barriers; first producer for DMA and at
barriers; first decoder at barriers and converting) within that span and
wave 0's equal to slot 6; combine
entry <= arguments <= first batch <= fold <= output written for every live
row, after the split's last partial.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import speculative_decode_verify_amd as va
import speculative_decode_verify_amd._binding as binding
from speculative_decode_verify_amd import synth
from test_gpu_parity import NAN, plan_for, run

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _trace_lib():
    product = binding.load_library()
    binding._LIB = None
    saved = binding._LIB_PATH
    binding._LIB_PATH = binding.trace_library_path()
    try:
        lib = binding.load_library()
    finally:
        binding._LIB_PATH = saved
        binding._LIB = product
    lib.va_trace_read.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
    return product, lib


def _records(lib, which, n):
    buf = np.zeros((n, 24 if which == 0 else 8), dtype=np.uint64)
    assert lib.va_trace_read(which, buf.ctypes.data, n) == 0
    return buf.astype(np.int64)


def _inputs(case):
    g = synth.gen(7100 + case)
    if case == 0:  # causal, 48 rows, 64 splits over 4K keys
        rows, live, Hq, Hkv, D, P = 8, 5, 6, 1, 128, 4096
        cap = P + rows + 64
        plan = plan_for(rows, live, Hq, Hkv, D, "causal", first_pos=P, kv_capacity=cap, scale=1 / math.sqrt(D))
        q = synth.normal_bf16((rows, Hq, D), g)
        k = synth.normal_bf16((Hkv, cap, D), g)
        v = synth.normal_bf16((Hkv, cap, D), g)
        return plan, q, k, v, synth.normal_f32((Hq,), g), None, live
    # quantised tree over 4K keys: 16 nodes, 4 KV heads, 24 query heads
    rows, Hq, Hkv, D, P = 16, 24, 4, 128, 4096
    cap = P + rows + 64
    plan = plan_for(rows, rows, Hq, Hkv, D, "tree", kv_fmt="e4m3_wht_i8", prefix_len=P,
                    parent=synth.random_tree(rows, g), kv_capacity=cap, scale=1 / math.sqrt(D))
    q = synth.normal_bf16((rows, Hq, D), g)
    k = torch.randint(0, 0x40, (Hkv, cap, D), dtype=torch.uint8, generator=g)
    k |= (torch.randint(0, 2, (Hkv, cap, D), dtype=torch.uint8, generator=g) << 7)
    v = torch.randint(-127, 128, (Hkv, cap, D), dtype=torch.int8, generator=g)
    vs = torch.rand((Hkv, cap), generator=g) * 0.02
    return plan, q, k, v, None, vs, rows


@pytest.mark.parametrize("case", [0, 1], ids=["causal-4K", "quantised-tree-4K"])
def test_trace_build_matches_product_and_orders_phases(case):
    plan, q, k, v, sink, vs, live = _inputs(case)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    sd = None if sink is None else sink.to(DEV)
    vsd = None if vs is None else vs.to(DEV)
    product, lib = _trace_lib()
    o_p, l_p, ws_p = run(plan, qd, kd, vd, sd, vsd)
    binding._LIB = lib
    try:
        o_t, l_t, ws_t = run(plan, qd, kd, vd, sd, vsd)
        n_split = plan.splits * plan.kv_heads * plan.info["row_groups"]
        n_comb = plan.rows * plan.q_heads * (plan.head_dim // 32)
        sp = _records(lib, 0, n_split)
        cb = _records(lib, 1, n_comb)
    finally:
        binding._LIB = product
    assert torch.equal(o_t.view(torch.int32), o_p.view(torch.int32)), "outputs differ"
    assert torch.equal(l_t.view(torch.int32), l_p.view(torch.int32)), "lse differs"
    nws = (plan.workspace_bytes + 3) // 4
    assert torch.equal(ws_t[:nws].view(torch.int32), ws_p[:nws].view(torch.int32)), "partials differ"

    # split records: the split table's chunk counts and ordered phases
    S = plan.splits
    C = plan.info["chunks"]
    want_nch = np.array([C // S + (1 if s < C % S else 0) for s in range(S)] * plan.kv_heads * plan.info["row_groups"])
    assert np.array_equal(sp[:, 7], want_nch)
    busy = sp[:, 7] > 0
    assert busy.any()
    e, a, dma, c0, last, wr, bar = (sp[busy, i] for i in (0, 1, 2, 3, 4, 5, 6))
    assert np.all(e <= a) and np.all(a <= c0) and np.all(dma <= c0)
    assert np.all(c0 <= last) and np.all(last <= wr)
    assert np.all((bar >= 0) & (bar <= last - c0))
    # each role's time at the later barriers (a duration inside the steps'
    # span); consumer wave 0's is the one already checked
    W = -(-plan.rows * (plan.q_heads // plan.kv_heads) // (16 * plan.info["row_groups"]))
    roles = [8 + w for w in range(W)] + [14, 15] + ([16, 17] if case == 1 else [])
    span = (wr - e)[:, None]
    waits = sp[busy][:, roles]
    assert np.array_equal(sp[busy, 8], bar)
    assert np.all((waits >= 0) & (waits <= span)), waits.max(axis=0)
    span_us = (wr.max() - e.min()) * 0.01
    assert 0 < span_us < 1000, span_us

    # combine records of the live rows
    # record index h + Hq * (row * D/32 + d slice)
    row = (np.arange(n_comb) // plan.q_heads) // (plan.head_dim // 32)
    c = cb[row < live]
    assert np.all(c[:, 0] <= c[:, 1]) and np.all(c[:, 1] <= c[:, 2])
    assert np.all(c[:, 2] <= c[:, 3]) and np.all(c[:, 3] <= c[:, 4])
    # the combine starts after the split's partials are written
    assert c[:, 0].min() >= wr.max()
