"""Row groups (two workgroups per split and KV head, each taking half the
16-row blocks) change no bit of the result: the same problem planned with
room for twice the workgroups (row groups 2) and without it (1), at the same
forced split count, gives bit-identical partials, outputs and lse, for bf16
and quantised tree caches, the device-state split and the fused append.  The
oracle parity of these shapes is covered by the tree tests; this pins the
row-group launch to the one-group launch."""
import math

import numpy as np
import pytest
import torch

import speculative_decode_verify_amd as va
from speculative_decode_verify_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAN = float("nan")
ROWS, HQ, HKV, D, P, S = 16, 24, 4, 128, 2048, 16


def _plans(num_cus_pair=(256, 64), **kw):
    plans = [va.Plan(rows=ROWS, live_rows=kw.pop("live", ROWS), q_heads=HQ, kv_heads=HKV, head_dim=D, mask="tree",
                     prefix_len=P, splits=S, scale=1 / math.sqrt(D), num_cus=n, **kw) for n in num_cus_pair]
    assert [p.info["row_groups"] for p in plans] == [2, 1]
    return plans


def _bufs(plan):
    ws = torch.full(((plan.workspace_bytes + 3) // 4,), NAN, dtype=torch.float32, device=DEV)
    out = torch.full((plan.rows, plan.q_heads, plan.head_dim), NAN, dtype=torch.float32, device=DEV)
    lse = torch.full((plan.rows, plan.q_heads), NAN, dtype=torch.float32, device=DEV)
    return ws, out, lse


def _live_units(plan, ws, live):
    """The workspace entries the split writes: {m, l} and O of live rows."""
    G = HQ // HKV
    n = plan.splits * HKV * ROWS * G
    ml_floats = ((n * 8 + 255) // 256 * 256) // 4
    flat = ws.cpu()
    ml = flat[:n * 2].view(plan.splits, HKV, ROWS * G, 2)[:, :, :live * G]
    o = flat[ml_floats:ml_floats + n * D].view(plan.splits, HKV, ROWS * G, D)[:, :, :live * G]
    return ml.contiguous().view(torch.int32), o.contiguous().view(torch.int32)


def _same(a, b, live, what):
    (wa, oa, la, pa), (wb, ob, lb, pb) = a, b
    mla, Oa = _live_units(pa, wa, live)
    mlb, Ob = _live_units(pb, wb, live)
    assert torch.equal(mla, mlb), f"{what}: (m, l) partials differ"
    assert torch.equal(Oa, Ob), f"{what}: O partials differ"
    assert torch.equal(oa.cpu().view(torch.int32), ob.cpu().view(torch.int32)), f"{what}: outputs differ"
    assert torch.equal(la.cpu().view(torch.int32), lb.cpu().view(torch.int32)), f"{what}: lse differs"


def _tree_inputs(seed, quant):
    g = synth.gen(seed)
    parent = synth.random_tree(ROWS, g)
    cap = P + ROWS + 64
    q = synth.normal_bf16((ROWS, HQ, D), g).to(DEV)
    if quant:
        k = torch.randint(0, 0x7F, (HKV, cap, D), dtype=torch.uint8, generator=g)  # no NaN code
        k |= torch.randint(0, 2, (HKV, cap, D), dtype=torch.uint8, generator=g) << 7
        v = torch.randint(-127, 128, (HKV, cap, D), dtype=torch.int8, generator=g)
        vs = (torch.rand((HKV, cap), generator=g) * 0.02).to(DEV)
    else:
        k = synth.normal_bf16((HKV, cap, D), g)
        v = synth.normal_bf16((HKV, cap, D), g)
        vs = None
    sink = synth.normal_f32((HQ,), g).to(DEV)
    return parent, cap, q, k.to(DEV), v.to(DEV), vs, sink


@pytest.mark.parametrize("quant", [False, True], ids=["bf16", "e4m3-int8"])
def test_row_groups_static_bit_identical(quant):
    parent, cap, q, k, v, vs, sink = _tree_inputs(31000 + quant, quant)
    plans = _plans(parent=parent, kv_capacity=cap, kv_fmt="e4m3_wht_i8" if quant else "bf16")
    res = []
    for plan in plans:
        ws, out, lse = _bufs(plan)
        va.verify_attn_split(plan, q, k, v, ws, v_scale=vs)
        va.verify_attn_combine(plan, ws, out, lse=lse, sink=sink)
        torch.cuda.synchronize()
        res.append((ws, out, lse, plan))
    _same(res[0], res[1], ROWS, "static")


def test_row_groups_state_bit_identical():
    """Device-state split: a state with 11 live nodes at a shorter prefix
    than the bucket, both launches reading it from device memory."""
    parent, cap, q, k, v, _, sink = _tree_inputs(31100, False)
    plans = _plans(parent=parent, kv_capacity=cap)
    st = va.pack_state(prefix_len=P - 700, live_rows=11, parent=parent).to(DEV)
    res = []
    for plan in plans:
        ws, out, lse = _bufs(plan)
        va.verify_attn_split_state(plan, st, q, k, v, ws)
        va.verify_attn_combine_state(plan, st, ws, out, lse=lse, sink=sink)
        torch.cuda.synchronize()
        res.append((ws, out, lse, plan))
    _same(res[0], res[1], 11, "state")


def test_row_groups_append_bit_identical():
    """Fused append: the tree nodes' K/V written by the split itself (once,
    by the first row group) and read from the staged tiles."""
    parent, cap, q, k0, v0, _, sink = _tree_inputs(31200, False)
    g = synth.gen(31201)
    k_new = synth.normal_bf16((ROWS, HKV, D), g).to(DEV)
    v_new = synth.normal_bf16((ROWS, HKV, D), g).to(DEV)
    plans = _plans(parent=parent, kv_capacity=cap)
    res, caches = [], []
    for plan in plans:
        k, v = k0.clone(), v0.clone()
        k[:, P:P + ROWS] = NAN  # the rows' slots hold stale data before the call
        v[:, P:P + ROWS] = NAN
        ws, out, lse = _bufs(plan)
        va.verify_attn_split_append(plan, q, k_new, v_new, k, v, ws)
        va.verify_attn_combine(plan, ws, out, lse=lse, sink=sink)
        torch.cuda.synchronize()
        res.append((ws, out, lse, plan))
        caches.append((k, v))
    _same(res[0], res[1], ROWS, "append")
    for k, v in caches:
        assert torch.equal(k[:, P:P + ROWS].cpu(), k_new.transpose(0, 1).cpu()), "appended keys"
        assert torch.equal(v[:, P:P + ROWS].cpu(), v_new.transpose(0, 1).cpu()), "appended values"
    assert torch.equal(caches[0][0].cpu().view(torch.int16), caches[1][0].cpu().view(torch.int16))
