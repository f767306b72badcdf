"""verify_attn_noalloc: split + combine with the library's static per-GPU
workspace, for callers that cannot allocate.

Gates: two calls in a row (the second with a smaller problem, so the array
still holds the first call's partials beyond what the second reads), each
bit-identical to verify_attn_split + verify_attn_combine with a caller
workspace on the same inputs, and within the graded gate of the float64
oracle; a third call on a quantised tree; a plan whose workspace exceeds the
array is refused before any launch.
"""
import math

import numpy as np
import pytest
import torch

import speculative_decode_verify_amd as va
from speculative_decode_verify_amd import synth
from oracle import attn as oattn
from oracle import codec as ocodec
from oracle.masks import Problem
from test_gpu_parity import NAN, check, f64, plan_for, run

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _noalloc(plan, q, k, v, sink=None, v_scale=None):
    out = torch.full((plan.rows, plan.q_heads, plan.head_dim), NAN, dtype=torch.float32, device=DEV)
    lse = torch.full((plan.rows, plan.q_heads), NAN, dtype=torch.float32, device=DEV)
    va.verify_attn_noalloc(plan, q, k, v, out, lse=lse, sink=sink, v_scale=v_scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _causal(seed, rows, live, Hq, Hkv, D, P, splits=0):
    g = synth.gen(seed)
    cap = P + rows + 64
    q = synth.normal_bf16((rows, Hq, D), g)
    k = synth.normal_bf16((Hkv, cap, D), g)
    v = synth.normal_bf16((Hkv, cap, D), g)
    k[:, P + live:] = NAN
    v[:, P + live:] = NAN
    s = synth.normal_f32((Hq,), g)
    plan = plan_for(rows, live, Hq, Hkv, D, "causal", first_pos=P, kv_capacity=cap, splits=splits,
                    scale=1 / math.sqrt(D))
    return plan, q, k, v, s


def _same_as_workspace_path(plan, q, k, v, s, live, name, v_scale=None):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    sd = None if s is None else s.to(DEV)
    vsd = None if v_scale is None else v_scale.to(DEV)
    o_n, l_n = _noalloc(plan, qd, kd, vd, sd, vsd)
    o_w, l_w, _ = run(plan, qd, kd, vd, sd, vsd)
    assert torch.equal(o_n.view(torch.int32), o_w.view(torch.int32)), f"{name}: out differs"
    assert torch.equal(l_n.view(torch.int32), l_w.view(torch.int32)), f"{name}: lse differs"
    assert torch.all(o_n[live:] == 0), f"{name}: padding rows"
    return o_n, l_n


def test_noalloc_two_calls_then_smaller():
    # 1: 64K context, 256 plan-chosen splits (6.4 MB of partials)
    plan, q, k, v, s = _causal(17001, 8, 7, 6, 1, 128, 65536)
    assert plan.splits == 256 and plan.workspace_bytes <= va.NOALLOC_WORKSPACE_BYTES
    o, l = _same_as_workspace_path(plan, q, k, v, s, 7, "64K")
    p = Problem("causal", 8, 7, first_pos=65536)
    ro, rl = oattn.verify_attn_ref(p, f64(q), oattn.Cache(f64(k[:, :65543]), f64(v[:, :65543])),
                                   plan.problem.scale, f64(s))
    check(o, l, ro, rl, 7, "noalloc 64K")
    # 2: a smaller problem right after (config-1 shape, 4 splits)
    plan2, q2, k2, v2, s2 = _causal(17002, 8, 5, 6, 1, 64, 1019, splits=4)
    o2, l2 = _same_as_workspace_path(plan2, q2, k2, v2, s2, 5, "1K")
    p2 = Problem("causal", 8, 5, first_pos=1019)
    ro2, rl2 = oattn.verify_attn_ref(p2, f64(q2), oattn.Cache(f64(k2[:, :1024]), f64(v2[:, :1024])),
                                     plan2.problem.scale, f64(s2))
    check(o2, l2, ro2, rl2, 5, "noalloc 1K")


def test_noalloc_quantised_tree():
    rows, live, Hq, Hkv, D, P = 16, 16, 24, 4, 128, 8192
    g = synth.gen(17003)
    parent = synth.random_tree(rows, g)
    cap = P + rows + 64
    hi = P + live
    q = synth.normal_bf16((rows, Hq, D), g)
    k_codes = ocodec.e4m3_encode(ocodec.wht(synth.normal_f32((Hkv, hi, D), g).double().numpy()))
    v_codes, v_sc = ocodec.i8_encode(synth.normal_f32((Hkv, hi, D), g).double().numpy())
    k8 = torch.full((Hkv, cap, D), 0x7F, dtype=torch.uint8)
    v8 = torch.zeros((Hkv, cap, D), dtype=torch.int8)
    vs = torch.full((Hkv, cap), NAN, dtype=torch.float32)
    k8[:, :hi] = torch.from_numpy(k_codes)
    v8[:, :hi] = torch.from_numpy(v_codes)
    vs[:, :hi] = torch.from_numpy(v_sc)
    plan = plan_for(rows, live, Hq, Hkv, D, "tree", kv_fmt="e4m3_wht_i8", prefix_len=P, parent=parent,
                    kv_capacity=cap, scale=1 / math.sqrt(D))
    _same_as_workspace_path(plan, q, k8, v8, None, live, "quantised tree", v_scale=vs)


def test_noalloc_refuses_a_workspace_beyond_the_array():
    plan, q, k, v, s = _causal(17004, 8, 8, 6, 1, 128, 65536, splits=2048)
    assert plan.workspace_bytes > va.NOALLOC_WORKSPACE_BYTES
    out = torch.empty((8, 6, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(va.VAError):
        va.verify_attn_noalloc(plan, q.to(DEV), k.to(DEV), v.to(DEV), out)
    torch.cuda.synchronize()
