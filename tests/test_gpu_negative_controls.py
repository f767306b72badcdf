"""Negative controls through the C ABI: valid calls with deliberately wrong
inputs, each asserted to fail the gate that is meant to catch that class of
mistake, beside the same call with the right inputs passing it.  No kernel
is altered; only the plan, the sink, the parents or the workspace handed to
the library are wrong.

Controls (IQuestRT report, "Let correctness checks change the design": a
check is trusted once a planted defect is shown to fail it):
* a causal plan one position late (first_pos + 1) fails the counting test
  against the oracle at first_pos;
* a window one key wider fails the counting test;
* a combine without the sink fails the q = 0 closed form with the sink;
* one split's partials overwritten with another's before the combine fail
  the LSE gate;
* a parent array that makes a non-ancestor visible fails the spike test.
"""
import math

import numpy as np
import pytest
import torch

import speculative_decode_verify_amd as va
from speculative_decode_verify_amd import synth
from oracle import attn as oattn
from oracle import masks as omasks
from oracle.masks import Problem
from test_gpu_parity import NAN, check, f64, gpu_and_oracle, partials, plan_for, run

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _labels(Hkv, n, D):
    return synth.position_labels(torch.arange(n), D).to(torch.bfloat16).unsqueeze(0).repeat(Hkv, 1, 1)


def _counting_gate(plan, p_oracle, k, v, D):
    """q = 0 counting test: the GPU partials of `plan` against the oracle's
    split form for problem `p_oracle` with the same split count (exact)."""
    rows, Hq = plan.rows, plan.q_heads
    q = torch.zeros((rows, Hq, D), dtype=torch.bfloat16)
    out, lse, ws = run(plan, q.to(DEV), k.to(DEV), v.to(DEV))
    m_g, l_g, O_g = partials(plan, ws)
    cache = oattn.Cache(f64(k), f64(v))
    m_o, l_o, O_o = oattn.split_partials(p_oracle, np.zeros((rows, Hq, D)), cache, plan.problem.scale, plan.splits)
    live = p_oracle.live_rows
    assert np.array_equal(l_g[:, :live], l_o[:, :live]), "counts differ"
    assert np.array_equal(O_g[:, :live], O_o[:, :live]), "label sums differ"
    assert np.array_equal(m_g[:, :live], m_o[:, :live]), "maxima differ"


@pytest.mark.parametrize("wrong", [False, True])
def test_control_causal_one_position_late(wrong):
    rows, live, Hq, Hkv, D, P, S = 8, 6, 6, 1, 64, 1000, 4
    cap = P + rows + 64
    g = synth.gen(16001)
    k = synth.normal_bf16((Hkv, cap, D), g)
    v = _labels(Hkv, cap, D)
    plan = plan_for(rows, live, Hq, Hkv, D, "causal", first_pos=P + (1 if wrong else 0), kv_capacity=cap, splits=S)
    p = Problem("causal", rows, live, first_pos=P)
    if wrong:
        with pytest.raises(AssertionError):
            _counting_gate(plan, p, k, v, D)
    else:
        _counting_gate(plan, p, k, v, D)


@pytest.mark.parametrize("wrong", [False, True])
def test_control_window_one_key_wider(wrong):
    rows, live, Hq, Hkv, D, t0, W, S = 8, 7, 6, 1, 64, 2000, 300, 3
    cap = t0 + rows + 64
    g = synth.gen(16002)
    k = synth.normal_bf16((Hkv, cap, D), g)
    v = _labels(Hkv, cap, D)
    plan = plan_for(rows, live, Hq, Hkv, D, "window", first_pos=t0, window=W + (1 if wrong else 0),
                    kv_capacity=cap, splits=S)
    p = Problem("window", rows, live, first_pos=t0, window=W)
    if wrong:
        with pytest.raises(AssertionError):
            _counting_gate(plan, p, k, v, D)
    else:
        _counting_gate(plan, p, k, v, D)


@pytest.mark.parametrize("wrong", [False, True])
def test_control_dropped_sink(wrong):
    """q = 0 with labels: o = sum(labels) / (n + e^sigma), lse = ln(n + e^sigma)
    for the sink the oracle holds; the combine is called without it."""
    rows, live, Hq, Hkv, D, P = 8, 5, 6, 1, 128, 3000
    cap = P + rows + 64
    g = synth.gen(16003)
    k = synth.normal_bf16((Hkv, cap, D), g)
    v = _labels(Hkv, cap, D)
    sink = synth.normal_f32((Hq,), g)
    plan = plan_for(rows, live, Hq, Hkv, D, "causal", first_pos=P, kv_capacity=cap, splits=6)
    q = torch.zeros((rows, Hq, D), dtype=torch.bfloat16)
    out, lse, _ = run(plan, q.to(DEV), k.to(DEV), v.to(DEV), None if wrong else sink.to(DEV))
    vals = f64(v[0])
    sums = np.stack([vals[:P + r + 1].sum(axis=0) for r in range(live)])        # [live, D]
    n = np.arange(P + 1, P + live + 1, dtype=np.float64)                         # visible keys per row
    den = n[:, None] + np.exp(f64(sink))[None, :]                                # [live, Hq]
    want_o = sums[:, None, :] / den[:, :, None]
    want_l = np.log(den)

    def gate():
        o = out.double().numpy()[:live]
        l = lse.double().numpy()[:live]
        assert np.all(np.abs(l - want_l) <= 1e-5), f"lse off by {np.abs(l - want_l).max():.2e}"
        assert np.all(np.abs(o - want_o) <= 1e-6 * np.abs(want_o) + 1e-12), "outputs off"

    if wrong:
        with pytest.raises(AssertionError):
            gate()
    else:
        gate()


@pytest.mark.parametrize("wrong", [False, True])
def test_control_split_partials_overwritten(wrong):
    """Split 1's partials copied over split 0's before the combine."""
    rows, live, Hq, Hkv, D, P, S = 8, 7, 6, 1, 128, 16384, 8
    cap = P + rows + 64
    g = synth.gen(16004)
    q = synth.normal_bf16((rows, Hq, D), g)
    k = synth.normal_bf16((Hkv, cap, D), g)
    v = synth.normal_bf16((Hkv, cap, D), g)
    k[:, P + live:] = NAN
    v[:, P + live:] = NAN
    s = synth.normal_f32((Hq,), g)
    plan = plan_for(rows, live, Hq, Hkv, D, "causal", first_pos=P, kv_capacity=cap, splits=S,
                    scale=1 / math.sqrt(D))
    ws = torch.full(((plan.workspace_bytes + 3) // 4,), NAN, dtype=torch.float32, device=DEV)
    out = torch.full((rows, Hq, D), NAN, dtype=torch.float32, device=DEV)
    lse = torch.full((rows, Hq), NAN, dtype=torch.float32, device=DEV)
    va.verify_attn_split(plan, q.to(DEV), k.to(DEV), v.to(DEV), ws)
    if wrong:
        units = Hkv * rows * (Hq // Hkv)                  # (KV head, matrix row) units per split
        ml_floats = ((S * units * 8 + 255) // 256 * 256) // 4
        ws[0:2 * units] = ws[2 * units:4 * units].clone()
        ws[ml_floats:ml_floats + units * D] = ws[ml_floats + units * D:ml_floats + 2 * units * D].clone()
    va.verify_attn_combine(plan, ws, out, lse=lse, sink=s.to(DEV))
    torch.cuda.synchronize()
    p = Problem("causal", rows, live, first_pos=P)
    cache = oattn.Cache(f64(k[:, :P + live]), f64(v[:, :P + live]))
    ro, rl = oattn.verify_attn_ref(p, f64(q), cache, plan.problem.scale, f64(s))
    lse_c = lse.cpu()

    def gate():
        l = lse_c.double().numpy()[:live]
        assert np.all(np.abs(l - rl[:live]) <= 1e-4), f"lse off by {np.abs(l - rl[:live]).max():.2e}"

    if wrong:
        with pytest.raises(AssertionError):
            gate()
    else:
        gate()
        check(out.cpu(), lse_c, ro, rl, live, "split partials control")


@pytest.mark.parametrize("wrong", [False, True])
def test_control_non_ancestor_made_visible(wrong):
    """The spike sits at node 5, not an ancestor of node 9 (parents 4, 1, 0);
    the GPU plan's parent array hangs node 9 under node 5 instead."""
    D, Hq, Hkv, rows, live, P = 64, 6, 1, 16, 16, 260
    parent = [-1, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 5, 6, 6, 7]
    gpu_parent = list(parent)
    if wrong:
        gpu_parent[9] = 5
    g = synth.gen(16005)
    u = synth.normal_f32((D,), g)
    u = u / u.norm()
    cap = P + rows + 64
    target = P + 5
    q = (u.unsqueeze(0).unsqueeze(0).repeat(rows, Hq, 1) * 8).to(torch.bfloat16)
    k = synth.normal_bf16((Hkv, cap, D), g)
    v = synth.normal_bf16((Hkv, cap, D), g)
    k[0, target] = (u * 20 * math.sqrt(D) / 8).to(torch.bfloat16)
    v[0, target] = 0
    v[0, target, 0] = 100
    k[:, P + live:] = NAN
    v[:, P + live:] = NAN
    s = synth.normal_f32((Hq,), g)
    plan = plan_for(rows, live, Hq, Hkv, D, "tree", prefix_len=P, parent=gpu_parent, kv_capacity=cap, splits=3)
    kw = dict(rows=rows, live=live, mask="tree", prefix_len=P, parent=parent)
    out, lse, ws, ro, rl, p, cache = gpu_and_oracle(plan, kw, q, k, v, s)
    if wrong:
        with pytest.raises(AssertionError):
            check(out, lse, ro, rl, live, "tree spike control (wrong parents)")
    else:
        check(out, lse, ro, rl, live, "tree spike control")
