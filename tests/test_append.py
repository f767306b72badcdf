"""verify_attn_split_append: the rows' own K/V stored and read in one launch.

Gates:
* window ring (config-3 shapes, and a 64-slot ring that wraps inside the
  step): the outputs against the float64 oracle on its own replayed ring,
  and the ring contents after the call bit-exact against that replay;
* every case: the split partials bit-identical to swa_ring_write /
  verify_kv_write followed by verify_attn_split on a copy of the same
  cache, and the cache contents after the call identical too;
* the new rows straddling a 32-key chunk boundary and a split boundary
  (two workgroups put rows into their tiles), no live row (the rows are
  stored, nothing read), 16 rows at D 128;
* tree mode: the node keys at prefix_len + i, a random tree, one case
  straddling a chunk boundary;
* the device-state variant under one bucket: partials and cache contents
  equal to the static append of the state's own problem;
* quantised caches are refused; a linear cache too short for the rows is
  refused before any launch.
The stale contents of the slots the rows take are scaled by 100, so a key
read from memory instead of from the new rows would show, or NaN (a fresh or
poisoned cache): no key of the read, masked ones included, may carry them
into the result.
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
from test_gpu_parity import NAN, check, f64, partials, plan_for

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ws(plan):
    return torch.full(((plan.workspace_bytes + 3) // 4,), NAN, dtype=torch.float32, device=DEV)


def _both(plan, q, k_new, v_new, k, v, write_then_split, sink):
    """(fused partials, out, lse, k, v), (reference partials, out, lse, k, v)."""
    res = []
    for fused in (True, False):
        kc, vc = k.clone(), v.clone()
        ws = _ws(plan)
        out = torch.full((plan.rows, plan.q_heads, plan.head_dim), NAN, dtype=torch.float32, device=DEV)
        lse = torch.full((plan.rows, plan.q_heads), NAN, dtype=torch.float32, device=DEV)
        if fused:
            va.verify_attn_split_append(plan, q, k_new, v_new, kc, vc, ws)
        else:
            write_then_split(kc, vc, ws)
        va.verify_attn_combine(plan, ws, out, lse=lse, sink=sink)
        torch.cuda.synchronize()
        res.append((partials(plan, ws.cpu()), out.cpu(), lse.cpu(), kc.cpu(), vc.cpu()))
    return res


def _same(fused, ref, live, name):
    (mf, lf, of), out_f, lse_f, kf, vf = fused
    (mr, lr, orr), out_r, lse_r, kr, vr = ref
    for a, b, what in ((mf, mr, "m"), (lf, lr, "l"), (of, orr, "O")):
        assert np.array_equal(a[:, :live], b[:, :live], equal_nan=True), f"{name}: {what} partials differ"
    assert torch.equal(out_f.view(torch.int32), out_r.view(torch.int32)), f"{name}: out differs"
    assert torch.equal(lse_f.view(torch.int32), lse_r.view(torch.int32)), f"{name}: lse differs"
    assert torch.equal(kf.view(torch.int16), kr.view(torch.int16)), f"{name}: K cache differs"
    assert torch.equal(vf.view(torch.int16), vr.view(torch.int16)), f"{name}: V cache differs"


@pytest.mark.parametrize("t0,W,C,live,splits,stale", [
    (5120, 4096, 4160, 5, 0, "loud"), (51200, 4096, 4160, 8, 0, "loud"), (194560, 4096, 4160, 7, 0, "loud"),
    (999, 57, 64, 8, 3, "loud"), (1021, 57, 64, 6, 2, "loud"),
    (5120, 4096, 4160, 5, 0, "nan"), (999, 57, 64, 8, 3, "nan"), (1021, 57, 64, 6, 2, "nan")])
def test_append_window_ring(t0, W, C, live, splits, stale):
    rows, Hq, Hkv, D = 8, 6, 1, 64
    g = synth.gen(12000 + t0 + live)
    base = t0 - C
    n = C + rows
    kl = synth.normal_bf16((Hkv, n, D), g)     # position base + i
    vl = synth.normal_bf16((Hkv, n, D), g)
    q = synth.normal_bf16((rows, Hq, D), g)
    s = synth.normal_f32((Hq,), g)
    k_ring = torch.empty((Hkv, C, D), dtype=torch.bfloat16)
    v_ring = torch.empty((Hkv, C, D), dtype=torch.bfloat16)
    for i in range(C):
        k_ring[:, (base + i) % C] = kl[:, i]
        v_ring[:, (base + i) % C] = vl[:, i]
    for r in range(rows):  # stale contents in the slots the rows take
        k_ring[:, (t0 + r) % C] = kl[:, r] * 100 if stale == "loud" else NAN
        v_ring[:, (t0 + r) % C] = vl[:, r] * 100 if stale == "loud" else NAN
    k_new = kl[:, C:C + rows].permute(1, 0, 2).contiguous().to(DEV)
    v_new = vl[:, C:C + rows].permute(1, 0, 2).contiguous().to(DEV)
    plan = plan_for(rows, live, Hq, Hkv, D, "window", first_pos=t0, window=W, ring_slots=C,
                    scale=1 / math.sqrt(D), splits=splits)
    qd, sd = q.to(DEV), s.to(DEV)

    def ref(kc, vc, ws):
        va.swa_ring_write(k_new, v_new, t0, kc, vc)
        va.verify_attn_split(plan, qd, kc, vc, ws)

    fused, unfused = _both(plan, qd, k_new, v_new, k_ring.to(DEV), v_ring.to(DEV), ref, sd)
    name = f"append window t0={t0} C={C} live={live} stale={stale}"
    _same(fused, unfused, live, name)
    # oracle: its own ring from the linear data, replaying the same positions
    labels = omasks.ring_replay(C, list(range(base, t0 + rows)))
    exp_k = torch.stack([kl[:, lab - base] for lab in labels], dim=1)
    assert torch.equal(fused[3].view(torch.int16), exp_k.view(torch.int16)), f"{name}: ring contents"
    ring_k = np.zeros((Hkv, C, D))
    ring_v = np.zeros((Hkv, C, D))
    for pos in range(base, t0 + rows):
        ring_k[:, pos % C] = f64(kl[:, pos - base])
        ring_v[:, pos % C] = f64(vl[:, pos - base])
    p = Problem("window", rows, live, first_pos=t0, window=W, ring_slots=C)
    ro, rl = oattn.verify_attn_ref(p, f64(q), oattn.Cache(ring_k, ring_v, ring_slots=C), plan.problem.scale, f64(s))
    check(fused[1], fused[2], ro, rl, live, name)


@pytest.mark.parametrize("rows,live,Hq,Hkv,D,fp,splits,stale", [
    (8, 8, 6, 1, 128, 4093, 0, "loud"),      # rows 4093..4100 straddle a chunk boundary
    (8, 6, 6, 1, 128, 1021, 32, "loud"),     # the chunk boundary is a split boundary too
    (16, 16, 8, 2, 128, 20005, 0, "loud"),   # 16 rows at D 128, two KV heads
    (8, 5, 6, 1, 64, 3000, 0, "loud"),
    (8, 0, 6, 1, 128, 500, 0, "loud"),       # no live row: stored, nothing read
    (8, 8, 6, 1, 128, 4093, 0, "nan"),
    (8, 6, 6, 1, 128, 1021, 32, "nan"),
    (16, 16, 8, 2, 128, 20005, 0, "nan"),
    (8, 5, 6, 1, 64, 3000, 0, "nan"),
    (8, 3, 6, 1, 128, 4000, 0, "nan"),       # the last live key mid-chunk, masked keys after it
])
def test_append_linear(rows, live, Hq, Hkv, D, fp, splits, stale):
    g = synth.gen(13000 + fp + rows)
    cap = fp + rows + 40
    k = synth.normal_bf16((Hkv, cap, D), g)
    v = synth.normal_bf16((Hkv, cap, D), g)
    k_new = synth.normal_bf16((rows, Hkv, D), g)
    v_new = synth.normal_bf16((rows, Hkv, D), g)
    k[:, fp:fp + rows] = k_new.permute(1, 0, 2) * 100 if stale == "loud" else NAN   # stale
    v[:, fp:fp + rows] = v_new.permute(1, 0, 2) * 100 if stale == "loud" else NAN
    k[:, fp + rows:] = NAN
    v[:, fp + rows:] = NAN
    q = synth.normal_bf16((rows, Hq, D), g)
    s = synth.normal_f32((Hq,), g)
    plan = plan_for(rows, live, Hq, Hkv, D, "causal", first_pos=fp, kv_capacity=cap, scale=1 / math.sqrt(D),
                    splits=splits)
    qd, kn, vn = q.to(DEV), k_new.to(DEV), v_new.to(DEV)

    def ref(kc, vc, ws):
        va.verify_kv_write(kn, vn, fp, kc, vc)
        va.verify_attn_split(plan, qd, kc, vc, ws)

    fused, unfused = _both(plan, qd, kn, vn, k.to(DEV), v.to(DEV), ref, s.to(DEV))
    name = f"append linear fp={fp} rows={rows} live={live} D={D} stale={stale}"
    _same(fused, unfused, live, name)
    assert torch.equal(fused[3][:, fp:fp + rows].view(torch.int16),
                       k_new.permute(1, 0, 2).contiguous().view(torch.int16)), f"{name}: stored K"
    if live:
        kf = k.clone()
        vf = v.clone()
        kf[:, fp:fp + rows] = k_new.permute(1, 0, 2)
        vf[:, fp:fp + rows] = v_new.permute(1, 0, 2)
        hi = fp + live
        p = Problem("causal", rows, live, first_pos=fp)
        ro, rl = oattn.verify_attn_ref(p, f64(q), oattn.Cache(f64(kf[:, :hi]), f64(vf[:, :hi])),
                                       plan.problem.scale, f64(s))
        check(fused[1], fused[2], ro, rl, live, name)


@pytest.mark.parametrize("P,live,Hq,Hkv,splits,stale", [
    (2048, 16, 24, 4, 0, "loud"), (700, 11, 6, 1, 0, "loud"), (700, 16, 6, 1, 22, "loud"),
    (2048, 16, 24, 4, 0, "nan"), (700, 11, 6, 1, 0, "nan"), (700, 16, 6, 1, 22, "nan")])
def test_append_tree(P, live, Hq, Hkv, splits, stale):
    rows, D = 16, 128
    g = synth.gen(14000 + P + live)
    parent = synth.random_tree(rows, g)
    cap = P + rows + 40
    k = synth.normal_bf16((Hkv, cap, D), g)
    v = synth.normal_bf16((Hkv, cap, D), g)
    k_new = synth.normal_bf16((rows, Hkv, D), g)
    v_new = synth.normal_bf16((rows, Hkv, D), g)
    k[:, P:P + rows] = k_new.permute(1, 0, 2) * 100 if stale == "loud" else NAN   # stale
    v[:, P:P + rows] = v_new.permute(1, 0, 2) * 100 if stale == "loud" else NAN
    k[:, P + rows:] = NAN
    v[:, P + rows:] = NAN
    q = synth.normal_bf16((rows, Hq, D), g)
    plan = plan_for(rows, live, Hq, Hkv, D, "tree", prefix_len=P, parent=parent, kv_capacity=cap,
                    scale=1 / math.sqrt(D), splits=splits)
    qd, kn, vn = q.to(DEV), k_new.to(DEV), v_new.to(DEV)

    def ref(kc, vc, ws):
        va.verify_kv_write(kn, vn, P, kc, vc)
        va.verify_attn_split(plan, qd, kc, vc, ws)

    fused, unfused = _both(plan, qd, kn, vn, k.to(DEV), v.to(DEV), ref, None)
    name = f"append tree P={P} live={live} Hkv={Hkv} stale={stale}"
    _same(fused, unfused, live, name)
    kf, vf = k.clone(), v.clone()
    kf[:, P:P + rows] = k_new.permute(1, 0, 2)
    vf[:, P:P + rows] = v_new.permute(1, 0, 2)
    hi = P + live
    p = Problem("tree", rows, live, prefix_len=P, parent=parent)
    ro, rl = oattn.verify_attn_ref(p, f64(q), oattn.Cache(f64(kf[:, :hi]), f64(vf[:, :hi])), plan.problem.scale,
                                   None)
    check(fused[1], fused[2], ro, rl, live, name)


@pytest.mark.parametrize("mode,pos,live,stale", [
    ("causal", 20000, 8, "loud"), ("causal", 4093, 8, "loud"), ("causal", 19990, 5, "loud"),
    ("causal", 100, 0, "loud"), ("window", 51200, 5, "loud"), ("window", 5120, 8, "loud"),
    ("tree", 700, 11, "loud"), ("tree", 2048, 16, "loud"),
    ("causal", 19990, 5, "nan"), ("window", 5120, 5, "nan"), ("tree", 700, 11, "nan")])
def test_append_state_matches_static(mode, pos, live, stale):
    """verify_attn_split_append_state under one bucket against
    verify_attn_split_append of the state's own problem with the state's
    split count (the bucket's, at most one granule each): the same partials
    bit for bit, the same cache contents, outputs equal up to the combine's
    FP32 order."""
    g = synth.gen(15000 + pos + live)
    Hq, Hkv = 6, 1
    if mode == "window":
        rows, D, W, C = 8, 64, 4096, 4160
        bucket_kw = dict(mask="window", first_pos=51200, window=W, ring_slots=C)
        state_kw = dict(mask="window", first_pos=pos, window=W, ring_slots=C)
        slots = C
        st = va.pack_state(first_pos=pos, live_rows=live)
    elif mode == "tree":
        rows, D = 16, 128
        parent = synth.random_tree(rows, g)
        slots = 2048 + rows + 64
        bucket_kw = dict(mask="tree", prefix_len=2048, parent=synth.random_tree(rows, g), kv_capacity=slots)
        state_kw = dict(mask="tree", prefix_len=pos, parent=parent, kv_capacity=slots)
        st = va.pack_state(prefix_len=pos, live_rows=live, parent=parent)
    else:
        rows, D = 8, 128
        slots = 20000 + rows + 64
        bucket_kw = dict(mask="causal", first_pos=20000, kv_capacity=slots)
        state_kw = dict(mask="causal", first_pos=pos, kv_capacity=slots)
        st = va.pack_state(first_pos=pos, live_rows=live)
    bucket = plan_for(rows, rows, Hq, Hkv, D, scale=1 / math.sqrt(D), **bucket_kw)
    own = plan_for(rows, live, Hq, Hkv, D, scale=1 / math.sqrt(D), **state_kw)
    S_eff = max(1, min(bucket.splits, own.info["chunks"]))
    stat = plan_for(rows, live, Hq, Hkv, D, scale=1 / math.sqrt(D), splits=S_eff, **state_kw)
    k = synth.normal_bf16((Hkv, slots, D), g).to(DEV)
    v = synth.normal_bf16((Hkv, slots, D), g).to(DEV)
    kn = synth.normal_bf16((rows, Hkv, D), g).to(DEV)
    vn = synth.normal_bf16((rows, Hkv, D), g).to(DEV)
    q = synth.normal_bf16((rows, Hq, D), g).to(DEV)
    sink = synth.normal_f32((Hq,), g).to(DEV)
    if stale == "nan":  # the slots the rows take hold NaN
        first = pos
        for r in range(rows):
            sl = (first + r) % slots if mode == "window" else first + r
            k[:, sl] = NAN
            v[:, sl] = NAN
    std = st.to(DEV)
    name = f"append state {mode} pos={pos} live={live} stale={stale}"
    ks, vs_ = k.clone(), v.clone()
    ws_s = _ws(bucket)
    out_s = torch.full((rows, Hq, D), NAN, dtype=torch.float32, device=DEV)
    va.verify_attn_split_append_state(bucket, std, q, kn, vn, ks, vs_, ws_s)
    va.verify_attn_combine_state(bucket, std, ws_s, out_s, sink=sink)
    kt, vt = k.clone(), v.clone()
    ws_t = _ws(stat)
    out_t = torch.full((rows, Hq, D), NAN, dtype=torch.float32, device=DEV)
    va.verify_attn_split_append(stat, q, kn, vn, kt, vt, ws_t)
    va.verify_attn_combine(stat, ws_t, out_t, sink=sink)
    torch.cuda.synchronize()
    ms, ls, Os = partials(bucket, ws_s.cpu())
    mt, lt, Ot = partials(stat, ws_t.cpu())
    for a, b, what in ((ms, mt, "m"), (ls, lt, "l"), (Os, Ot, "O")):
        assert np.array_equal(a[:S_eff, :live], b[:, :live], equal_nan=True), f"{name}: {what} partials differ"
    assert torch.equal(ks.view(torch.int16), kt.view(torch.int16)), f"{name}: K cache differs"
    assert torch.equal(vs_.view(torch.int16), vt.view(torch.int16)), f"{name}: V cache differs"
    o, ot = out_s.cpu()[:live].double().numpy(), out_t.cpu()[:live].double().numpy()
    assert np.allclose(o, ot, rtol=1e-5, atol=1e-6), f"{name}: out differs"
    assert torch.all(out_s.cpu()[live:] == 0), f"{name}: padding rows"


@pytest.mark.parametrize("mode", ["causal", "window"])
def test_append_state_without_live_rows_far_away(mode):
    """A state with no live rows is valid at any position up to 2^61.  Its
    rows go to the slots of their own keys: none in a linear cache far
    shorter than the position (nothing stored, nothing read), slot
    (pos + r) mod C in a ring."""
    g = synth.gen(15999)
    rows, Hq, Hkv = 8, 6, 1
    pos = 3_000_000_123
    if mode == "window":
        D, W, C = 64, 4096, 4160
        bucket = plan_for(rows, rows, Hq, Hkv, D, "window", first_pos=51200, window=W, ring_slots=C)
        slots = C
    else:
        D = 128
        slots = 20000 + rows + 64
        bucket = plan_for(rows, rows, Hq, Hkv, D, "causal", first_pos=20000, kv_capacity=slots)
    k = synth.normal_bf16((Hkv, slots, D), g).to(DEV)
    v = synth.normal_bf16((Hkv, slots, D), g).to(DEV)
    kn = synth.normal_bf16((rows, Hkv, D), g).to(DEV)
    vn = synth.normal_bf16((rows, Hkv, D), g).to(DEV)
    q = synth.normal_bf16((rows, Hq, D), g).to(DEV)
    st = va.pack_state(first_pos=pos, live_rows=0).to(DEV)
    ks, vs_ = k.clone(), v.clone()
    ws = _ws(bucket)
    out = torch.full((rows, Hq, D), NAN, dtype=torch.float32, device=DEV)
    va.verify_attn_split_append_state(bucket, st, q, kn, vn, ks, vs_, ws)
    va.verify_attn_combine_state(bucket, st, ws, out)
    torch.cuda.synchronize()
    assert torch.all(out.cpu() == 0)
    ek, ev = k.clone(), v.clone()
    if mode == "window":
        for r in range(rows):
            ek[:, (pos + r) % C] = kn[r]
            ev[:, (pos + r) % C] = vn[r]
    assert torch.equal(ks.view(torch.int16), ek.view(torch.int16))
    assert torch.equal(vs_.view(torch.int16), ev.view(torch.int16))


def test_append_refused():
    g = synth.gen(13999)
    q = synth.normal_bf16((8, 6, 128), g).to(DEV)
    kn = synth.normal_bf16((8, 1, 128), g).to(DEV)
    k = torch.zeros((1, 600, 128), dtype=torch.bfloat16, device=DEV)
    quant = plan_for(8, 8, 6, 1, 128, "causal", kv_fmt="e4m3_wht_i8", first_pos=500, kv_capacity=600)
    with pytest.raises((va.VAError, ValueError, TypeError)):
        va.verify_attn_split_append(quant, q, kn, kn, k, k.clone(), va.workspace_for(quant, DEV))
    # capacity 506 holds the live rows' keys (hi = 504) but not all 8 rows:
    # refused by the library (the tensor is longer than the plan's capacity)
    # and by the binding (a tensor too short for the rows)
    short = plan_for(8, 4, 6, 1, 128, "causal", first_pos=500, kv_capacity=506)
    with pytest.raises(va.VAError):
        va.verify_attn_split_append(short, q, kn, kn, k, k.clone(), va.workspace_for(short, DEV))
    ks = torch.zeros((1, 506, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        va.verify_attn_split_append(short, q, kn, kn, ks, ks.clone(), va.workspace_for(short, DEV))
    torch.cuda.synchronize()
