"""Per-call state in device memory: verify_attn_split_state / verify_attn_combine_state.

A plan built for a bucket fixes the grid and the workspace; the positions,
live rows and tree of each call come from a va_state record on the device.
Gates:
* the state path against the float64 oracle, as in the static parity tests;
* its split partials bit-identical to the static path's for the same
  problem with the state's split count min(S_bucket, granules), and the
  workspace of the splits above that count untouched (NaN sentinel);
* one captured graph replayed over several states, each replay equal bit for
  bit to the eager state call;
* every invalid state: NaN in every output and the workspace untouched.
The static path is itself pinned to the oracle by test_gpu_parity.
"""
import ctypes

import numpy as np
import pytest
import torch

import speculative_decode_verify_amd as va
from speculative_decode_verify_amd import _binding, synth
from oracle import attn as oattn
from oracle.masks import Problem
from test_gpu_parity import check, f64, partials, run

DEV = "cuda"
NAN = float("nan")


# ----------------------------------------------------------------------------- CPU

def test_state_record_layout():
    st = _binding.va_state
    assert ctypes.sizeof(st) == 88
    assert (st.first_pos.offset, st.prefix_len.offset, st.live_rows.offset, st.reserved.offset,
            st.parent.offset) == (0, 8, 16, 20, 24)
    t = va.pack_state(first_pos=7, prefix_len=9, live_rows=3, parent=[-1, 0, 1])
    assert t.dtype == torch.int64 and t.numel() == 11
    w = t.numpy().view(np.int32)
    assert t[0] == 7 and t[1] == 9 and w[4] == 3 and w[5] == 0
    assert list(w[6:9]) == [-1, 0, 1] and np.all(w[9:] == -1)


@pytest.mark.parametrize("bad", [None, 0x100004])
def test_state_pointer_rejected_before_launch(bad):
    """NULL or misaligned state: VA_ERR_INVALID from both entry points; the
    check comes first, so no other argument is looked at."""
    plan = va.Plan(rows=4, live_rows=4, q_heads=2, kv_heads=1, head_dim=64, first_pos=100, kv_capacity=200)
    lib = va.load_library()
    fake = ctypes.c_void_p(0x100000)
    st = None if bad is None else ctypes.c_void_p(bad)
    r1 = lib.verify_attn_split_state(ctypes.byref(plan.plan), st, fake, fake, fake, None, 0, 200 * 64, 64, fake,
                                     plan.workspace_bytes, None)
    r2 = lib.verify_attn_combine_state(ctypes.byref(plan.plan), st, fake, plan.workspace_bytes, None, fake, None,
                                       None)
    assert r1 == 1 and r2 == 1


# ----------------------------------------------------------------------------- GPU helpers

def run_state(plan, state, q, k, v, s, v_scale=None):
    """State split + combine with NaN-filled workspace and outputs."""
    ws = torch.full(((plan.workspace_bytes + 3) // 4,), NAN, dtype=torch.float32, device=DEV)
    out = torch.full((plan.rows, plan.q_heads, plan.head_dim), NAN, dtype=torch.float32, device=DEV)
    lse = torch.full((plan.rows, plan.q_heads), NAN, dtype=torch.float32, device=DEV)
    st = state.to(DEV)
    va.verify_attn_split_state(plan, st, q, k, v, ws, v_scale=v_scale)
    va.verify_attn_combine_state(plan, st, ws, out, lse=lse, sink=s)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), ws.cpu()


def effective_splits(bucket, static_kw):
    """min(S_bucket, granules of the state's extent), at least 1."""
    probe = va.Plan(**static_kw, splits=1)
    return max(1, min(bucket.splits, probe.info["chunks"]))


def compare_with_static(bucket, static_kw, ws_state, q, k, v, s, name, v_scale=None):
    """Partials of splits below S_eff bit-identical to the static path's with
    S_eff splits; splits at and above S_eff untouched.  Returns the static
    path's (out, lse)."""
    S_eff = effective_splits(bucket, static_kw)
    stat = va.Plan(**static_kw, splits=S_eff)
    assert stat.splits == S_eff
    out_s, lse_s, ws_s = run(stat, q, k, v, s, v_scale)
    ms, ls, Os = partials(bucket, ws_state)
    mt, lt, Ot = partials(stat, ws_s)
    for a, b, what in ((ms, mt, "m"), (ls, lt, "l"), (Os, Ot, "O")):
        assert np.array_equal(a[:S_eff], b, equal_nan=True), f"{name}: {what} partials differ from static"
        assert np.all(np.isnan(a[S_eff:])), f"{name}: {what} written above the state's {S_eff} splits"
    return out_s, lse_s


def close_to_static(out, lse, out_s, lse_s, live, name):
    """The combine may sum the same partials in another order (its batch
    width follows the bucket's split count): FP32 rounding apart."""
    o, os_ = out[:live].double().numpy(), out_s[:live].double().numpy()
    assert np.allclose(o, os_, rtol=1e-5, atol=1e-6), f"{name}: out differs from the static path"
    l, ls = lse[:live].double().numpy(), lse_s[:live].double().numpy()
    assert np.array_equal(np.isfinite(l), np.isfinite(ls))
    fin = np.isfinite(l)
    assert np.allclose(l[fin], ls[fin], rtol=1e-6, atol=1e-5), f"{name}: lse differs from the static path"


# ----------------------------------------------------------------------------- chain

CHAIN_BUCKET = dict(rows=16, live=16, fp=20000)
CHAIN_STATES = [(20000, 16), (19990, 16), (4000, 9), (37, 16), (0, 1), (100, 0), (20010, 6)]


@pytest.mark.gpu
@pytest.mark.parametrize("fp,live", CHAIN_STATES)
def test_state_causal_in_bucket(fp, live):
    """Causal rows at fp..fp+live-1 under a 16-row bucket at 20000 (reads
    end at or below 20016); keys at and past the state's own hi are NaN."""
    rows, Hq, Hkv, D = 16, 8, 2, 128
    cap = CHAIN_BUCKET["fp"] + rows + 64
    bucket = va.Plan(rows=rows, live_rows=rows, q_heads=Hq, kv_heads=Hkv, head_dim=D, mask="causal",
                     first_pos=CHAIN_BUCKET["fp"], kv_capacity=cap)
    g = synth.gen(9100 + fp + live)
    hi = fp + live
    q = synth.normal_bf16((rows, Hq, D), g)
    k = synth.normal_bf16((Hkv, cap, D), g)
    v = synth.normal_bf16((Hkv, cap, D), g)
    k[:, hi:] = NAN
    v[:, hi:] = NAN
    s = synth.normal_f32((Hq,), g)
    qd, kd, vd, sd = q.to(DEV), k.to(DEV), v.to(DEV), s.to(DEV)
    state = va.pack_state(first_pos=fp, live_rows=live)
    out, lse, ws = run_state(bucket, state, qd, kd, vd, sd)
    name = f"state causal fp={fp} live={live}"
    p = Problem("causal", rows, live, first_pos=fp)
    cache = oattn.Cache(f64(k[:, :max(hi, 1)]), f64(v[:, :max(hi, 1)]))
    ro, rl = oattn.verify_attn_ref(p, f64(q), cache, bucket.problem.scale, f64(s))
    check(out, lse, ro, rl, live, name)
    static_kw = dict(rows=rows, live_rows=live, q_heads=Hq, kv_heads=Hkv, head_dim=D, mask="causal",
                     first_pos=fp, kv_capacity=cap)
    out_s, lse_s = compare_with_static(bucket, static_kw, ws, qd, kd, vd, sd, name)
    close_to_static(out, lse, out_s, lse_s, live, name)


# ----------------------------------------------------------------------------- window ring

@pytest.mark.gpu
@pytest.mark.parametrize("fp,live", [(50000, 8), (49000, 8), (3000, 5), (500, 3), (0, 8), (1020, 8)])
def test_state_window_ring_in_bucket(fp, live):
    """Window 1,024 over a 1,088-slot ring, bucket 8 rows at 50000.  The
    ring holds the state's keys [lo, hi) at slot pos mod 1088; every other
    slot is NaN."""
    rows, Hq, Hkv, D, W, C = 8, 6, 1, 64, 1024, 1088
    bucket = va.Plan(rows=rows, live_rows=rows, q_heads=Hq, kv_heads=Hkv, head_dim=D, mask="window",
                     first_pos=50000, window=W, ring_slots=C)
    g = synth.gen(9200 + fp + live)
    lo, hi = max(0, fp - W + 1), fp + live
    kl = synth.normal_bf16((Hkv, hi - lo, D), g)   # position lo + i
    vl = synth.normal_bf16((Hkv, hi - lo, D), g)
    q = synth.normal_bf16((rows, Hq, D), g)
    s = synth.normal_f32((Hq,), g)
    k_ring = torch.full((Hkv, C, D), NAN, dtype=torch.bfloat16)
    v_ring = torch.full((Hkv, C, D), NAN, dtype=torch.bfloat16)
    slots = torch.arange(lo, hi) % C
    k_ring[:, slots] = kl
    v_ring[:, slots] = vl
    qd, kd, vd, sd = q.to(DEV), k_ring.to(DEV), v_ring.to(DEV), s.to(DEV)
    state = va.pack_state(first_pos=fp, live_rows=live)
    out, lse, ws = run_state(bucket, state, qd, kd, vd, sd)
    name = f"state window fp={fp} live={live}"
    ring_k = np.nan_to_num(f64(k_ring), nan=0.0)
    ring_v = np.nan_to_num(f64(v_ring), nan=0.0)
    p = Problem("window", rows, live, first_pos=fp, window=W, ring_slots=C)
    ro, rl = oattn.verify_attn_ref(p, f64(q), oattn.Cache(ring_k, ring_v, ring_slots=C), bucket.problem.scale,
                                   f64(s))
    check(out, lse, ro, rl, live, name)
    static_kw = dict(rows=rows, live_rows=live, q_heads=Hq, kv_heads=Hkv, head_dim=D, mask="window",
                     first_pos=fp, window=W, ring_slots=C)
    out_s, lse_s = compare_with_static(bucket, static_kw, ws, qd, kd, vd, sd, name)
    close_to_static(out, lse, out_s, lse_s, live, name)


# ----------------------------------------------------------------------------- tree

TREE_STATES = ["bucket", "chain", "star", "empty_prefix", "short", "late"]


def tree_state(kind, g):
    if kind == "bucket":
        return 6000, 16, synth.random_tree(16, g)
    if kind == "chain":
        return 100, 5, [-1, 0, 1, 2, 3]
    if kind == "star":
        return 3001, 16, [-1] + [0] * 15
    if kind == "empty_prefix":
        return 0, 4, [-1, 0, 0, 1]
    if kind == "short":
        return 33, 1, [-1]
    return 6010, 6, [-1, 0, 1, 1, 2, 0]


@pytest.mark.gpu
@pytest.mark.parametrize("kind", TREE_STATES)
def test_state_tree_in_bucket(kind):
    """Trees under a 16-node bucket over a 6,000-key prefix (12 q heads on
    2 KV heads, D 128); states differ in prefix, node count and shape."""
    rows, Hq, Hkv, D = 16, 12, 2, 128
    cap = 6000 + rows + 64
    g = synth.gen(9300 + TREE_STATES.index(kind))
    bucket = va.Plan(rows=rows, live_rows=rows, q_heads=Hq, kv_heads=Hkv, head_dim=D, mask="tree",
                     prefix_len=6000, parent=synth.random_tree(rows, g), kv_capacity=cap)
    P, live, parent = tree_state(kind, g)
    hi = P + live
    q = synth.normal_bf16((rows, Hq, D), g)
    k = synth.normal_bf16((Hkv, cap, D), g)
    v = synth.normal_bf16((Hkv, cap, D), g)
    k[:, hi:] = NAN
    v[:, hi:] = NAN
    s = synth.normal_f32((Hq,), g)
    qd, kd, vd, sd = q.to(DEV), k.to(DEV), v.to(DEV), s.to(DEV)
    state = va.pack_state(prefix_len=P, live_rows=live, parent=parent)
    out, lse, ws = run_state(bucket, state, qd, kd, vd, sd)
    name = f"state tree {kind} P={P} live={live}"
    p = Problem("tree", rows, live, prefix_len=P, parent=parent + [-1] * (rows - len(parent)))
    cache = oattn.Cache(f64(k[:, :hi]), f64(v[:, :hi]))
    ro, rl = oattn.verify_attn_ref(p, f64(q), cache, bucket.problem.scale, f64(s))
    check(out, lse, ro, rl, live, name)
    static_kw = dict(rows=rows, live_rows=live, q_heads=Hq, kv_heads=Hkv, head_dim=D, mask="tree",
                     prefix_len=P, parent=parent, kv_capacity=cap)
    out_s, lse_s = compare_with_static(bucket, static_kw, ws, qd, kd, vd, sd, name)
    close_to_static(out, lse, out_s, lse_s, live, name)


# ----------------------------------------------------------------------------- quantised cache

@pytest.mark.gpu
@pytest.mark.parametrize("fp,live", [(12000, 16), (700, 7)])
def test_state_quantized_matches_static(fp, live):
    """E4M3 keys and INT8 values: the state path's partials equal the static
    path's bit for bit (the static quantised path is pinned to the oracle by
    the parity tests).  Codes are random bytes with NaN key codes 0x7F/0xFF
    mapped to finite ones; slots at and past hi hold NaN codes and scales."""
    rows, Hq, Hkv, D = 16, 6, 1, 128
    cap = 12000 + rows + 64
    bucket = va.Plan(rows=rows, live_rows=rows, q_heads=Hq, kv_heads=Hkv, head_dim=D, mask="causal",
                     kv_fmt="e4m3_wht_i8", first_pos=12000, kv_capacity=cap)
    g = synth.gen(9400 + live)
    hi = fp + live
    kc = torch.randint(0, 256, (Hkv, cap, D), generator=g, dtype=torch.int64)
    kc[(kc & 0x7F) == 0x7F] -= 1
    kc[:, hi:] = 0x7F
    vc = torch.randint(-127, 128, (Hkv, cap, D), generator=g, dtype=torch.int64).to(torch.int8)
    sc = torch.rand((Hkv, cap), generator=g) * 0.02 + 1e-3
    sc[:, hi:] = NAN
    q = synth.normal_bf16((rows, Hq, D), g)
    qd, kd, vd, scd = q.to(DEV), kc.to(torch.uint8).to(DEV), vc.to(DEV), sc.to(DEV)
    state = va.pack_state(first_pos=fp, live_rows=live)
    out, lse, ws = run_state(bucket, state, qd, kd, vd, None, v_scale=scd)
    name = f"state quantised fp={fp} live={live}"
    assert torch.isfinite(out[:live]).all() and torch.isfinite(lse[:live]).all(), name
    static_kw = dict(rows=rows, live_rows=live, q_heads=Hq, kv_heads=Hkv, head_dim=D, mask="causal",
                     kv_fmt="e4m3_wht_i8", first_pos=fp, kv_capacity=cap)
    out_s, lse_s = compare_with_static(bucket, static_kw, ws, qd, kd, vd, None, name, v_scale=scd)
    close_to_static(out, lse, out_s, lse_s, live, name)


# ----------------------------------------------------------------------------- graphs

@pytest.mark.gpu
def test_state_graph_replays_follow_the_state():
    """Split + combine captured once; the state tensor is rewritten between
    replays (eager work and synchronisations in between).  Each replay equals
    the eager state call bit for bit, and the last one the oracle."""
    rows, Hq, Hkv, D = 16, 8, 2, 128
    cap = 8000 + rows + 64
    bucket = va.Plan(rows=rows, live_rows=rows, q_heads=Hq, kv_heads=Hkv, head_dim=D, mask="causal",
                     first_pos=8000, kv_capacity=cap)
    g = synth.gen(9500)
    q = synth.normal_bf16((rows, Hq, D), g).to(DEV)
    k = synth.normal_bf16((Hkv, cap, D), g)
    v = synth.normal_bf16((Hkv, cap, D), g)
    s = synth.normal_f32((Hq,), g).to(DEV)
    kd, vd = k.to(DEV), v.to(DEV)
    st = va.pack_state(first_pos=8000, live_rows=16).to(DEV)
    ws = va.workspace_for(bucket, DEV)
    out = torch.empty((rows, Hq, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((rows, Hq), dtype=torch.float32, device=DEV)
    va.verify_attn_split_state(bucket, st, q, kd, vd, ws)
    va.verify_attn_combine_state(bucket, st, ws, out, lse=lse, sink=s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        va.verify_attn_split_state(bucket, st, q, kd, vd, ws)
        va.verify_attn_combine_state(bucket, st, ws, out, lse=lse, sink=s)
    states = [(8000, 16), (5000, 3), (64, 16), (7990, 11), (0, 2), (8000, 16)]
    for fp, live in states:
        host = va.pack_state(first_pos=fp, live_rows=live)
        st.copy_(host)
        out.fill_(NAN)
        lse.fill_(NAN)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eo, el, _ = run_state(bucket, host, q, kd, vd, s)
        assert torch.equal(out.cpu().view(torch.int32), eo.view(torch.int32)), f"replay fp={fp} live={live}"
        assert torch.equal(lse.cpu().view(torch.int32), el.view(torch.int32)), f"replay fp={fp} live={live}"
    p = Problem("causal", rows, 16, first_pos=8000)
    ro, rl = oattn.verify_attn_ref(p, f64(q), oattn.Cache(f64(k[:, :8016]), f64(v[:, :8016])),
                                   bucket.problem.scale, f64(s))
    check(out.cpu(), lse.cpu(), ro, rl, 16, "state graph last replay")


# ----------------------------------------------------------------------------- invalid states

def _invalid_states():
    bad_reserved = va.pack_state(first_pos=100, live_rows=4)
    bad_reserved.numpy().view(np.int32)[5] = 1
    return {
        "reserved": ("causal", bad_reserved),
        "live_above_rows": ("causal", va.pack_state(first_pos=100, live_rows=17)),
        "live_negative": ("causal", va.pack_state(first_pos=100, live_rows=-1)),
        "position_negative": ("causal", va.pack_state(first_pos=-5, live_rows=4)),
        "past_bucket": ("causal", va.pack_state(first_pos=4000, live_rows=1)),
        "past_bucket_by_one": ("causal", va.pack_state(first_pos=3985, live_rows=16)),
        "parent_forward": ("tree", va.pack_state(prefix_len=100, live_rows=4, parent=[-1, 0, 3, 1])),
        "parent_below_minus_one": ("tree", va.pack_state(prefix_len=100, live_rows=4, parent=[-1, -2, 0, 1])),
        "prefix_negative": ("tree", va.pack_state(prefix_len=-1, live_rows=4, parent=[-1, 0, 0, 1])),
        "tree_past_bucket": ("tree", va.pack_state(prefix_len=3990, live_rows=16, parent=[-1] * 16)),
    }


@pytest.mark.gpu
@pytest.mark.parametrize("which", list(_invalid_states()))
def test_invalid_state_gives_nan_and_reads_nothing(which):
    """Every output and lse NaN; no workspace element written."""
    mask, state = _invalid_states()[which]
    rows, Hq, Hkv, D = 16, 6, 1, 64
    cap = 4000 + 64
    if mask == "causal":
        bucket = va.Plan(rows=rows, live_rows=rows, q_heads=Hq, kv_heads=Hkv, head_dim=D, mask="causal",
                         first_pos=4000 - rows, kv_capacity=cap)
    else:
        bucket = va.Plan(rows=rows, live_rows=rows, q_heads=Hq, kv_heads=Hkv, head_dim=D, mask="tree",
                         prefix_len=4000 - rows, parent=[-1] * rows, kv_capacity=cap)
    assert bucket.info["hi"] == 4000
    g = synth.gen(9600)
    q = synth.normal_bf16((rows, Hq, D), g).to(DEV)
    k = synth.normal_bf16((Hkv, cap, D), g).to(DEV)
    v = synth.normal_bf16((Hkv, cap, D), g).to(DEV)
    out, lse, ws = run_state(bucket, state, q, k, v, None)
    assert torch.all(torch.isnan(out)), which
    assert torch.all(torch.isnan(lse)), which
    assert torch.all(torch.isnan(ws)), which
