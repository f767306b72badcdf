"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Gates:
* every live output element: |gpu - ref| <= 2e-3 + 1e-2 |ref|;
* lse: |gpu - ref| <= 1e-4 (the quantised-key case adds a bound derived
  from rounding the rotated query to bf16, see _q_rounding_bound);
* padding rows exactly 0 and lse -inf;
* bit-exact: the counting test's partials (q = 0, integer labels in V), the
  ring contents after the write, determinism, append invariance.

Inputs are seeded (speculative_decode_verify_amd.synth); capacity beyond the
read extent and the workspace are filled with NaN before each call, so any
read outside the extent or any unwritten output shows up.
"""
import math

import numpy as np
import pytest
import torch

import speculative_decode_verify_amd as va
from speculative_decode_verify_amd import synth
from oracle import attn as oattn
from oracle import codec as ocodec
from oracle import masks as omasks
from oracle.masks import Problem

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL_ABS, TOL_REL, TOL_LSE = 2e-3, 1e-2, 1e-4
NAN = float("nan")


# ----------------------------------------------------------------------------- helpers

def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def run(plan, q, k, v, sink=None, v_scale=None):
    """Split + combine with a NaN-filled workspace and NaN-filled outputs."""
    ws = torch.full(((plan.workspace_bytes + 3) // 4,), NAN, dtype=torch.float32, device=DEV)
    out = torch.full((plan.rows, plan.q_heads, plan.head_dim), NAN, dtype=torch.float32, device=DEV)
    lse = torch.full((plan.rows, plan.q_heads), NAN, dtype=torch.float32, device=DEV)
    va.verify_attn_split(plan, q, k, v, ws, v_scale=v_scale)
    va.verify_attn_combine(plan, ws, out, lse=lse, sink=sink)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), ws.cpu()


def partials(plan, ws):
    """Workspace -> (m natural-log units, l, O) indexed [S, R, Hq(, D)]."""
    S, Hkv, D = plan.splits, plan.kv_heads, plan.head_dim
    R, Hq = plan.rows, plan.q_heads
    G = Hq // Hkv
    MR = R * G
    n = S * Hkv * MR
    ml_floats = ((n * 8 + 255) // 256 * 256) // 4
    flat = ws.numpy()
    ml = flat[: n * 2].reshape(S, Hkv, R, G, 2).transpose(0, 2, 1, 3, 4).reshape(S, R, Hq, 2)
    O = flat[ml_floats: ml_floats + n * D].reshape(S, Hkv, R, G, D).transpose(0, 2, 1, 3, 4).reshape(S, R, Hq, D)
    return ml[..., 0].astype(np.float64) * math.log(2.0), ml[..., 1].astype(np.float64), O.astype(np.float64)


def check(out, lse, ro, rl, live, name, lse_tol=TOL_LSE):
    o = out.double().numpy()
    l = lse.double().numpy()
    assert np.isfinite(o).all(), f"{name}: non-finite output"
    err = np.abs(o[:live] - ro[:live])
    tol = TOL_ABS + TOL_REL * np.abs(ro[:live])
    bad = err > tol
    rel_l2 = np.linalg.norm(o[:live] - ro[:live]) / max(np.linalg.norm(ro[:live]), 1e-300)
    print(f"{name}: max|err| {err.max() if err.size else 0:.3e}  rel-L2 {rel_l2:.3e}", flush=True)
    assert not bad.any(), f"{name}: {bad.sum()} elements outside the gate, max err {err.max():.3e}"
    assert np.all(o[live:] == 0), f"{name}: padding rows not zero"
    assert np.all(l[live:] == -np.inf), f"{name}: padding lse not -inf"
    fin = np.isfinite(rl[:live])
    assert np.array_equal(fin, np.isfinite(l[:live])), f"{name}: lse finiteness differs"
    dl = np.abs(l[:live][fin] - rl[:live][fin])
    tol_l = lse_tol if np.isscalar(lse_tol) else np.asarray(lse_tol)[:live][fin]
    assert np.all(dl <= tol_l), f"{name}: lse err {dl.max():.3e}"


def plan_for(rows, live, Hq, Hkv, D, mask="causal", **kw):
    return va.Plan(rows=rows, live_rows=live, q_heads=Hq, kv_heads=Hkv, head_dim=D, mask=mask, **kw)


def oracle_problem(plan_kw):
    return Problem(plan_kw.get("mask", "causal"), plan_kw["rows"], plan_kw["live"],
                   first_pos=plan_kw.get("first_pos", 0), prefix_len=plan_kw.get("prefix_len", 0),
                   parent=plan_kw.get("parent"), window=plan_kw.get("window", 0),
                   ring_slots=plan_kw.get("ring_slots", 0))


def linear_case(seed, rows, live, Hq, Hkv, D, mask, first_pos=0, prefix_len=0, parent=None, sink=True,
                splits=0, extra_cap=64, window=0):
    """Random bf16 q/K/V on a linear cache; slots beyond the extent are NaN."""
    g = synth.gen(seed)
    if mask == "tree":
        hi = prefix_len + live
        cap = prefix_len + rows + extra_cap
    else:
        hi = first_pos + live
        cap = first_pos + rows + extra_cap
    q = synth.normal_bf16((rows, Hq, D), g)
    k = synth.normal_bf16((Hkv, cap, D), g)
    v = synth.normal_bf16((Hkv, cap, D), g)
    k[:, hi:] = NAN
    v[:, hi:] = NAN
    s = synth.normal_f32((Hq,), g) if sink else None
    kw = dict(rows=rows, live=live, mask=mask, first_pos=first_pos, prefix_len=prefix_len, parent=parent,
              window=window)
    plan = plan_for(rows, live, Hq, Hkv, D, mask, first_pos=first_pos, prefix_len=prefix_len, parent=parent,
                    window=window, kv_capacity=cap, splits=splits, scale=1.0 / math.sqrt(D))
    return plan, kw, q, k, v, s


def gpu_and_oracle(plan, kw, q, k, v, s, v_scale=None, cache=None, q_oracle=None):
    out, lse, ws = run(plan, q.to(DEV), k.to(DEV), v.to(DEV), None if s is None else s.to(DEV),
                       None if v_scale is None else v_scale.to(DEV))
    p = oracle_problem(kw)
    lo, hi = omasks.union_extent_fast(p)
    if cache is None:
        # only slots below hi are ever needed; NaN beyond them is never touched by the oracle
        cache = oattn.Cache(f64(k[:, :max(hi, 1)]), f64(v[:, :max(hi, 1)]))
    qo = f64(q) if q_oracle is None else q_oracle
    ro, rl = oattn.verify_attn_ref(p, qo, cache, plan.problem.scale, None if s is None else f64(s))
    return out, lse, ws, ro, rl, p, cache


# ----------------------------------------------------------------------------- configs

def test_config1_tiny_causal():
    """1 KV head, 6 q heads, D 64, 8 rows (5 live) at 1019..1026, read extent
    1,024 keys, capacity 1,032 with the padding rows' slots poisoned, 4 splits."""
    plan, kw, q, k, v, s = linear_case(101, 8, 5, 6, 1, 64, "causal", first_pos=1019, splits=4, extra_cap=5)
    assert plan.problem.kv_capacity == 1032 and plan.info["hi"] == 1024 and plan.info["chunks"] == 32
    out, lse, ws, ro, rl, p, cache = gpu_and_oracle(plan, kw, q, k, v, s)
    check(out, lse, ro, rl, 5, "config1")
    # partials against the oracle's split form (same 4 granule-aligned splits)
    m_g, l_g, O_g = partials(plan, ws)
    m_o, l_o, O_o = oattn.split_partials(p, f64(q), cache, plan.problem.scale, 4)
    live = 5
    assert np.array_equal(np.isfinite(m_g[:, :live]), np.isfinite(m_o[:, :live]))
    fin = np.isfinite(m_o[:, :live])
    assert np.all(np.abs(m_g[:, :live][fin] - m_o[:, :live][fin]) <= 1e-5)
    assert np.allclose(l_g[:, :live], l_o[:, :live], rtol=1e-5, atol=0)
    dO = np.linalg.norm(O_g[:, :live] - O_o[:, :live], axis=-1)
    assert np.all(dO <= 1e-2 * np.linalg.norm(O_o[:, :live], axis=-1) + 1e-3)
    # padding rows' partials are never stored: the NaN fill survives
    assert np.all(np.isnan(m_g[:, live:])) and np.all(np.isnan(l_g[:, live:])) and np.all(np.isnan(O_g[:, live:]))


CONFIG2_CONTEXTS = [1024, 4096, 16384, 32768, 65536, 131072, 196608]


@pytest.mark.parametrize("ctx", CONFIG2_CONTEXTS)
def test_config2_full_attention_sweep(ctx):
    """1 KV head, 6 q heads, D 128, 8 rows with 4..8 live at positions ctx..,
    capacity 262,144 (NaN beyond the read), sink on, plan-chosen splits."""
    g = synth.gen(2000 + ctx // 1024)
    live = synth.live_count(g)
    rows, Hq, Hkv, D, cap = 8, 6, 1, 128, 262144
    hi = ctx + live
    q = synth.normal_bf16((rows, Hq, D), g)
    k = torch.full((Hkv, cap, D), NAN, dtype=torch.bfloat16)
    v = torch.full((Hkv, cap, D), NAN, dtype=torch.bfloat16)
    k[:, :hi] = synth.normal_bf16((Hkv, hi, D), g)
    v[:, :hi] = synth.normal_bf16((Hkv, hi, D), g)
    s = synth.normal_f32((Hq,), g)
    plan = plan_for(rows, live, Hq, Hkv, D, "causal", first_pos=ctx, kv_capacity=cap, scale=1 / math.sqrt(D))
    kw = dict(rows=rows, live=live, mask="causal", first_pos=ctx)
    out, lse, ws, ro, rl, p, cache = gpu_and_oracle(plan, kw, q, k, v, s)
    check(out, lse, ro, rl, live, f"config2 ctx={ctx} live={live} S={plan.splits}")


@pytest.mark.parametrize("t0", [5120, 51200, 194560])
def test_config3_window_ring(t0):
    """D 64, window 4096 over a 4,160-slot ring; the 8 rows' K/V are written
    into the ring first (over stale slots); the ring has wrapped."""
    rows, live, Hq, Hkv, D, W, C = 8, 5, 6, 1, 64, 4096, 4160
    g = synth.gen(3000 + t0 // 1024)
    base = t0 - C
    n = C + rows
    kl = synth.normal_bf16((Hkv, n, D), g)     # position base + i
    vl = synth.normal_bf16((Hkv, n, D), g)
    stale_k = synth.normal_bf16((Hkv, rows, D), g) * 100
    stale_v = synth.normal_bf16((Hkv, rows, D), g) * 100
    q = synth.normal_bf16((rows, Hq, D), g)
    s = synth.normal_f32((Hq,), g)
    # ring before the step: history [t0 - C, t0) at slot p mod C, then stale
    # data in the slots the new rows will take
    k_ring = torch.empty((Hkv, C, D), dtype=torch.bfloat16)
    v_ring = torch.empty((Hkv, C, D), dtype=torch.bfloat16)
    for i in range(C):
        pos = base + i
        k_ring[:, pos % C] = kl[:, i]
        v_ring[:, pos % C] = vl[:, i]
    for r in range(rows):
        k_ring[:, (t0 + r) % C] = stale_k[:, r]
        v_ring[:, (t0 + r) % C] = stale_v[:, r]
    k_new = kl[:, C:C + rows].permute(1, 0, 2).contiguous()      # [rows, Hkv, D]
    v_new = vl[:, C:C + rows].permute(1, 0, 2).contiguous()
    kr, vr = k_ring.to(DEV), v_ring.to(DEV)
    va.swa_ring_write(k_new.to(DEV), v_new.to(DEV), t0, kr, vr)
    torch.cuda.synchronize()
    # ring contents: bit-exact against a replay of the same writes (oracle)
    labels = omasks.ring_replay(C, list(range(base, t0 + rows)))
    exp_k = torch.stack([kl[:, lab - base] for lab in labels], dim=1)
    exp_v = torch.stack([vl[:, lab - base] for lab in labels], dim=1)
    assert torch.equal(kr.cpu().view(torch.int16), exp_k.view(torch.int16))
    assert torch.equal(vr.cpu().view(torch.int16), exp_v.view(torch.int16))
    plan = plan_for(rows, live, Hq, Hkv, D, "window", first_pos=t0, window=W, ring_slots=C,
                    scale=1 / math.sqrt(D))
    out, lse, ws = run(plan, q.to(DEV), kr, vr, s.to(DEV))
    # oracle: its own ring from the linear data, replaying the same positions
    ring_k = np.zeros((Hkv, C, D))
    ring_v = np.zeros((Hkv, C, D))
    for pos in range(base, t0 + rows):
        ring_k[:, pos % C] = f64(kl[:, pos - base])
        ring_v[:, pos % C] = f64(vl[:, pos - base])
    p = Problem("window", rows, live, first_pos=t0, window=W, ring_slots=C)
    ro, rl = oattn.verify_attn_ref(p, f64(q), oattn.Cache(ring_k, ring_v, ring_slots=C), plan.problem.scale, f64(s))
    check(out, lse, ro, rl, live, f"config3 t0={t0}")


@pytest.mark.parametrize("P,with_sink", [(2048, False), (8192, False), (32768, False), (8192, True)])
def test_config4_tree(P, with_sink):
    """16-node random best-first tree, 24 q heads / 4 KV heads, D 128."""
    g = synth.gen(4000 + P // 1024 + (7 if with_sink else 0))
    parent = synth.random_tree(16, g)
    plan, kw, q, k, v, s = linear_case(int(g.initial_seed()) + 1, 16, 16, 24, 4, 128, "tree", prefix_len=P,
                                       parent=parent, sink=with_sink)
    out, lse, ws, ro, rl, p, cache = gpu_and_oracle(plan, kw, q, k, v, s)
    check(out, lse, ro, rl, 16, f"config4 P={P} sink={with_sink} S={plan.splits}")


def _q_rounding_bound(q_rot, keys_dec, scale, vis_hi):
    """Upper bound on |score(bf16-rounded q') - score(q')| over every key a row
    can see: scale * sum_d |q'_d| 2^-8 |k_d| (bf16 keeps 8 significant bits)."""
    qa = np.abs(q_rot) * 2.0 ** -8                      # [R, Hq, D]
    ka = np.abs(keys_dec[:, :vis_hi])                   # [Hkv, L, D]
    Hkv = ka.shape[0]
    G = q_rot.shape[1] // Hkv
    out = np.zeros(q_rot.shape[:2])
    for h in range(q_rot.shape[1]):
        out[:, h] = scale * (qa[:, h] @ ka[h // G].T).max(axis=1)
    return out


@pytest.mark.parametrize("P,live", [(65536, 16), (4000, 9), (3001, 11)])
def test_config5_quantized_tree(P, live):
    """Config 4's tree and heads at 64K: keys E4M3 after the 128-point WHT,
    values INT8 with one FP32 scale per (token, head).  The shorter cases
    leave some 16-row blocks of the 96 matrix rows without a live row (54
    and 66 live matrix rows)."""
    rows, Hq, Hkv, D = 16, 24, 4, 128
    g = synth.gen(5000 + (P % 997) + live)
    parent = synth.random_tree(rows, g)
    cap = P + rows + 64
    hi = P + live
    q = synth.normal_bf16((rows, Hq, D), g)
    k_raw = synth.normal_f32((Hkv, hi, D), g).double().numpy()
    k_codes = ocodec.e4m3_encode(ocodec.wht(k_raw))
    v_raw = synth.normal_f32((Hkv, hi, D), g).double().numpy()
    v_codes, v_sc = ocodec.i8_encode(v_raw)
    k_store = torch.full((Hkv, cap, D), 0x7F, dtype=torch.uint8)       # NaN codes beyond the extent
    v_store = torch.zeros((Hkv, cap, D), dtype=torch.int8)
    sc_store = torch.full((Hkv, cap), NAN, dtype=torch.float32)
    k_store[:, :hi] = torch.from_numpy(k_codes)
    v_store[:, :hi] = torch.from_numpy(v_codes)
    sc_store[:, :hi] = torch.from_numpy(v_sc)
    plan = plan_for(rows, live, Hq, Hkv, D, "tree", kv_fmt="e4m3_wht_i8", prefix_len=P, parent=parent,
                    kv_capacity=cap, scale=1 / math.sqrt(D))
    out, lse, ws = run(plan, q.to(DEV), k_store.to(DEV), v_store.to(DEV), None, sc_store.to(DEV))
    k_dec = ocodec.e4m3_decode(k_codes)
    v_dec = ocodec.i8_decode(v_codes, v_sc)
    q_rot = ocodec.wht(f64(q))
    p = Problem("tree", rows, live, prefix_len=P, parent=parent)
    ro, rl = oattn.verify_attn_ref(p, q_rot, oattn.Cache(k_dec, v_dec), plan.problem.scale)
    bound = TOL_LSE + _q_rounding_bound(q_rot, k_dec, plan.problem.scale, hi)
    check(out, lse, ro, rl, live, f"config5 P={P} live={live} S={plan.splits}", lse_tol=bound)


@pytest.mark.parametrize("call", [0, 1, 2])
def test_quantized_decode_every_code(call):
    """Every finite E4M3 key code and every INT8 value through the kernel.

    A star tree over an empty prefix makes row r see key r alone.  Query
    q = H[:, i] / 8 (exact in bf16) rotates to sqrt(2) e_i, so row r, head h
    reads one coordinate i of its key: lse = scale * sqrt(2) * decode(code),
    up to the bf16 rounding of sqrt(2) (relative 2^-8); a wrong decode is off
    by at least one E4M3 step (relative 2^-3).  Values carry scale 1, so the
    output equals the INT8 codes exactly."""
    rows, Hq, Hkv, D = 16, 6, 1, 128
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.int64)
    H = ocodec.hadamard(D)
    # coordinate read by (row r, head h), and the code placed there
    coord = np.zeros((rows, Hq), dtype=np.int64)
    k_codes = np.zeros((Hkv, rows + 64, D), dtype=np.uint8)
    rng = np.random.default_rng(40 + call)
    k_codes[:, :rows] = rng.choice(finite, size=(Hkv, rows, D)).astype(np.uint8)
    q = np.zeros((rows, Hq, D))
    want = []
    for r in range(rows):
        for h in range(Hq):
            idx = call * rows * Hq + r * Hq + h
            i = (7 * idx + call) % D
            coord[r, h] = i
            k_codes[0, r, i] = finite[idx % len(finite)]
            want.append(finite[idx % len(finite)])
            q[r, h] = H[:, i] / 8.0
    if call == 2:
        assert set(want) | set(finite[:2 * rows * Hq]) >= set(finite.tolist())
    v_codes = np.zeros((Hkv, rows + 64, D), dtype=np.int8)
    v_codes[0, :rows] = ((np.arange(rows * D).reshape(rows, D) + 37 * call) % 255 - 127).astype(np.int8)
    v_sc = np.ones((Hkv, rows + 64), dtype=np.float32)
    parent = [-1] * rows
    plan = plan_for(rows, rows, Hq, Hkv, D, "tree", kv_fmt="e4m3_wht_i8", prefix_len=0, parent=parent,
                    kv_capacity=rows + 64, scale=0.01)
    qt = torch.from_numpy(q).to(torch.bfloat16)
    assert torch.equal(qt.double(), torch.from_numpy(q))              # q is exact in bf16
    out, lse, ws = run(plan, qt.to(DEV), torch.from_numpy(k_codes).to(DEV), torch.from_numpy(v_codes).to(DEV),
                       None, torch.from_numpy(v_sc).to(DEV))
    # values: exact
    o = out.double().numpy()
    for r in range(rows):
        for h in range(Hq):
            assert np.array_equal(o[r, h], v_codes[0, r].astype(np.float64)), (r, h)
    # keys: lse against scale * sqrt(2) * decoded code
    dec = ocodec.e4m3_decode(k_codes[0, :rows])
    l = lse.double().numpy()
    for r in range(rows):
        for h in range(Hq):
            ref = 0.01 * math.sqrt(2.0) * dec[r, coord[r, h]]
            tol = 1e-5 + abs(ref) * 2.0 ** -8
            assert abs(l[r, h] - ref) <= tol, (r, h, k_codes[0, r, coord[r, h]], l[r, h], ref)


# ----------------------------------------------------------------------------- exact gates

def _label_values(Hkv, n, D, base=0):
    lab = synth.position_labels(torch.arange(base, base + n), D)   # [n, D], integers < 64
    return lab.to(torch.bfloat16).unsqueeze(0).repeat(Hkv, 1, 1)


@pytest.mark.parametrize("case", ["causal", "causal_many_splits", "window", "window_small_ring", "tree", "tree96",
                                  "quant", "causal_s300", "causal_s600"])
def test_counting_partials_bit_exact(case):
    """q = 0: every visible score is 0, so each split's m = 0, l = the number
    of visible keys and O = the sum of their integer labels, all exact."""
    g = synth.gen(6000 + hash(case) % 1000)
    if case in ("causal_s300", "causal_s600"):
        # config-2 shapes with more than 256 splits: the combine's widest
        # batch, and (600) more than one round of batches per thread
        rows, live, Hq, Hkv, D = 8, 7, 6, 1, 128
        P, S = (16384, 300) if case == "causal_s300" else (32768, 600)
        kw = dict(rows=rows, live=live, mask="causal", first_pos=P)
        cap = P + rows + 64
        plan = plan_for(rows, live, Hq, Hkv, D, "causal", first_pos=P, kv_capacity=cap, splits=S)
    elif case.startswith("causal"):
        rows, live, Hq, Hkv, D, P = 8, 6, 6, 1, 64, 1000
        S = 4 if case == "causal" else 40
        kw = dict(rows=rows, live=live, mask="causal", first_pos=P)
        cap = P + rows + 64
        plan = plan_for(rows, live, Hq, Hkv, D, "causal", first_pos=P, kv_capacity=cap, splits=S)
    elif case.startswith("window"):
        rows, live, Hq, Hkv, D = 8, 7, 6, 1, 64
        W, C, t0 = (300, 320, 2000) if case == "window" else (57, 64, 999)
        kw = dict(rows=rows, live=live, mask="window", first_pos=t0, window=W, ring_slots=C)
        plan = plan_for(rows, live, Hq, Hkv, D, "window", first_pos=t0, window=W, ring_slots=C, splits=3)
    else:
        rows, live = 16, 16
        Hq, Hkv = (24, 4) if case != "tree96" else (6, 1)
        D = 128
        P = 700
        parent = synth.random_tree(16, g)
        kw = dict(rows=rows, live=live, mask="tree", prefix_len=P, parent=parent)
        cap = P + rows + 64
        fmt = "e4m3_wht_i8" if case == "quant" else "bf16"
        plan = plan_for(rows, live, Hq, Hkv, D, "tree", kv_fmt=fmt, prefix_len=P, parent=parent, kv_capacity=cap,
                        splits=5)
    q = torch.zeros((rows, Hq, D), dtype=torch.bfloat16)
    p = oracle_problem(kw)
    lo, hi = omasks.union_extent_fast(p)
    if case.startswith("window"):
        # ring holding the label of position p in slot p mod C (after the writes)
        labels_pos = omasks.ring_replay(C, list(range(max(0, t0 + rows - C), t0 + rows)))
        k = synth.normal_bf16((Hkv, C, D), g)
        v = torch.stack([synth.position_labels(torch.tensor([max(lab, 0)]), D)[0] for lab in labels_pos]).to(
            torch.bfloat16).unsqueeze(0)
        cache = oattn.Cache(f64(k), f64(v), ring_slots=C)
        out, lse, ws = run(plan, q.to(DEV), k.to(DEV), v.to(DEV))
    elif case == "quant":
        k_codes = torch.randint(0, 0x7E, (Hkv, cap, D), generator=g, dtype=torch.int64).to(torch.uint8)
        labs = synth.position_labels(torch.arange(cap), D)                  # integer labels < 64
        v_codes = labs.to(torch.int8).unsqueeze(0).repeat(Hkv, 1, 1)
        v_sc = torch.ones((Hkv, cap), dtype=torch.float32)
        out, lse, ws = run(plan, q.to(DEV), k_codes.to(DEV), v_codes.to(DEV), None, v_sc.to(DEV))
        cache = oattn.Cache(ocodec.e4m3_decode(k_codes.numpy()), ocodec.i8_decode(v_codes.numpy(), v_sc.numpy()))
    else:
        k = synth.normal_bf16((Hkv, cap, D), g)
        v = _label_values(Hkv, cap, D)
        k[:, hi:] = NAN
        v[:, hi:] = NAN
        cache = oattn.Cache(f64(k[:, :hi]), f64(v[:, :hi]))
        out, lse, ws = run(plan, q.to(DEV), k.to(DEV), v.to(DEV))
    m_g, l_g, O_g = partials(plan, ws)
    m_o, l_o, O_o = oattn.split_partials(p, np.zeros((rows, Hq, D)), cache, plan.problem.scale, plan.splits)
    assert np.array_equal(m_g[:, :live], m_o[:, :live]), case
    assert np.array_equal(l_g[:, :live], l_o[:, :live]), case
    assert np.array_equal(O_g[:, :live], O_o[:, :live]), case
    assert np.all(np.isnan(m_g[:, live:])) and np.all(np.isnan(O_g[:, live:])), f"{case}: padding partials stored"
    ro, rl = oattn.verify_attn_ref(p, np.zeros((rows, Hq, D)), cache, plan.problem.scale)
    o = out.double().numpy()
    # one FP32 division of exact integers
    assert np.all(np.abs(o[:live] - ro[:live]) <= 2 * np.spacing(np.abs(ro[:live]).astype(np.float32)))
    assert np.all(np.abs(lse.double().numpy()[:live] - rl[:live]) <= 1e-5)


@pytest.mark.parametrize("where", ["causal_next", "causal_last_visible", "window_below", "window_lowest",
                                   "tree_non_ancestor", "tree_ancestor"])
def test_spike_at_the_boundary(where):
    """One key aligned with every query (score about +20) and a value of
    100 e_0, placed just outside (leak) or just inside (exclusion) a row's
    visible set."""
    g = synth.gen(7000 + hash(where) % 1000)
    D, Hq, Hkv = 64, 6, 1
    u = synth.normal_f32((D,), g)
    u = u / u.norm()
    if where.startswith("causal"):
        rows, live, P = 8, 6, 300
        kw = dict(rows=rows, live=live, mask="causal", first_pos=P)
        cap = P + rows + 64
        target = P + 2 + (1 if where == "causal_next" else 0)          # row 2 sees up to P + 2
        plan = plan_for(rows, live, Hq, Hkv, D, "causal", first_pos=P, kv_capacity=cap, splits=3)
    elif where.startswith("window"):
        rows, live, t0, W = 8, 6, 700, 200
        kw = dict(rows=rows, live=live, mask="window", first_pos=t0, window=W)
        cap = t0 + rows + 64
        target = t0 + 3 - W + (0 if where == "window_below" else 1)    # row 3 sees t0+3-W+1 .. t0+3
        plan = plan_for(rows, live, Hq, Hkv, D, "window", first_pos=t0, window=W, kv_capacity=cap, splits=3)
    else:
        rows, live, P = 16, 16, 260
        parent = [-1, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 5, 6, 6, 7]
        kw = dict(rows=rows, live=live, mask="tree", prefix_len=P, parent=parent)
        cap = P + rows + 64
        # node 9 (parent 4, grandparent 1, root 0): node 5 is not an ancestor, node 4 is
        target = P + (5 if where == "tree_non_ancestor" else 4)
        plan = plan_for(rows, live, Hq, Hkv, D, "tree", prefix_len=P, parent=parent, kv_capacity=cap, splits=3)
    q = (u.unsqueeze(0).unsqueeze(0).repeat(rows, Hq, 1) * 8).to(torch.bfloat16)
    k = synth.normal_bf16((Hkv, cap, D), g)
    v = synth.normal_bf16((Hkv, cap, D), g)
    k[0, target] = (u * 20 * math.sqrt(D) / 8).to(torch.bfloat16)
    v[0, target] = 0
    v[0, target, 0] = 100
    p = oracle_problem(kw)
    lo, hi = omasks.union_extent_fast(p)
    k[:, hi:] = NAN
    v[:, hi:] = NAN
    s = synth.normal_f32((Hq,), g)
    out, lse, ws, ro, rl, p, cache = gpu_and_oracle(plan, kw, q, k, v, s)
    check(out, lse, ro, rl, live, f"spike {where}")


def test_poisoned_tail_is_never_read():
    """NaN beyond the extent gives bit-identical results to a zero tail."""
    plan, kw, q, k, v, s = linear_case(8001, 8, 5, 6, 1, 128, "causal", first_pos=5000, splits=7)
    k0, v0 = k.clone(), v.clone()
    hi = 5000 + 5
    k0[:, hi:] = 0
    v0[:, hi:] = 0
    a = run(plan, q.to(DEV), k.to(DEV), v.to(DEV), s.to(DEV))
    b = run(plan, q.to(DEV), k0.to(DEV), v0.to(DEV), s.to(DEV))
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def test_deterministic_repeat():
    plan, kw, q, k, v, s = linear_case(8002, 8, 8, 6, 1, 128, "causal", first_pos=20000)
    a = run(plan, q.to(DEV), k.to(DEV), v.to(DEV), s.to(DEV))
    b = run(plan, q.to(DEV), k.to(DEV), v.to(DEV), s.to(DEV))
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def test_graph_replay_matches_eager():
    """Split + combine captured in a HIP graph: every replay, with eager work
    and synchronisations between replays, equals the eager launch bit for bit."""
    plan, kw, q, k, v, s = linear_case(8003, 8, 6, 6, 1, 128, "causal", first_pos=9000)
    q, k, v, s = q.to(DEV), k.to(DEV), v.to(DEV), s.to(DEV)
    ws = va.workspace_for(plan, DEV)
    out = torch.empty((plan.rows, plan.q_heads, plan.head_dim), dtype=torch.float32, device=DEV)
    lse = torch.empty((plan.rows, plan.q_heads), dtype=torch.float32, device=DEV)
    va.verify_attn_split(plan, q, k, v, ws)
    va.verify_attn_combine(plan, ws, out, lse=lse, sink=s)
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        va.verify_attn_split(plan, q, k, v, ws)
        va.verify_attn_combine(plan, ws, out, lse=lse, sink=s)
    for rep in range(4):
        out.fill_(NAN)
        lse.fill_(NAN)
        ws.fill_(NAN)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref_o.view(torch.int32)), f"replay {rep}: out differs"
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), f"replay {rep}: lse differs"
        # eager work between replays
        o2, l2, _ = run(plan, q, k, v, s)
        assert torch.equal(o2.view(torch.int32), ref_o.cpu().view(torch.int32))


@pytest.mark.parametrize("mask", ["causal", "tree"])
def test_append_invariance(mask):
    """Changing keys and values a row does not see leaves that row's output
    bit-identical (stability under appended tokens)."""
    if mask == "causal":
        plan, kw, q, k, v, s = linear_case(8003, 8, 8, 6, 1, 128, "causal", first_pos=3000, splits=5)
        row = 2
    else:
        par = [-1, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 5, 6, 6, 7]
        plan, kw, q, k, v, s = linear_case(8004, 16, 16, 24, 4, 128, "tree", prefix_len=3000, parent=par,
                                           splits=5)
        row = 9
    p = oracle_problem(kw)
    lo, hi = omasks.union_extent_fast(p)
    k2, v2 = k.clone(), v.clone()
    g = synth.gen(8005)
    for j in range(lo, hi):
        if not omasks.visible(p, row, j):
            k2[:, j] = synth.normal_bf16((k.shape[0], k.shape[2]), g) * 3
            v2[:, j] = synth.normal_bf16((k.shape[0], k.shape[2]), g) * 3
    a = run(plan, q.to(DEV), k.to(DEV), v.to(DEV), s if s is None else s.to(DEV))
    b = run(plan, q.to(DEV), k2.to(DEV), v2.to(DEV), s if s is None else s.to(DEV))
    assert torch.equal(a[0][row].view(torch.int32), b[0][row].view(torch.int32))
    assert torch.equal(a[1][row].view(torch.int32), b[1][row].view(torch.int32))
    assert not torch.equal(a[0].view(torch.int32), b[0].view(torch.int32))   # other rows did change


# ----------------------------------------------------------------------------- edge cases

def test_all_padding_rows():
    plan, kw, q, k, v, s = linear_case(9001, 8, 0, 6, 1, 64, "causal", first_pos=500)
    out, lse, ws = run(plan, q.to(DEV), k.to(DEV), v.to(DEV), s.to(DEV))
    assert torch.all(out == 0) and torch.all(lse == -math.inf)


def test_single_visible_key_is_exact():
    """Row 0 at position 0 sees key 0 only; without a sink o = v_0 exactly."""
    plan, kw, q, k, v, s = linear_case(9002, 8, 1, 6, 1, 128, "causal", first_pos=0, sink=False)
    out, lse, ws = run(plan, q.to(DEV), k.to(DEV), v.to(DEV))
    assert torch.equal(out[0], v[0, 0].float().unsqueeze(0).repeat(6, 1))
    sc = (q[0].double() @ k[0, 0].double()) / math.sqrt(128)
    assert torch.all((lse[0].double() - sc).abs() <= 1e-5)


@pytest.mark.parametrize("rows,live,Hq,Hkv,D,P,S", [
    (8, 5, 6, 1, 64, 1019, 64),     # more splits than granules: empty splits
    (16, 16, 2, 2, 64, 777, 0),     # G = 1: 16 matrix rows
    (8, 8, 8, 1, 128, 2500, 0),     # 64 matrix rows: two row groups of two blocks
    (16, 13, 5, 1, 64, 1500, 0),    # 80 matrix rows: third block of the second group empty
    (16, 16, 6, 1, 128, 63, 0),     # 96 matrix rows, context shorter than a 64-key tile
    (16, 11, 6, 1, 128, 2000, 0),   # 66 live of 96: the last wave's second block has no live row
    (16, 7, 6, 1, 128, 5000, 0),    # 42 live of 96: the middle wave half live, the last idle
    (16, 5, 6, 1, 64, 3000, 0),     # 30 live of 96 at D 64: one live wave
    (1, 1, 6, 1, 128, 4095, 0),     # a single row
    (8, 7, 6, 1, 128, 100000, 3),   # few long splits
    (8, 6, 6, 1, 128, 16384, 300),  # more than 256 splits: the combine's widest batch
    (8, 8, 6, 1, 128, 32768, 600),  # two rounds of combine batches per thread
])
def test_shapes_and_split_counts(rows, live, Hq, Hkv, D, P, S):
    plan, kw, q, k, v, s = linear_case(9100 + P, rows, live, Hq, Hkv, D, "causal", first_pos=P, splits=S)
    out, lse, ws, ro, rl, p, cache = gpu_and_oracle(plan, kw, q, k, v, s)
    check(out, lse, ro, rl, live, f"shape R{rows}/{live} Hq{Hq} Hkv{Hkv} D{D} P{P} S{plan.splits}")


@pytest.mark.parametrize("t0,W", [(3, 4096), (4000, 4096), (130, 64)])
def test_window_young_sequence_linear(t0, W):
    """Window mode on a linear cache, including rows whose window is clipped at 0."""
    plan, kw, q, k, v, s = linear_case(9200 + t0, 8, 6, 6, 1, 64, "window", first_pos=t0, window=W)
    out, lse, ws, ro, rl, p, cache = gpu_and_oracle(plan, kw, q, k, v, s)
    check(out, lse, ro, rl, 6, f"window t0={t0} W={W}")


def test_token_major_strides():
    """K/V stored token-major [slots, Hkv, D] and passed as a strided view."""
    g = synth.gen(9301)
    rows, live, Hq, Hkv, D, P = 16, 16, 24, 4, 128, 2000
    parent = synth.random_tree(16, g)
    cap = P + rows + 64
    q = synth.normal_bf16((rows, Hq, D), g)
    kt = synth.normal_bf16((cap, Hkv, D), g)
    vt = synth.normal_bf16((cap, Hkv, D), g)
    s = synth.normal_f32((Hq,), g)
    plan = plan_for(rows, live, Hq, Hkv, D, "tree", prefix_len=P, parent=parent, kv_capacity=cap,
                    scale=1 / math.sqrt(D))
    kd, vd = kt.to(DEV).permute(1, 0, 2), vt.to(DEV).permute(1, 0, 2)
    out, lse, ws = run(plan, q.to(DEV), kd, vd, s.to(DEV))
    p = Problem("tree", rows, live, prefix_len=P, parent=parent)
    ro, rl = oattn.verify_attn_ref(p, f64(q), oattn.Cache(f64(kt.permute(1, 0, 2)), f64(vt.permute(1, 0, 2))),
                                   plan.problem.scale, f64(s))
    check(out, lse, ro, rl, live, "token-major strides")


def test_bad_arguments_raise():
    plan, kw, q, k, v, s = linear_case(9401, 8, 5, 6, 1, 64, "causal", first_pos=100)
    ws = va.workspace_for(plan)
    small = torch.empty(4, dtype=torch.float32, device=DEV)
    with pytest.raises(va.VAError):
        va.verify_attn_split(plan, q.to(DEV), k.to(DEV), v.to(DEV), small)
    with pytest.raises(ValueError):
        va.verify_attn_split(plan, q.to(DEV)[:4], k.to(DEV), v.to(DEV), ws)
    hi = plan.info["hi"]
    with pytest.raises(ValueError):  # a cache shorter than the keys the plan reads
        va.verify_attn_split(plan, q.to(DEV), k.to(DEV)[:, :hi - 1], v.to(DEV)[:, :hi - 1], ws)
    flat_k = torch.empty(k.numel() + 1, dtype=torch.bfloat16, device=DEV)
    flat_v = torch.empty(v.numel() + 1, dtype=torch.bfloat16, device=DEV)
    km = flat_k[1:].view(k.shape)      # 2-byte offset: rows not 16-byte aligned
    vm = flat_v[1:].view(v.shape)
    with pytest.raises(va.VAError):
        va.verify_attn_split(plan, q.to(DEV), km, vm, ws)
