"""verify_kv_write: the rows' K/V written into a linear cache or a ring, copied
(bf16) or encoded (FP8 keys after the 128-point rotation, INT8 values with a
per-token scale).

Gates:
* bf16: the written slots equal the inputs bit for bit; every other slot keeps
  its NaN fill.
* quantised keys: against the float64 definition e4m3_encode(wht(k)).  Where
  no E4M3 rounding midpoint lies within the FP32 error bound of the rotation
  (codec.wht_f32_error_bound) the code must equal the definition's bit for
  bit; elsewhere either neighbour is accepted, and such cases must stay rare.
  A NaN key element makes the whole row's codes 0x7F.
* quantised values: codes and scales equal the oracle's INT8 rule
  (codec.i8_encode: FP32 scale max|v|/127, round-half-even codes) bit for
  bit, exact ties included; a row with NaN or an infinity has a non-finite
  scale and zero codes.
* data from the FP8 subnormal range to saturation, zero rows, signed zeros.
* end to end: tree verification over a quantised cache whose node rows were
  written by the kernel matches the oracle run on the stored bytes.
The CPU tests check the argument validation, which returns before any launch.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import speculative_decode_verify_amd as va
from speculative_decode_verify_amd import synth
from oracle import attn as oattn
from oracle import codec as ocodec
from oracle.masks import Problem

DEV = "cuda"
NAN = float("nan")
OK, INVALID, UNSUPPORTED, CAPACITY = 0, 1, 2, 3


# ----------------------------------------------------------------------------- CPU: validation

def _call(rows=8, first_pos=0, kv_heads=1, head_dim=128, kv_fmt=0, ptrs=True, v_scale=True, vss=0,
          capacity=1 << 20, ring=0, hs=1 << 20, rs=128):
    lib = va.load_library()
    p = ctypes.c_void_p(0x100000) if ptrs else None  # never dereferenced: every case returns before a launch
    return lib.verify_kv_write(p, p, rows, first_pos, kv_heads, head_dim, kv_fmt, p, p,
                               ctypes.c_void_p(0x100000) if v_scale else None, vss, capacity, ring, hs, rs, None)


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1), INVALID), (dict(rows=4097), INVALID), (dict(kv_heads=0), INVALID),
    (dict(head_dim=96), INVALID), (dict(kv_fmt=7), INVALID), (dict(first_pos=-1), INVALID),
    (dict(kv_fmt=1, head_dim=64, rs=64), UNSUPPORTED), (dict(ring=100), INVALID), (dict(ring=4), INVALID),
    (dict(rows=0, ptrs=False), OK), (dict(ptrs=False), INVALID), (dict(rs=64), INVALID),
    (dict(rs=132), INVALID), (dict(hs=-128), INVALID), (dict(kv_fmt=1, v_scale=False), INVALID),
    (dict(kv_fmt=1, vss=-1), INVALID), (dict(capacity=7), CAPACITY), (dict(first_pos=10, capacity=17), CAPACITY),
])
def test_kv_write_argument_checks(kw, status):
    assert _call(**kw) == status


# ----------------------------------------------------------------------------- GPU helpers

def _bf16_rows(g, rows, hkv, d, scale=1.0):
    return (synth.normal_f32((rows, hkv, d), g) * scale).to(torch.bfloat16)


def _slots(first_pos, rows, ring):
    return [(first_pos + r) % ring if ring else first_pos + r for r in range(rows)]


def _expected_values(v_new):
    """Oracle INT8 codes and scales for [rows, Hkv, 128] bf16 rows."""
    return ocodec.i8_encode(v_new.double().numpy())


def _key_codes_ok(codes, k_new, name, max_undecided=2e-3):
    """Key codes [rows, Hkv, 128] against the float64 definition with the FP32
    rotation's error bound: decided codes bit-exact, the rest a neighbour."""
    kd = k_new.double().numpy()
    y = ocodec.wht(kd)
    ok, decided = ocodec.e4m3_codes_acceptable(codes, y, ocodec.wht_f32_error_bound(kd))
    bad = np.argwhere(~ok)
    assert bad.size == 0, f"{name}: key code {codes[tuple(bad[0])]:#04x} at {bad[0].tolist()} " \
                          f"for rotated value {y[tuple(bad[0])]!r}"
    # exact zeros (zero rows, keys that rotate onto one coordinate) are
    # undecided only in the sign of zero; the rest must stay rare
    finite = ~np.isnan(y) & (y != 0)
    assert (~decided & finite).sum() <= max(2, max_undecided * finite.sum()), f"{name}: too many undecided codes"
    return int((~decided & finite).sum())


# ----------------------------------------------------------------------------- GPU: bf16

@pytest.mark.gpu
@pytest.mark.parametrize("ring,first_pos,d,hkv", [(0, 1019, 64, 1), (0, 70000, 128, 4), (4160, 4157, 64, 1),
                                                  (4160, 194560, 128, 2)])
def test_bf16_write_is_a_copy(ring, first_pos, d, hkv):
    rows = 8
    g = synth.gen(7000 + first_pos % 97)
    k_new, v_new = _bf16_rows(g, rows, hkv, d), _bf16_rows(g, rows, hkv, d)
    slots = ring if ring else first_pos + rows + 5
    kc = torch.full((hkv, slots, d), NAN, dtype=torch.bfloat16, device=DEV)
    vc = torch.full((hkv, slots, d), NAN, dtype=torch.bfloat16, device=DEV)
    va.verify_kv_write(k_new.to(DEV), v_new.to(DEV), first_pos, kc, vc, ring_slots=ring)
    torch.cuda.synchronize()
    kc, vc = kc.cpu(), vc.cpu()
    written = _slots(first_pos, rows, ring)
    for r, s in enumerate(written):
        assert torch.equal(kc[:, s].view(torch.int16), k_new[r].view(torch.int16))
        assert torch.equal(vc[:, s].view(torch.int16), v_new[r].view(torch.int16))
    rest = torch.ones(slots, dtype=torch.bool)
    rest[written] = False
    assert torch.isnan(kc[:, rest].float()).all() and torch.isnan(vc[:, rest].float()).all()


# ----------------------------------------------------------------------------- GPU: quantised

def _quant_write(k_new, v_new, first_pos, ring, token_major=False):
    rows, hkv, d = k_new.shape
    slots = ring if ring else first_pos + rows + 3
    if token_major:
        k8 = torch.full((slots, hkv, d), 0x7F, dtype=torch.uint8, device=DEV).permute(1, 0, 2)
        v8 = torch.full((slots, hkv, d), 0x55, dtype=torch.uint8, device=DEV).view(torch.int8).permute(1, 0, 2)
    else:
        k8 = torch.full((hkv, slots, d), 0x7F, dtype=torch.uint8, device=DEV)
        v8 = torch.full((hkv, slots, d), 0x55, dtype=torch.uint8, device=DEV).view(torch.int8)
    vs = torch.full((hkv, slots), NAN, dtype=torch.float32, device=DEV)
    va.verify_kv_write(k_new.to(DEV), v_new.to(DEV), first_pos, k8, v8, v_scale=vs, ring_slots=ring)
    torch.cuda.synchronize()
    return k8.cpu(), v8.cpu(), vs.cpu()


def _check_quant(k_new, v_new, first_pos, ring, name, token_major=False):
    k8, v8, vs = _quant_write(k_new, v_new, first_pos, ring, token_major)
    vc, sc = _expected_values(v_new)
    written = _slots(first_pos, k_new.shape[0], ring)
    got_k = np.stack([k8[:, s].numpy() for s in written])   # [rows, Hkv, 128]
    _key_codes_ok(got_k, k_new, name)
    for r, s in enumerate(written):
        assert np.array_equal(v8[:, s].numpy(), vc[r]), f"{name}: value codes differ at row {r}"
        got_s = vs[:, s].numpy()
        fin = ~np.isnan(sc[r])
        assert np.array_equal(np.isnan(got_s), ~fin), f"{name}: NaN scales differ at row {r}"
        assert np.array_equal(got_s[fin].view(np.int32), sc[r][fin].view(np.int32)), f"{name}: scale differs"
    rest = np.ones(k8.shape[1], dtype=bool)
    rest[written] = False
    assert (k8[:, rest] == 0x7F).all() and (v8[:, rest].view(torch.uint8) == 0x55).all()
    assert torch.isnan(vs[:, rest]).all()
    return k8, v8, vs


@pytest.mark.gpu
@pytest.mark.parametrize("scale", [1.0, 1e-3, 2.0 ** -12, 40.0, 3000.0])
def test_quant_codes_match_the_oracle(scale):
    """Random rows at magnitudes from the FP8 subnormal range to saturation."""
    g = synth.gen(7100 + int(math.log2(scale) + 20))
    rows, hkv = 16, 4
    _check_quant(_bf16_rows(g, rows, hkv, 128, scale), _bf16_rows(g, rows, hkv, 128, scale), 65536, 0,
                 f"scale {scale}")


@pytest.mark.gpu
def test_quant_codes_special_rows():
    """Zero rows (scale 0, all codes 0), signed zeros, one-hot keys, keys that
    rotate onto one coordinate (a Hadamard column: a single saturated code),
    and values with one large entry."""
    rows, hkv, d = 8, 2, 128
    k = torch.zeros((rows, hkv, d), dtype=torch.float32)
    v = torch.zeros((rows, hkv, d), dtype=torch.float32)
    k[1] = -0.0
    v[1] = -0.0
    k[2, :, 7] = 3.0
    k[3, 0] = torch.from_numpy(ocodec.hadamard(128)[:, 9] * 50.0).float()
    k[3, 1] = torch.from_numpy(ocodec.hadamard(128)[:, 100] * -0.001).float()
    v[4, :, 3] = 1000.0
    v[4, :, 4] = -1.0
    g = synth.gen(7200)
    k[5:] = synth.normal_f32((3, hkv, d), g)
    v[5:] = synth.normal_f32((3, hkv, d), g) * 1e-30
    _check_quant(k.to(torch.bfloat16), v.to(torch.bfloat16), 100, 0, "special")


@pytest.mark.gpu
def test_quant_value_ties_round_half_even():
    """Exact INT8 ties: a row with max 127 has scale 1 and one with max 63.5
    scale 0.5, so v / s = +-0.5, 1.5, 2.5, 3.5, 126.5 are exact halves and
    round to the even code (0, 2, 2, 4, 126), not away from zero."""
    rows, hkv, d = 2, 1, 128
    v = torch.zeros((rows, hkv, d), dtype=torch.float32)
    v[0, 0, :12] = torch.tensor([127, 0.5, 1.5, 2.5, 3.5, 126.5, -0.5, -1.5, -2.5, -3.5, -126.5, 0.25])
    v[1, 0, :8] = torch.tensor([63.5, 0.25, 0.75, 1.25, -0.25, -0.75, -1.25, 63.25])
    k = synth.normal_f32((rows, hkv, d), synth.gen(7250))
    k8, v8, vs = _check_quant(k.to(torch.bfloat16), v.to(torch.bfloat16), 40, 0, "ties")
    assert vs[0, 40].item() == 1.0 and vs[0, 41].item() == 0.5
    assert v8[0, 40, :12].tolist() == [127, 0, 2, 2, 4, 126, 0, -2, -2, -4, -126, 0]
    assert v8[0, 41, :8].tolist() == [127, 0, 2, 2, 0, -2, -2, 126]


@pytest.mark.gpu
def test_quant_non_finite_rows():
    """A NaN key element reaches every rotated coordinate: the whole row's
    codes are 0x7F, as the definition's.  A value row holding NaN or an
    infinity stores a NaN or infinite scale and zero codes."""
    rows, hkv, d = 4, 2, 128
    g = synth.gen(7260)
    k = synth.normal_f32((rows, hkv, d), g)
    v = synth.normal_f32((rows, hkv, d), g)
    k[0, 1, 17] = float("nan")
    v[1, 0, 3] = float("nan")
    v[2, 1, 100] = -float("inf")
    k8, v8, vs = _check_quant(k.to(torch.bfloat16), v.to(torch.bfloat16), 9, 0, "non-finite")
    assert (k8[1, 9] == 0x7F).all()
    assert torch.isnan(vs[0, 10]) and torch.isinf(vs[1, 11])
    assert (v8[0, 10] == 0).all() and (v8[1, 11] == 0).all()


@pytest.mark.gpu
@pytest.mark.parametrize("first_pos", [4157, 194560])
def test_quant_ring_and_token_major(first_pos):
    g = synth.gen(7300 + first_pos % 13)
    rows, hkv = 8, 1
    k, v = _bf16_rows(g, rows, hkv, 128), _bf16_rows(g, rows, hkv, 128)
    _check_quant(k, v, first_pos, 4160, "ring")
    _check_quant(k, v, first_pos, 0, "linear token-major", token_major=True)


@pytest.mark.gpu
def test_tree_verify_reads_rows_written_by_the_encoder():
    """Config 5's shape at a 4K prefix: the prefix is encoded by the oracle,
    the 16 node rows by verify_kv_write, then the tree is verified; the
    oracle reads the same stored bytes."""
    P, rows, live, Hq, Hkv, D = 4096, 16, 16, 24, 4, 128
    g = synth.gen(7400)
    parent = synth.random_tree(rows, g)
    cap = P + rows + 64
    q = synth.normal_bf16((rows, Hq, D), g)
    k_pre = synth.normal_f32((Hkv, P, D), g).double().numpy()
    v_pre = synth.normal_f32((Hkv, P, D), g).double().numpy()
    k_nodes, v_nodes = _bf16_rows(g, rows, Hkv, D), _bf16_rows(g, rows, Hkv, D)
    k8 = torch.full((Hkv, cap, D), 0x7F, dtype=torch.uint8)
    v8 = torch.zeros((Hkv, cap, D), dtype=torch.int8)
    vs = torch.full((Hkv, cap), NAN, dtype=torch.float32)
    k8[:, :P] = torch.from_numpy(ocodec.e4m3_encode(ocodec.wht(k_pre)))
    vc, sc = ocodec.i8_encode(v_pre)
    v8[:, :P] = torch.from_numpy(vc)
    vs[:, :P] = torch.from_numpy(sc)
    k8, v8, vs = k8.to(DEV), v8.to(DEV), vs.to(DEV)
    va.verify_kv_write(k_nodes.to(DEV), v_nodes.to(DEV), P, k8, v8, v_scale=vs)
    plan = va.Plan(rows=rows, live_rows=live, q_heads=Hq, kv_heads=Hkv, head_dim=D, mask="tree",
                   kv_fmt="e4m3_wht_i8", prefix_len=P, parent=parent, kv_capacity=cap, scale=1 / math.sqrt(D))
    ws = torch.full(((plan.workspace_bytes + 3) // 4,), NAN, dtype=torch.float32, device=DEV)
    out = torch.full((rows, Hq, D), NAN, dtype=torch.float32, device=DEV)
    lse = torch.full((rows, Hq), NAN, dtype=torch.float32, device=DEV)
    va.verify_attn_split(plan, q.to(DEV), k8, v8, ws, v_scale=vs)
    va.verify_attn_combine(plan, ws, out, lse=lse)
    torch.cuda.synchronize()
    hi = P + live
    k_dec = ocodec.e4m3_decode(k8[:, :hi].cpu().numpy())
    v_dec = ocodec.i8_decode(v8[:, :hi].cpu().numpy(), vs[:, :hi].cpu().numpy())
    # the node rows the kernel wrote are the definition's codes
    _key_codes_ok(k8[:, P:hi].cpu().numpy().transpose(1, 0, 2), k_nodes, "tree nodes")
    vcn, scn = _expected_values(v_nodes)
    assert np.array_equal(v8[:, P:hi].cpu().numpy(), vcn.transpose(1, 0, 2))
    q_rot = ocodec.wht(q.double().numpy())
    p = Problem("tree", rows, live, prefix_len=P, parent=parent)
    ro, rl = oattn.verify_attn_ref(p, q_rot, oattn.Cache(k_dec, v_dec), 1 / math.sqrt(D))
    o = out.cpu().double().numpy()
    err = np.abs(o - ro)
    assert np.all(err <= 2e-3 + 1e-2 * np.abs(ro)), f"max err {err.max():.3e}"
    # lse: scores move by at most scale * sum 2^-8 |q'||k| from rounding q' to bf16
    qa = np.abs(q_rot).reshape(-1, D)
    worst = max(float((qa @ np.abs(k_dec[gi]).T).max()) for gi in range(Hkv))
    bound = 1e-4 + (1 / math.sqrt(D)) * 2.0 ** -8 * worst
    assert np.all(np.abs(lse.cpu().double().numpy() - rl) <= bound)
