"""Pins for the float64 oracle, against things other than the oracle itself.

Pins used: a hand-worked fixture (tests/golden/hand_example.json), torch's
float64 scaled_dot_product_attention and scipy's logsumexp (library
routines), closed forms, brute-force enumeration, an independent ancestor
closure, scipy's Hadamard matrix and torch's float8_e4m3fn decoder.  The
planted-mistake tests at the end show that each pin fails for a plausible
mistake in the oracle.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch
import torch.nn.functional as F

from oracle import attn, codec, masks
from oracle.masks import Problem, CAUSAL, WINDOW, TREE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    if x is None:
        return None
    if isinstance(x, str):
        assert x.startswith("ln")
        return math.log(float(x[2:]))
    return float(x)


# ---------------------------------------------------------------- hand-worked fixture

def test_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    s = g["setup"]
    k = np.array([[_num(a) for a in row] for row in s["keys"]])[None]
    v = np.array(s["values"], dtype=np.float64)[None]
    cache = attn.Cache(k, v)
    for c in g["cases"]:
        if c["mask"] == TREE:
            p = Problem(TREE, rows=len(c["parent"]), live_rows=len(c["parent"]),
                        prefix_len=c["prefix_len"], parent=c["parent"])
            r = c["row"]
            q = np.tile(np.array(s["q"]), (p.rows, 1, 1))
        else:
            p = Problem(c["mask"], rows=1, live_rows=1, first_pos=c["first_pos"],
                        window=c.get("window", 0))
            r = 0
            q = np.array(s["q"])[None, None]
        sink = None if c["sink"] is None else np.array([_num(c["sink"])])
        o, lse = attn.verify_attn_ref(p, q, cache, s["scale"], sink)
        np.testing.assert_allclose(o[r, 0], c["o"], rtol=0, atol=1e-12, err_msg=c["name"])
        assert abs(lse[r, 0] - _num(c["lse"])) < 1e-12, c["name"]
        o2, lse2 = attn.verify_attn_ref_split(p, q, cache, s["scale"], 1, sink)
        np.testing.assert_allclose(o2[r, 0], c["o"], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- helpers

def _rand_case(rng, mask, R=8, live=5, Hkv=2, G=3, D=16, P=150, window=40, ring=0):
    if mask == TREE:
        parent = [-1] + [int(rng.integers(0, i)) for i in range(1, R)]
        p = Problem(TREE, R, live, prefix_len=P, parent=parent)
        n_keys = P + R
    elif mask == WINDOW:
        p = Problem(WINDOW, R, live, first_pos=P, window=window, ring_slots=ring)
        n_keys = P + R
    else:
        p = Problem(CAUSAL, R, live, first_pos=P)
        n_keys = P + R
    q = rng.standard_normal((R, Hkv * G, D))
    k = rng.standard_normal((Hkv, n_keys + 7, D))
    v = rng.standard_normal((Hkv, n_keys + 7, D))
    return p, q, attn.Cache(k, v)


MASK_CASES = [
    (CAUSAL, dict()),
    (CAUSAL, dict(live=8, P=0)),
    (CAUSAL, dict(live=1, P=63)),
    (WINDOW, dict(window=40, P=150)),
    (WINDOW, dict(window=300, P=20)),       # window reaches below position 0
    (TREE, dict(R=16, live=16, P=100)),
    (TREE, dict(R=16, live=16, P=0)),
]


# ---------------------------------------------------------------- library-routine pins

@pytest.mark.parametrize("mask,kw", MASK_CASES)
@pytest.mark.parametrize("with_sink", [False, True])
def test_definition_matches_torch_sdpa(mask, kw, with_sink):
    """Torch's float64 SDPA with a boolean mask; the sink as one extra key of
    score sigma and value zero."""
    rng = np.random.default_rng(11)
    p, q, cache = _rand_case(rng, mask, **kw)
    R, Hq, D = q.shape
    Hkv = cache.k.shape[0]
    G = Hq // Hkv
    scale = 1 / math.sqrt(D)
    sink = rng.standard_normal(Hq) if with_sink else None
    o, lse = attn.verify_attn_ref(p, q, cache, scale, sink)
    N = cache.k.shape[1]
    vis = np.array([[masks.visible(p, r, j) for j in range(N)] for r in range(R)])
    for h in range(Hq):
        g = h // G
        for r in range(p.live_rows):
            qq = torch.tensor(q[r, h])[None, None, None]             # [1,1,1,D]
            kk = torch.tensor(cache.k[g])[None, None]                 # [1,1,N,D]
            vv = torch.tensor(cache.v[g])[None, None]
            mk = torch.tensor(vis[r])[None, None, None]
            if with_sink:
                # a key whose score is exactly sigma (q . k_extra * scale = sigma)
                k_extra = torch.zeros(1, 1, 1, D, dtype=torch.float64)
                qq2 = torch.cat([qq, torch.ones(1, 1, 1, 1, dtype=torch.float64)], -1)
                kk2 = torch.cat([kk, torch.zeros(1, 1, N, 1, dtype=torch.float64)], -1)
                k_extra = torch.cat([k_extra, torch.full((1, 1, 1, 1), sink[h] / scale, dtype=torch.float64)], -1)
                kk2 = torch.cat([kk2, k_extra], 2)
                vv2 = torch.cat([vv, torch.zeros(1, 1, 1, D, dtype=torch.float64)], 2)
                mk2 = torch.cat([mk, torch.ones(1, 1, 1, 1, dtype=torch.bool)], -1)
                ref = F.scaled_dot_product_attention(qq2, kk2, vv2, attn_mask=mk2, scale=scale)
                sc = np.concatenate([scale * (cache.k[g] @ q[r, h])[vis[r]], [sink[h]]])
            else:
                ref = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mk, scale=scale)
                sc = scale * (cache.k[g] @ q[r, h])[vis[r]]
            np.testing.assert_allclose(o[r, h], ref.numpy().reshape(D), rtol=1e-12, atol=1e-13)
            assert abs(lse[r, h] - scipy.special.logsumexp(sc)) < 1e-12
    # padding rows
    assert np.all(o[p.live_rows:] == 0) and np.all(lse[p.live_rows:] == -np.inf)


# ---------------------------------------------------------------- split form

@pytest.mark.parametrize("mask,kw", MASK_CASES)
def test_split_form_equals_definition(mask, kw):
    rng = np.random.default_rng(5)
    p, q, cache = _rand_case(rng, mask, **kw)
    scale = 1 / math.sqrt(q.shape[-1])
    sink = rng.standard_normal(q.shape[1])
    o, lse = attn.verify_attn_ref(p, q, cache, scale, sink)
    lo, hi = masks.union_extent_fast(p)
    T = -(-hi // 64) - lo // 64
    for S in sorted({1, 2, 3, 4, 7, 64, T}):
        o2, lse2 = attn.verify_attn_ref_split(p, q, cache, scale, S, sink)
        np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse2[np.isfinite(lse)], lse[np.isfinite(lse)], rtol=1e-13)


def test_split_form_random_long():
    """Several 32-key granules and a ragged tail, splits that leave some empty."""
    rng = np.random.default_rng(6)
    p, q, cache = _rand_case(rng, CAUSAL, R=8, live=6, Hkv=1, G=6, D=8, P=1000)
    o, lse = attn.verify_attn_ref(p, q, cache, 0.3, None)
    for S in (5, 16, 17, 40):
        o2, lse2 = attn.verify_attn_ref_split(p, q, cache, 0.3, S, None)
        np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- closed forms

def test_single_visible_key_gives_that_value():
    rng = np.random.default_rng(1)
    p = Problem(CAUSAL, rows=8, live_rows=1, first_pos=0)      # row 0 sees key 0 only
    q = rng.standard_normal((8, 6, 64))
    k = rng.standard_normal((1, 16, 64))
    v = rng.standard_normal((1, 16, 64))
    o, lse = attn.verify_attn_ref(p, q, attn.Cache(k, v), 0.125)
    for h in range(6):
        assert np.array_equal(o[0, h], v[0, 0])
        assert abs(lse[0, h] - 0.125 * q[0, h] @ k[0, 0]) < 1e-14


def test_zero_query_mean_and_sink():
    """q = 0: every visible score is 0, o = sum v / (n + e^sigma), lse = ln(n + e^sigma)."""
    rng = np.random.default_rng(2)
    p = Problem(WINDOW, rows=8, live_rows=5, first_pos=90, window=30)
    q = np.zeros((8, 6, 8))
    k = rng.standard_normal((1, 100, 8))
    v = rng.standard_normal((1, 100, 8))
    sink = rng.standard_normal(6)
    o, lse = attn.verify_attn_ref(p, q, attn.Cache(k, v), 1.0, sink)
    for r in range(5):
        t = 90 + r
        vis = list(range(t - 29, t + 1))
        for h in range(6):
            den = len(vis) + math.exp(sink[h])
            np.testing.assert_allclose(o[r, h], v[0, vis].sum(0) / den, rtol=1e-13)
            assert abs(lse[r, h] - math.log(den)) < 1e-13


def test_empty_context_with_sink_gives_zero():
    """Every split empty, sink present: o = 0 and lse = sigma (sink alone)."""
    S, R, Hq, D = 3, 2, 4, 8
    m = np.full((S, R, Hq), -np.inf)
    l = np.zeros((S, R, Hq))
    O = np.zeros((S, R, Hq, D))
    sink = np.array([0.5, -1.0, 2.0, 0.0])
    o, lse = attn.combine(m, l, O, live_rows=R, sink=sink)
    assert np.all(o == 0)
    np.testing.assert_allclose(lse, np.tile(sink, (R, 1)), rtol=0, atol=1e-15)
    o, lse = attn.combine(m, l, O, live_rows=R, sink=None)
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_all_padding_problem():
    p = Problem(CAUSAL, rows=8, live_rows=0, first_pos=10)
    q = np.ones((8, 6, 8))
    c = attn.Cache(np.ones((1, 20, 8)), np.ones((1, 20, 8)))
    o, lse = attn.verify_attn_ref(p, q, c, 1.0, np.zeros(6))
    assert np.all(o == 0) and np.all(lse == -np.inf)
    assert masks.union_extent_fast(p) == (0, 0)


def test_identical_keys_closed_form():
    """n identical visible keys with score s: o = v * n e^s / (n e^s + e^sigma)."""
    p = Problem(CAUSAL, rows=1, live_rows=1, first_pos=9)
    D = 4
    k = np.tile(np.array([0.5, -0.25, 1.0, 2.0]), (1, 12, 1))
    v = np.tile(np.array([1.0, 2.0, -3.0, 4.0]), (1, 12, 1))
    q = np.array([[[1.0, 1.0, 1.0, 1.0]]])
    s = 0.7 * 3.25
    sig = 1.5
    o, lse = attn.verify_attn_ref(p, q, attn.Cache(k, v), 0.7, np.array([sig]))
    n = 10
    np.testing.assert_allclose(o[0, 0], v[0, 0] * n * math.exp(s) / (n * math.exp(s) + math.exp(sig)), rtol=1e-14)
    assert abs(lse[0, 0] - math.log(n * math.exp(s) + math.exp(sig))) < 1e-13


# ---------------------------------------------------------------- masks

def _ancestors_by_closure(parent):
    """Reflexive-transitive closure of the child->parent relation by boolean
    matrix squaring (a different algorithm from the parent walk)."""
    n = len(parent)
    a = np.eye(n, dtype=bool)
    for i, pa in enumerate(parent):
        if pa >= 0:
            a[i, pa] = True
    for _ in range(n.bit_length() + 1):
        a = a | ((a.astype(np.int64) @ a.astype(np.int64)) > 0)
    return [sum(1 << j for j in range(n) if a[i, j]) for i in range(n)]


def test_tree_ancestors_vs_closure():
    rng = np.random.default_rng(3)
    for _ in range(200):
        n = int(rng.integers(1, 17))
        parent = [-1] + [int(rng.integers(-1, i)) for i in range(1, n)]
        assert masks.tree_ancestors(parent) == _ancestors_by_closure(parent)


def test_chain_tree_is_causal_and_star_tree_is_prefix_plus_self():
    P = 77
    chain = Problem(TREE, 16, 16, prefix_len=P, parent=[-1] + list(range(15)))
    causal = Problem(CAUSAL, 16, 16, first_pos=P)
    star = Problem(TREE, 16, 16, prefix_len=P, parent=[-1] * 16)
    for r in range(16):
        assert masks.visible_keys(chain, r) == masks.visible_keys(causal, r)
        assert masks.visible_keys(star, r) == list(range(P)) + [P + r]


@pytest.mark.parametrize("mask,kw", MASK_CASES)
def test_visible_matrix_and_extent_vs_enumeration(mask, kw):
    rng = np.random.default_rng(4)
    p, _, _ = _rand_case(rng, mask, **kw)
    lo, hi = masks.union_extent(p)
    assert masks.union_extent_fast(p) == (lo, hi)
    vm = masks.visible_matrix(p, 0, hi + 70)
    for r in range(p.rows):
        assert list(np.nonzero(vm[r])[0]) == masks.visible_keys(p, r)


def test_window_counts():
    for t0 in (0, 1, 5, 4094, 4095, 4096, 5000):
        p = Problem(WINDOW, 8, 8, first_pos=t0, window=4096)
        for r in range(8):
            t = t0 + r
            keys = masks.visible_keys(p, r)
            assert len(keys) == min(4096, t + 1)
            assert keys[-1] == t and keys[0] == max(0, t - 4095)


@pytest.mark.parametrize("lo,hi", [(0, 1), (0, 32), (0, 64), (0, 1024), (0, 1029), (970, 5100), (5, 6),
                                   (31, 33), (63, 65)])
def test_split_ranges_partition(lo, hi):
    C = -(-hi // 32) - lo // 32
    for S in (1, 2, 3, 4, 8, C, C + 3):
        rr = masks.split_key_ranges(lo, hi, S)
        assert len(rr) == S
        covered = [j for a, b in rr for j in range(a, b)]
        assert covered == list(range(lo, hi))
        chunks = []
        for a, b in rr:
            if b > a:
                if a != lo:
                    assert a % 32 == 0
                if b != hi:
                    assert b % 32 == 0
                chunks.append(-(-b // 32) - a // 32)
            else:
                chunks.append(0)
        assert max(chunks) - min(chunks) <= 1
        # the first splits take the extra chunk
        assert chunks == sorted(chunks, reverse=True)


# ---------------------------------------------------------------- ring

def _ring_check(C, W, R, t0):
    """Position labels: history [t0 - C, t0) then R new rows; does every live
    row find the label of every position in its window?"""
    events = list(range(max(0, t0 - C), t0)) + list(range(t0, t0 + R))
    labels = masks.ring_replay(C, events)
    p = Problem(WINDOW, R, R, first_pos=t0, window=W, ring_slots=C)
    bad = []
    for r in range(R):
        for j in masks.visible_keys(p, r):
            if labels[j % C] != j:
                bad.append((r, j))
    return bad


def test_ring_4160_keeps_every_window():
    for t0 in (5120, 51200, 194560, 4160 * 7 + 3, 12):
        assert _ring_check(4160, 4096, 8, t0) == []


def test_ring_4096_loses_history_for_row0():
    """Negative control from the IQuestRT correctness section: with exactly
    4,096 slots the later writes evict keys row 0 still needs."""
    bad = _ring_check(4096, 4096, 8, 51200)
    assert bad and all(r < 7 for r, _ in bad) and any(r == 0 for r, _ in bad)


def test_ring_equals_linear_in_oracle():
    rng = np.random.default_rng(8)
    C, W, R, t0, D = 192, 128, 8, 1000, 8
    p = Problem(WINDOW, R, 6, first_pos=t0, window=W, ring_slots=C)
    kl = rng.standard_normal((1, t0 + R, D))
    vl = rng.standard_normal((1, t0 + R, D))
    kr = np.full((1, C, D), np.nan)
    vr = np.full((1, C, D), np.nan)
    for pos in range(t0 + R):
        kr[0, pos % C] = kl[0, pos]
        vr[0, pos % C] = vl[0, pos]
    q = rng.standard_normal((R, 6, D))
    o1, l1 = attn.verify_attn_ref(p, q, attn.Cache(kl, vl), 0.4, None)
    o2, l2 = attn.verify_attn_ref(p, q, attn.Cache(kr, vr, ring_slots=C), 0.4, None)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------- codec

def test_e4m3_decode_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codec.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.nanmax(got) == 448.0 and nan.sum() == 2


def test_e4m3_encode_vs_torch_in_range():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (0.01, 1, 30, 150)])
    x = np.concatenate([x, codec.e4m3_decode(np.arange(256))[:0x7F], -codec.e4m3_decode(np.arange(0x7F))])
    x = x.astype(np.float32).astype(np.float64)              # torch rounds through fp32
    x = x[np.abs(x) < 464]
    ours = codec.e4m3_encode(x)
    ref = torch.tensor(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturates_and_midpoints():
    assert codec.e4m3_encode(np.array([1000.0, -1e9, 448.0, 470.0]))[:].tolist() == [0x7E, 0xFE, 0x7E, 0x7E]
    # 2^-10 lies halfway between 0 and the smallest subnormal 2^-9: tie to even -> 0
    assert codec.e4m3_encode(np.array([2.0 ** -10, 3 * 2.0 ** -10])).tolist() == [0x00, 0x02]
    assert codec.e4m3_encode(np.array([np.nan])).tolist() == [0x7F]


def test_e4m3_code_interval_at_midpoints():
    """1.0625 is the midpoint of 1.0 (0x38) and 1.125 (0x39): with no error
    the definition's tie-to-even code 0x38 is decided; within any error both
    neighbours are correct and nothing else is; a value far from every
    midpoint is decided; zero accepts both signed zeros; NaN only 0x7F."""
    lo, hi, dec = codec.e4m3_code_interval(np.array([1.0625, 1.0625, 1.02, 0.0, 500.0]),
                                           np.array([0.0, 1e-6, 1e-6, 1e-7, 1.0]))
    assert lo.tolist() == [0x38, 0x38, 0x38, 0x80, 0x7E]
    assert hi.tolist() == [0x38, 0x39, 0x38, 0x00, 0x7E]
    assert dec.tolist() == [True, False, True, False, True]
    y = np.array([1.0625] * 4 + [1.02] * 2 + [0.0] * 3 + [np.nan, np.nan])
    b = np.array([1e-6] * 4 + [1e-6] * 2 + [1e-7] * 3 + [0.0, 0.0])
    codes = np.array([0x38, 0x39, 0x3A, 0xB8, 0x38, 0x39, 0x00, 0x80, 0x01, 0x7F, 0xFF], np.uint8)
    ok, decided = codec.e4m3_codes_acceptable(codes, y, b)
    assert ok.tolist() == [True, True, False, False, True, False, True, True, False, True, False]
    assert decided.tolist() == [False] * 4 + [True] * 2 + [False] * 5


def _fwht_f32(x, order, scale_first):
    """An FP32 encoder's rotation, written here only to exercise the bound:
    butterflies (a, b) -> (a + b, a - b) in float32, stage widths in the
    given order, scaled by float32(1/sqrt(n)) before or after them."""
    y = np.array(x, dtype=np.float32, copy=True)
    n = y.shape[-1]
    inv = np.float32(1.0 / math.sqrt(n))
    if scale_first:
        y = y * inv
    for width in order:
        z = y.reshape(y.shape[:-1] + (n // (2 * width), 2, width))
        a, b = z[..., 0, :].copy(), z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(y.shape)
    return y if scale_first else y * inv


@pytest.mark.parametrize("order,scale_first", [((1, 2, 4, 8, 16, 32, 64), False),
                                               ((64, 32, 16, 8, 4, 2, 1), False),
                                               ((1, 2, 4, 8, 16, 32, 64), True)])
def test_wht_error_bound_covers_fp32_encoders(order, scale_first):
    """The bound holds for FP32 rotations in several evaluation orders (and
    is not vacuous: the worst error reaches a fair share of it); the codes of
    such an encoder are acceptable everywhere, and the cases left undecided
    by the bound are rare at the data's magnitudes."""
    rng = np.random.default_rng(24)
    x = (rng.standard_normal((3000, 128)) * rng.choice([2.0 ** -12, 1e-3, 1.0, 40.0, 3000.0],
                                                       size=(3000, 1))).astype(np.float32)
    y = codec.wht(x.astype(np.float64))
    got = _fwht_f32(x, order, scale_first).astype(np.float64)
    b = codec.wht_f32_error_bound(x.astype(np.float64))
    err = np.abs(got - y)
    assert np.all(err <= b)
    assert (err / b).max() > 0.05
    ok, decided = codec.e4m3_codes_acceptable(codec.e4m3_encode(got), y, b)
    assert ok.all()
    assert (~decided).mean() < 2e-3


def test_key_codes_of_a_one_hot_key():
    """A one-hot key rotates to +-c/sqrt(128) everywhere: one code magnitude,
    signs from the Hadamard column (scipy's matrix)."""
    k = np.zeros((1, 128))
    k[0, 5] = 2.0
    codes = codec.e4m3_encode(codec.wht(k))[0]
    mag = codec.e4m3_encode(np.array([2.0 / math.sqrt(128)]))[0]
    signs = scipy.linalg.hadamard(128)[:, 5] < 0
    assert np.array_equal(codes, np.where(signs, mag | 0x80, mag).astype(np.uint8))


def test_wht_vs_scipy_and_orthonormal():
    H = codec.hadamard(128)
    assert np.array_equal(H, scipy.linalg.hadamard(128))
    Hn = H / math.sqrt(128)
    np.testing.assert_allclose(Hn @ Hn.T, np.eye(128), atol=1e-14)
    rng = np.random.default_rng(10)
    q = rng.standard_normal((5, 128))
    k = rng.standard_normal((7, 128))
    np.testing.assert_allclose(codec.wht(q) @ codec.wht(k).T, q @ k.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(codec.wht(q), q @ scipy.linalg.hadamard(128).T / math.sqrt(128), rtol=1e-15, atol=1e-15)


def test_i8_codec():
    rng = np.random.default_rng(12)
    v = rng.standard_normal((4, 300, 128))
    v[1, 5] = 0.0
    codes, scale = codec.i8_encode(v)
    assert codes.dtype == np.int8 and scale.dtype == np.float32
    assert np.all(np.abs(codes.astype(int)) <= 127)
    assert np.all(codes[1, 5] == 0) and scale[1, 5] == 0
    nz = scale > 0
    assert np.all(np.abs(codes.astype(int)).max(-1)[nz] == 127)
    dq = codec.i8_decode(codes, scale)
    assert np.all(np.abs(dq - v) <= scale[..., None].astype(np.float64) * 0.5 * (1 + 1e-6))
    # dequantisation is exact: every product is a float64 without rounding
    assert np.array_equal(dq, codes.astype(np.float64) * scale.astype(np.float64)[..., None])


def test_i8_ties_round_half_even():
    """Exact ties.  A row with max 127 has s = 1 and one with max 63.5 has
    s = 0.5 (both exact in FP32), so v / s = +-0.5, 1.5, 2.5, 3.5, 126.5 are
    exact halves: round-half-even gives 0, 2, 2, 4, 126 (half away from zero
    would give 1, 2, 3, 4, 127)."""
    v = np.zeros((2, 128))
    v[0, :12] = [127, 0.5, 1.5, 2.5, 3.5, 126.5, -0.5, -1.5, -2.5, -3.5, -126.5, 0.25]
    v[1, :8] = [63.5, 0.25, 0.75, 1.25, -0.25, -0.75, -1.25, 63.25]
    codes, scale = codec.i8_encode(v)
    assert scale.tolist() == [1.0, 0.5]
    assert codes[0, :12].tolist() == [127, 0, 2, 2, 4, 126, 0, -2, -2, -4, -126, 0]
    assert codes[1, :8].tolist() == [127, 0, 2, 2, 0, -2, -2, 126]


def _fp32_round_exact(fr):
    """Correctly rounded FP32 value of a rational (nearest, ties to even),
    from exact comparisons with the neighbours of a first guess."""
    from fractions import Fraction
    f = np.float32(float(fr))
    cands = {f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))}
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(np.array(c).view(np.int32)) & 1))
    return best


def test_i8_codes_equal_exact_rational_rounding():
    """Scale and codes against exact rational arithmetic: s = the correctly
    rounded FP32 of max|v| / 127, code = the integer nearest v / s (ties to
    even), clamped -- no float64 division involved."""
    from fractions import Fraction
    rng = np.random.default_rng(25)
    v = (rng.standard_normal((48, 128)) * rng.choice([1e-3, 1.0, 40.0], size=(48, 1)))
    v = v.astype(np.float32).astype(np.float64)
    v[3, 7] = 0.0
    codes, scale = codec.i8_encode(v)
    for r in range(v.shape[0]):
        amax = max(abs(Fraction(float(t))) for t in v[r])
        s = _fp32_round_exact(amax / 127)
        assert scale[r] == s
        sf = Fraction(float(s))
        for d in range(v.shape[1]):
            qv = Fraction(float(v[r, d])) / sf
            n = math.floor(qv)
            frac = qv - n
            want = n + 1 if (frac > Fraction(1, 2) or (frac == Fraction(1, 2) and n % 2 == 1)) else n
            assert codes[r, d] == max(-127, min(127, want)), (r, d)


def test_i8_non_finite_and_zero_rows():
    v = np.ones((3, 128))
    v[0] = 0.0
    v[1, 4] = np.nan
    v[2, 9] = -np.inf
    codes, scale = codec.i8_encode(v)
    assert scale[0] == 0 and np.isnan(scale[1]) and np.isinf(scale[2])
    assert (codes == 0).all()
    dq = codec.i8_decode(codes, scale)
    assert (dq[0] == 0).all() and np.isnan(dq[1]).all() and np.isnan(dq[2]).all()



# ---------------------------------------------------------------- planted mistakes

def test_planted_causal_off_by_one_fails_sdpa_pin(monkeypatch):
    """A row that also sees position t+1 must be caught by the torch pin."""
    orig = masks.visible_matrix

    def leaky(p, lo, hi):
        vm = orig(p, lo, hi)
        if p.mask == CAUSAL:
            j = np.arange(lo, hi)[None, :]
            r = np.arange(p.rows)[:, None]
            vm = vm | ((j == p.first_pos + r + 1) & (r < p.live_rows))
        return vm

    monkeypatch.setattr(attn, "visible_matrix", leaky)
    with pytest.raises(AssertionError):
        test_definition_matches_torch_sdpa(CAUSAL, dict(), False)


def test_planted_dropped_sink_fails_closed_form(monkeypatch):
    orig = attn.verify_attn_ref

    def no_sink(p, q, cache, scale, sink=None):
        return orig(p, q, cache, scale, None)

    monkeypatch.setattr(attn, "verify_attn_ref", no_sink)
    with pytest.raises(AssertionError):
        test_zero_query_mean_and_sink()


def test_planted_skipped_split_fails_split_pin(monkeypatch):
    orig = masks.split_key_ranges

    def skip_one(lo, hi, S):
        rr = orig(lo, hi, S)
        if S > 1:
            a, b = rr[1]
            rr[1] = (a, a)
        return rr

    monkeypatch.setattr(attn, "split_key_ranges", skip_one)
    with pytest.raises(AssertionError):
        test_split_form_random_long()


def test_planted_window_off_by_one_fails_count(monkeypatch):
    orig = masks.visible

    def wide(p, r, j):
        if p.mask == WINDOW and r < p.live_rows and j == p.first_pos + r - p.window and j >= 0:
            return True
        return orig(p, r, j)

    monkeypatch.setattr(masks, "visible", wide)
    with pytest.raises(AssertionError):
        test_window_counts()


def test_planted_tree_non_ancestor_fails_star_pin(monkeypatch):
    orig = masks.tree_ancestors

    def extra(parent):
        a = orig(parent)
        if len(a) > 2:
            a[2] |= 1 << 1     # node 1 made visible to node 2
        return a

    monkeypatch.setattr(masks, "tree_ancestors", extra)
    with pytest.raises(AssertionError):
        test_chain_tree_is_causal_and_star_tree_is_prefix_plus_self()


def test_planted_half_away_rounding_fails_tie_pin(monkeypatch):
    """INT8 codes rounded half away from zero must be caught by the tie pin."""
    monkeypatch.setattr(codec, "_rne", lambda x: np.sign(x) * np.floor(np.abs(x) + 0.5))
    with pytest.raises(AssertionError):
        test_i8_ties_round_half_even()


def test_planted_tight_bound_fails_fp32_encoder_pin(monkeypatch):
    """An error bound that ignores the FP32 rotation's rounding leaves codes
    the FP32 encoder rounds the other way rejected."""
    monkeypatch.setattr(codec, "WHT_F32_ERR_SUM", 0.0)
    monkeypatch.setattr(codec, "WHT_F32_ERR_OUT", 0.0)
    with pytest.raises(AssertionError):
        test_wht_error_bound_covers_fp32_encoders((1, 2, 4, 8, 16, 32, 64), False)
