"""Sampling and acceptance on the GPU (va_sample, va_accept, va_sample_accept)
against the float64 oracle in oracle/sampling.py.

Gates:
* candidate ids: identical (the top-k order is exact: logit, then lower id);
* kept count and drawn token: identical wherever the oracle's margin for
  that decision exceeds 1e-5 (FP32 sums cannot move the decision there);
  elsewhere the GPU's choice must still be a valid one (a kept count within
  one of the oracle's, a token among the kept candidates), and such rows
  must stay rare;
* kept probabilities: |gpu - oracle| <= 1e-6 + 1e-5 * oracle;
* acceptance: the accepted count and every output token identical to the
  oracle run on the same FP32 lists wherever every decision's margin
  exceeds 1e-6;
* the fused call equals the two separate calls bit for bit, also replayed
  from a HIP graph.
"""
import ctypes

import numpy as np
import pytest
import torch

import speculative_decode_verify_amd as va
from speculative_decode_verify_amd import _binding, synth
from oracle import sampling as osamp

DEV = "cuda"
MARGIN = 1e-5
PURPOSE_DRAFT = 3


# ----------------------------------------------------------------------------- CPU

def test_param_record_layout_and_workspace_size():
    assert ctypes.sizeof(_binding.va_sample_params) == 56
    p = va.sample_params(8, 160000, top_k=20)
    tiles = (160000 + 8191) // 8192
    assert va.sample_workspace_bytes(p) == 256 + 8 * tiles * 20 * 8
    assert va.sample_workspace_bytes(va.sample_params(8, 262144, top_k=64)) == 256 + 8 * 32 * 64 * 8


@pytest.mark.parametrize("field,value", [("rows", 0), ("rows", 17), ("top_k", 0), ("top_k", 65), ("vocab", 0),
                                         ("vocab", 262145), ("row_stride", 999), ("temperature", 0.0),
                                         ("temperature", float("inf")), ("top_p", 0.0), ("top_p", float("nan")),
                                         ("first_position", -1), ("reserved", 1)])
def test_invalid_params_rejected_before_launch(field, value):
    p = va.sample_params(4, 1000, top_k=20, row_stride=1004)
    setattr(p, field, value)
    assert va.sample_workspace_bytes(p) == 0
    lib = va.load_library()
    fake = ctypes.c_void_p(0x100000)
    assert lib.va_sample(ctypes.byref(p), fake, fake, fake, fake, fake, fake, 1 << 20, None) == 1


def test_accept_arguments_rejected_before_launch():
    lib = va.load_library()
    f = ctypes.c_void_p(0x100000)
    assert lib.va_accept(f, f, f, f, 20, f, f, f, 20, f, 0, 0, 0, f, f, None) == 1      # n = 0
    assert lib.va_accept(f, f, f, f, 20, f, f, f, 20, f, 17, 0, 0, f, f, None) == 1     # n > 16
    assert lib.va_accept(f, f, f, f, 65, f, f, f, 20, f, 4, 0, 0, f, f, None) == 1      # p stride
    assert lib.va_accept(f, f, f, f, 20, None, f, f, 20, f, 4, 0, 0, f, f, None) == 1   # drafts need q lists
    assert lib.va_accept(f, f, f, f, 20, f, f, f, 20, f, 4, 0, -1, f, f, None) == 1     # position


# ----------------------------------------------------------------------------- helpers

def to_np(out):
    return {k: v.cpu().numpy() for k, v in out.items()}


def compare_sample(g, z, k, top_p, temp, seed, pos0, purpose, name):
    """GPU outputs g (numpy dict) against the oracle on logits z (CPU FP32).
    Returns the number of rows whose kept count or token was within a margin."""
    rows, V = z.shape
    # the ABI takes top_p and the temperature as FP32: the oracle gets the same values
    ref = osamp.sample(z.double().numpy(), k, float(np.float32(top_p)), float(np.float32(temp)), seed, pos0, purpose)
    kc = min(k, V)
    near = 0
    for r, o in enumerate(ref):
        assert np.array_equal(g["ids"][r, :kc], o["ids"]), f"{name} row {r}: candidate ids differ"
        assert np.all(g["ids"][r, kc:] == -1), f"{name} row {r}: ids past V not -1"
        m_gpu, m_ref = int(g["kept"][r]), o["kept"]
        kept_ids = list(g["ids"][r, :m_gpu])
        if o["topp_margin"] <= MARGIN:
            near += 1
            assert abs(m_gpu - m_ref) <= 1, f"{name} row {r}: kept {m_gpu} vs {m_ref} at a near boundary"
            assert int(g["tokens"][r]) in kept_ids
            continue
        assert m_gpu == m_ref, f"{name} row {r}: kept {m_gpu} vs {m_ref} (margin {o['topp_margin']:.2e})"
        pg = g["probs"][r].astype(np.float64)
        assert np.all(np.abs(pg[:kc] - o["probs"]) <= 1e-6 + 1e-5 * o["probs"]), f"{name} row {r}: probs"
        assert np.all(pg[m_gpu:] == 0)
        if o["draw_margin"] <= MARGIN:
            near += 1
            assert int(g["tokens"][r]) in kept_ids
        else:
            assert int(g["tokens"][r]) == o["token"], f"{name} row {r}: token {g['tokens'][r]} vs {o['token']}"
    return near


# ----------------------------------------------------------------------------- sampling

CASES = [
    # (rows, vocab, k, top_p, temperature, kind)
    (8, 160000, 20, 0.95, 1.0, "lm"),
    (8, 20000, 20, 0.95, 1.0, "lm"),
    (8, 160000, 20, 0.95, 1.0, "flat"),
    (8, 160000, 20, 0.95, 1.0, "bf16"),
    (4, 160000, 20, 0.95, 1.0, "masked"),
    (4, 20000, 20, 0.95, 1.0, "few"),
    (4, 20000, 20, 1.0, 1.0, "few"),
    (2, 20000, 20, 0.93, 1.0, "equal"),
    (4, 160000, 20, 0.95, 1.0, "spike"),
    (16, 8193, 64, 0.9, 0.7, "lm"),
    (3, 262144, 64, 1.0, 1.3, "flat"),
    (5, 8192, 1, 0.95, 1.0, "bf16"),
    (1, 3, 20, 0.95, 1.0, "lm"),
    (1, 1, 20, 0.95, 1.0, "lm"),
    (6, 24577, 33, 0.5, 2.0, "lm"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("rows,vocab,k,top_p,temp,kind", CASES)
def test_sample_vs_oracle(rows, vocab, k, top_p, temp, kind):
    g = synth.gen(rows * 1_000_003 + vocab * 7 + k * 131 + synth.LOGIT_KINDS.index(kind))
    z = synth.logits_f32(rows, vocab, g, kind)
    seed, pos0 = 0x1234_5678_9ABC + vocab, 777 + rows
    out = to_np(va.va_sample(z.to(DEV), top_k=k, top_p=top_p, temperature=temp, seed=seed, first_position=pos0))
    near = compare_sample(out, z, k, top_p, temp, seed, pos0, 0, f"{kind} V={vocab} k={k}")
    assert near <= max(1, rows // 4), f"{near} rows within a decision margin"


@pytest.mark.gpu
def test_sample_strided_rows_and_many_positions():
    """Rows with padding between them (row stride 160,004); 16 rows at a
    position past 2^32 (both counter words in use)."""
    g = synth.gen(77)
    z = synth.logits_f32(16, 160004, g, "lm")
    pos0 = (1 << 33) + 5
    view = z.to(DEV)[:, :160000]
    assert view.stride(0) == 160004
    out = to_np(va.va_sample(view, seed=99, first_position=pos0))
    near = compare_sample(out, z[:, :160000].contiguous(), 20, 0.95, 1.0, 99, pos0, 0, "strided")
    assert near <= 2


@pytest.mark.gpu
def test_workspace_reused_across_shapes():
    """One zero-filled workspace serves calls of other shapes in a row (its
    counters return to zero after every call), with and without acceptance."""
    big = va.sample_params(16, 160000, top_k=64)
    ws = va.sample_workspace_for(big, DEV)
    g = synth.gen(31)
    for rows, V, k in ((16, 160000, 64), (3, 20000, 20), (8, 8193, 7), (16, 160000, 64), (1, 5, 20)):
        z = synth.logits_f32(rows, V, g, "lm")
        a = to_np(va.va_sample(z.to(DEV), top_k=k, seed=rows, first_position=V, workspace=ws))
        near = compare_sample(a, z, k, 0.95, 1.0, rows, V, 0, f"reuse rows={rows} V={V}")
        assert near <= max(1, rows // 4)
        out, acc, toks = va.va_sample_accept(z.to(DEV), *([None] * 4 if rows == 1 else [
            torch.from_numpy(a["ids"][: rows - 1]).to(DEV), torch.from_numpy(a["probs"][: rows - 1]).to(DEV),
            torch.from_numpy(a["kept"][: rows - 1]).to(DEV), torch.from_numpy(a["tokens"][: rows - 1]).to(DEV)]),
            top_k=k, seed=rows, first_position=V, workspace=ws)
        b = to_np(out)
        for key in a:
            assert np.array_equal(a[key], b[key]), key
        # drafts equal to the target's own draws with q = p are all accepted
        assert int(acc.item()) == rows - 1


@pytest.mark.gpu
def test_sample_deterministic_and_seeded():
    g = synth.gen(5)
    z = synth.logits_f32(8, 20000, g, "flat").to(DEV)
    a = to_np(va.va_sample(z, seed=1, first_position=10))
    b = to_np(va.va_sample(z, seed=1, first_position=10))
    c = to_np(va.va_sample(z, seed=2, first_position=10))
    for key in a:
        assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["tokens"], c["tokens"])   # 8 draws from ~19 tokens


# ----------------------------------------------------------------------------- acceptance

def draft_and_target(n, vocab, seed, noise, g):
    """Target logits for n rows and draft logits = target + noise for n - 1
    rows: the draft samples its proposals (purpose 3) at the same positions."""
    zt = synth.logits_f32(n, vocab, g, "lm")
    zd = zt[: max(n - 1, 1)] + noise * torch.randn((max(n - 1, 1), vocab), generator=g)
    return zt, zd


def run_accept_case(n, vocab, seed, pos0, noise, g, fused=False):
    zt, zd = draft_and_target(n, vocab, seed, noise, g)
    tgt = va.va_sample(zt.to(DEV), seed=seed, first_position=pos0)
    if n > 1:
        dr = va.va_sample(zd.to(DEV), seed=seed, first_position=pos0, purpose=PURPOSE_DRAFT)
        q = (dr["ids"][: n - 1].contiguous(), dr["probs"][: n - 1].contiguous(), dr["kept"][: n - 1].contiguous(),
             dr["tokens"][: n - 1].contiguous())
    else:
        q = (None, None, None, None)
    acc, toks = va.va_accept(tgt["ids"], tgt["probs"], tgt["kept"], tgt["tokens"], *q, seed, pos0)
    res = dict(tgt=to_np(tgt), q=[None if x is None else x.cpu().numpy() for x in q],
               acc=int(acc.item()), toks=toks.cpu().numpy())
    if fused:
        out, acc2, toks2 = va.va_sample_accept(zt.to(DEV), *q, seed=seed, first_position=pos0)
        res["fused"] = (to_np(out), int(acc2.item()), toks2.cpu().numpy())
    return res


def oracle_accept(res, n, seed, pos0):
    t = res["tgt"]
    qi, qp, qk, dr = res["q"]
    if n == 1:
        qi, qp, qk, dr = [], [], [], []
    return osamp.accept(t["ids"], t["probs"], t["kept"], t["tokens"], qi, qp, qk, dr, n, seed, pos0)


@pytest.mark.gpu
@pytest.mark.parametrize("n,noise", [(8, 0.3), (8, 1.5), (5, 0.0), (16, 0.5), (2, 3.0), (1, 0.0)])
def test_accept_vs_oracle(n, noise):
    """Many requests (seeds): the GPU's acceptance on the GPU's own FP32
    lists against the oracle's on the same lists."""
    accepts, rejects, compared = 0, 0, 0
    for s in range(12):
        seed, pos0 = 1000 + 17 * s, 50 + 3 * s
        g = synth.gen(seed)
        res = run_accept_case(n, 20000, seed, pos0, noise, g)
        a, toks, margin = oracle_accept(res, n, seed, pos0)
        if margin <= 1e-6:
            continue
        compared += 1
        assert res["acc"] == a, f"seed {seed}: accepted {res['acc']} vs {a}"
        assert list(res["toks"][: a + 1]) == toks, f"seed {seed}: tokens {res['toks']} vs {toks}"
        assert np.all(res["toks"][a + 1:] == -1)
        accepts += a == n - 1
        rejects += a < n - 1
    assert compared >= 10
    if n > 1 and noise > 0:
        assert rejects > 0, "no rejection exercised"


@pytest.mark.gpu
def test_accept_crafted_lists():
    """Hand-set lists: a draft outside the target's list is rejected at once
    and replaced from the target's list (residual = p there); q(d) = 0 with
    p(d) > 0 is accepted; all accepted gives the last row's own sample."""
    K = 4
    p_ids = torch.tensor([[5, 6, 7, -1], [8, 9, -1, -1], [1, 2, 3, 4]], dtype=torch.int32)
    p_probs = torch.tensor([[0.5, 0.3, 0.2, 0], [0.9, 0.1, 0, 0], [0.4, 0.3, 0.2, 0.1]], dtype=torch.float32)
    p_kept = torch.tensor([3, 2, 4], dtype=torch.int32)
    p_tok = torch.tensor([6, 8, 3], dtype=torch.int32)
    q_ids = torch.tensor([[11, -1, -1, -1], [8, -1, -1, -1]], dtype=torch.int32)
    q_probs = torch.tensor([[1.0, 0, 0, 0], [1.0, 0, 0, 0]], dtype=torch.float32)
    q_kept = torch.tensor([1, 1], dtype=torch.int32)
    dev = lambda *ts: [t.to(DEV) for t in ts]
    # draft 11 is outside row 0's list: rejected, replacement from {5, 6, 7}
    acc, toks = va.va_accept(*dev(p_ids, p_probs, p_kept, p_tok, q_ids, q_probs, q_kept), torch.tensor(
        [11, 8], dtype=torch.int32, device=DEV), 3, 0)
    a, t, _ = osamp.accept(p_ids.numpy(), p_probs.numpy(), p_kept.numpy(), p_tok.numpy(), q_ids.numpy(),
                           q_probs.numpy(), q_kept.numpy(), [11, 8], 3, 3, 0)
    assert int(acc.item()) == 0 == a and int(toks[0].item()) == t[0] and t[0] in (5, 6, 7)
    # drafts 5 (q = 0, p = 0.5 -> accepted) then 8 (q = 1, p = 0.9: accepted iff u < 0.9)
    q_ids2 = torch.tensor([[12, -1, -1, -1], [8, -1, -1, -1]], dtype=torch.int32)
    for seed in range(20):
        acc, toks = va.va_accept(*dev(p_ids, p_probs, p_kept, p_tok, q_ids2, q_probs, q_kept),
                                 torch.tensor([5, 8], dtype=torch.int32, device=DEV), seed, 40)
        a, t, m = osamp.accept(p_ids.numpy(), p_probs.numpy(), p_kept.numpy(), p_tok.numpy(), q_ids2.numpy(),
                               q_probs.numpy(), q_kept.numpy(), [5, 8], 3, seed, 40)
        assert a >= 1 and int(acc.item()) == a and list(toks.cpu().numpy()[: a + 1]) == t
        if a == 2:
            assert t == [5, 8, 3]


@pytest.mark.gpu
@pytest.mark.parametrize("n", [8, 1])
def test_fused_equals_separate_and_graph_replay(n):
    seed, pos0 = 4242, 900
    g = synth.gen(seed)
    res = run_accept_case(n, 160000, seed, pos0, 0.4, g, fused=True)
    out, acc2, toks2 = res["fused"]
    for key in out:
        assert np.array_equal(out[key], res["tgt"][key]), key
    assert acc2 == res["acc"] and np.array_equal(toks2, res["toks"])
    # one graph, replayed with eager work in between; the counter resets itself
    g2 = synth.gen(seed)
    zt, zd = draft_and_target(n, 160000, seed, 0.4, g2)
    zt = zt.to(DEV)
    q = [None if x is None else torch.from_numpy(x).to(DEV) for x in res["q"]]
    p = va.sample_params(n, 160000, seed=seed, first_position=pos0)
    ws = va.sample_workspace_for(p, DEV)
    o = dict(ids=torch.empty((n, 20), dtype=torch.int32, device=DEV),
             probs=torch.empty((n, 20), dtype=torch.float32, device=DEV),
             kept=torch.empty(n, dtype=torch.int32, device=DEV), tokens=torch.empty(n, dtype=torch.int32, device=DEV))
    acc = torch.empty(1, dtype=torch.int32, device=DEV)
    tk = torch.empty(n, dtype=torch.int32, device=DEV)
    va.va_sample_accept(zt, *q, seed=seed, first_position=pos0, workspace=ws, out=o, accepted=acc, out_tokens=tk)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        va.va_sample_accept(zt, *q, seed=seed, first_position=pos0, workspace=ws, out=o, accepted=acc,
                            out_tokens=tk)
    for rep in range(4):
        acc.fill_(-7)
        tk.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(acc.item()) == res["acc"], f"replay {rep}"
        assert np.array_equal(tk.cpu().numpy(), res["toks"]), f"replay {rep}"
        va.va_sample(zt, seed=seed + rep, first_position=pos0)   # eager work between replays
