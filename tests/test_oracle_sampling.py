"""Pins for the sampling and acceptance oracle (oracle/sampling.py).

Pins: Philox4x32-10 known-answer vectors (tests/golden/philox_kat.json),
hand-worked top-p and draw cases, brute-force ordering with ties, numpy's
softmax-free closed forms, the exact measure of every draw over a grid of
u, and the theorem that rejection sampling against the draft's proposal
reproduces the target distribution (enumerated over the draft token and
grids of the two uniforms).  The planted-mistake tests at the end show that
a plausible slip in each step fails a pin.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import sampling as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    g = json.load(open(os.path.join(GOLDEN, "philox_kat.json")))
    for v in g["vectors"]:
        out = S.philox4x32_10([int(x, 16) for x in v["counter"]], [int(x, 16) for x in v["key"]])
        assert out == [int(x, 16) for x in v["out"]]


def test_uniform_grid_range_and_mean():
    us = np.array([S.uniform(12345, p, 0) for p in range(4000)])
    assert np.all(us >= 0) and np.all(us < 1)
    assert np.all(us * 2 ** 24 == np.floor(us * 2 ** 24))
    assert abs(us.mean() - 0.5) < 0.02
    # purpose and seed change the stream
    assert S.uniform(1, 5, 0) != S.uniform(1, 5, 1) and S.uniform(1, 5, 0) != S.uniform(2, 5, 0)
    # 64-bit seeds and positions use both words
    assert S.uniform(1 << 40, 5, 0) != S.uniform(0, 5, 0)
    assert S.uniform(1, (1 << 33) + 5, 0) != S.uniform(1, 5, 0)


def test_topk_order_brute_force_with_ties():
    rng = np.random.default_rng(0)
    for trial in range(200):
        V = int(rng.integers(1, 40))
        z = rng.integers(-3, 4, size=V).astype(np.float64)   # many ties
        if trial % 3 == 0:
            z[rng.integers(0, V, size=V // 2)] = -np.inf
        k = int(rng.integers(1, 25))
        want = [i for _, i in sorted((-z[i], i) for i in range(V))][:k]
        assert list(S.topk_ids(z, k)) == want


def test_sample_row_hand_worked():
    z = np.log([0.2, 0.5, 0.3])            # ids 1, 2, 0 in order
    r = S.sample_row(z, 20, 0.75, 1.0, 0.7)
    # p = 0.5, 0.3, 0.2: id 2 kept since 0.5 < 0.75, id 0 dropped since 0.8 >= 0.75
    assert list(r["ids"]) == [1, 2, 0] and r["kept"] == 2
    assert np.allclose(r["probs"], [0.625, 0.375, 0.0])
    # weights 1, 0.6: u = 0.7 -> 1.12 lies above 1 -> second candidate
    assert r["token"] == 2
    assert S.sample_row(z, 20, 0.75, 1.0, 0.5)["token"] == 1      # 0.8 < 1
    assert S.sample_row(z, 20, 1.0, 1.0, 0.0)["kept"] == 3
    assert S.sample_row(z, 20, 0.5, 1.0, 0.9)["kept"] == 1        # 0 < 0.5, then 0.5 >= 0.5
    assert S.sample_row(z, 2, 1.0, 1.0, 0.99)["kept"] == 2        # top-k before top-p
    # temperature 2: weights are the square roots of the probabilities
    r2 = S.sample_row(z, 20, 1.0, 2.0, 0.0)
    w = np.sqrt([0.5, 0.3, 0.2])
    assert np.allclose(r2["probs"], w / w.sum())


def test_zero_mass_candidates_never_kept():
    z = np.array([0.0, -np.inf, -np.inf, 1.0])
    r = S.sample_row(z, 4, 1.0, 1.0, 0.999)
    assert r["kept"] == 2 and list(r["ids"][:2]) == [3, 0]
    assert r["token"] in (3, 0) and r["probs"][2] == 0 and r["probs"][3] == 0


def test_top_k_one_is_argmax_lowest_id():
    rng = np.random.default_rng(1)
    for _ in range(50):
        z = rng.integers(0, 3, size=30).astype(np.float64)
        r = S.sample_row(z, 1, 0.95, 1.0, float(rng.random()))
        assert r["token"] == int(np.argmax(z))      # numpy's argmax takes the first maximum


def test_draw_measure_on_a_grid():
    """Over u on a uniform grid of N points each candidate is drawn with
    frequency w_i / sum(w) up to 1/N (inverse CDF)."""
    rng = np.random.default_rng(2)
    N = 4096
    for _ in range(20):
        w = rng.random(int(rng.integers(1, 21))) ** 3
        counts = np.zeros(w.size)
        for j in range(N):
            counts[S.draw(w, (j + 0.5) / N)[0]] += 1
        assert np.all(np.abs(counts / N - w / w.sum()) <= 1.0 / N + 1e-12)


def _lists(p_dict, K):
    ids = np.full(K, -1)
    pr = np.zeros(K)
    for j, (t, v) in enumerate(sorted(p_dict.items(), key=lambda kv: -kv[1])):
        ids[j], pr[j] = t, v
    return ids, pr, len(p_dict)


def test_rejection_sampling_reproduces_the_target():
    """One draft (n = 2): P(first output = t) = sum_d q(d) [a(d) 1{t = d} +
    (1 - a(d)) res_d(t)] with a(d), res_d measured through the oracle over
    grids of u; it must equal p(t) (speculative sampling's correctness)."""
    assert _theorem_holds(range(6))


def _theorem_holds(trials):
    rng = np.random.default_rng(3)
    N, M = 2048, 512
    grid = (np.arange(N) + 0.5) / N
    rgrid = (np.arange(M) + 0.5) / M
    for trial in range(max(trials) + 1):
        V = 8
        sp = rng.choice(V, size=int(rng.integers(1, 6)), replace=False)
        sq = rng.choice(V, size=int(rng.integers(1, 6)), replace=False)
        if trial == 0:
            sq = sp                                 # same support
        pw, qw = rng.random(sp.size) + 0.05, rng.random(sq.size) + 0.05
        p = {int(t): float(v) for t, v in zip(sp, pw / pw.sum())}
        q = {int(t): float(v) for t, v in zip(sq, qw / qw.sum())}
        pi, pp, pc = _lists(p, 8)
        qi, qp, qc = _lists(q, 8)
        p_tok = [int(pi[0]), int(pi[0])]
        out = np.zeros(V)
        args = ([pi, pi], [pp, pp], [pc, pc], p_tok, [qi], [qp], [qc])
        for d, qd in q.items():
            acc = [S.accept_with(*args, [d], 2, lambda i, purpose, ua=ua: ua)[0] for ua in grid]
            a = float(np.mean(acc))
            out[d] += qd * a
            if a == 1.0:
                continue
            ua_rej = grid[acc.index(0)]
            for ur in rgrid:
                a2, toks2, _ = S.accept_with(*args, [d], 2,
                                             lambda i, purpose, ur=ur: ua_rej if purpose == S.PURPOSE_ACCEPT else ur)
                assert a2 == 0
                out[toks2[0]] += qd * (1 - a) / M
        want = np.zeros(V)
        for t, v in p.items():
            want[t] = v
        if trial in trials and not np.allclose(out, want, atol=2.0 / N + 2.0 / M):
            return False
    return True


def test_all_accepted_gives_bonus_and_q_zero_rule():
    pi = np.array([5, 6, -1]); pp = np.array([0.7, 0.3, 0.0])
    qi = np.array([5, -1, -1]); qp = np.array([1.0, 0.0, 0.0])
    a, toks, _ = S.accept_with([pi, pi, pi], [pp, pp, pp], [2, 2, 2], [6, 6, 9], [qi, qi], [qp, qp], [1, 1],
                               [5, 5], 3, lambda i, purpose: 0.5)
    assert a == 2 and toks == [5, 5, 9]
    # q(d) = 0: accepted iff p(d) > 0
    a, toks, _ = S.accept_with([pi, pi], [pp, pp], [2, 2], [6, 6], [qi], [qp], [1], [6], 2, lambda i, pu: 0.99)
    assert a == 1 and toks == [6, 6]
    a, toks, _ = S.accept_with([pi, pi], [pp, pp], [2, 2], [6, 6], [qi], [qp], [1], [7], 2, lambda i, pu: 0.0)
    assert a == 0 and toks[0] in (5, 6)


# ---------------------------------------------------------------- planted mistakes

def test_planted_mistakes_are_caught(monkeypatch):
    """Each pin fails for a plausible slip in the oracle."""
    g = json.load(open(os.path.join(GOLDEN, "philox_kat.json")))
    v = g["vectors"][2]
    ctr, key = [int(x, 16) for x in v["counter"]], [int(x, 16) for x in v["key"]]
    good = S.philox4x32_10(ctr, key)
    # swapped multipliers
    monkeypatch.setattr(S, "PHILOX_M0", 0xCD9E8D57)
    monkeypatch.setattr(S, "PHILOX_M1", 0xD2511F53)
    assert S.philox4x32_10(ctr, key) != good
    monkeypatch.undo()
    # ties taken by higher id
    z = np.array([1.0, 2.0, 2.0])
    assert list(S.topk_ids(z, 2)) == [1, 2]
    assert list(np.argsort(-z, kind="stable")[::-1][:2]) != [1, 2]
    # top-p cut on the inclusive prefix keeps one candidate fewer in the hand case
    p = np.array([0.5, 0.3, 0.2])
    incl = np.cumsum(p)
    assert int(np.sum(incl < 0.75)) == 1 != S.sample_row(np.log([0.2, 0.5, 0.3]), 20, 0.75, 1.0, 0.0)["kept"]
    # replacement drawn from p instead of the residual max(0, p - q)
    monkeypatch.setattr(S, "residual", lambda pi, pp, pc, qi, qp, qc: np.asarray(pp[:int(pc)], dtype=np.float64))
    assert not _theorem_holds([3])
    monkeypatch.undo()
    # acceptance ratio inverted (q/p)
    orig = S._prob_of
    monkeypatch.setattr(S, "accept_with", _planted_accept(S.accept_with, orig))
    assert not _theorem_holds([3])


def _planted_accept(real, prob_of):
    """accept_with with p and q exchanged in the acceptance test only."""
    def planted(p_ids, p_probs, p_count, p_tokens, q_ids, q_probs, q_count, drafts, n, u_of):
        d = int(drafts[0])
        pd, qd = prob_of(p_ids[0], p_probs[0], p_count[0], d), prob_of(q_ids[0], q_probs[0], q_count[0], d)
        if u_of(0, S.PURPOSE_ACCEPT) * pd < qd:
            return 1, [d, int(p_tokens[1])], 1.0
        return real(p_ids, p_probs, p_count, p_tokens, q_ids, q_probs, q_count, drafts, n,
                    lambda i, purpose: 1.0 - 2 ** -24 if purpose == S.PURPOSE_ACCEPT else u_of(i, purpose))
    return planted
