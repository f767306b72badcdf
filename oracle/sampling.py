"""Sampling and draft acceptance after verification, in float64 from the definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

IQuestRT report, "Include sampling and acceptance in the execution path":
the target samples with temperature 1, top-k 20 and top-p 0.95; the draft
samples too and keeps the distribution it actually proposed from; a draft
token d is accepted with probability min(1, p(d)/q(d)); at the first
rejection a replacement is drawn from max(0, p - q) renormalised; when every
draft is accepted the target's extra row gives a bonus token; random numbers
depend only on the request seed and the token position.  "Parallelize the
Top-K vocabulary scan" (same report) describes how the top-k is found, not
what it is, so it does not enter here.

Readings where the pages are silent (each is one of the listed choices):
1. Candidate order: logit descending, equal logits by lower token id first.
   top-k keeps the first min(k, V) of that order.
2. Temperature T > 0 divides the logits; the K candidates' probabilities are
   p_i = exp((z_i - z_0)/T) / sum_j exp((z_j - z_0)/T) (z_0 the largest).
3. top-p keeps candidate i iff p_i > 0 and sum_{j<i} p_j < top_p: the
   shortest prefix whose mass reaches top_p, never a zero-mass token, at
   least one token.  The kept probabilities are renormalised.
4. Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
   random numbers: as easy as 1, 2, 3", SC'11) with key (seed low word, seed
   high word) and counter (position low word, position high word, purpose,
   0); the first output word x gives u = (x >> 8) * 2^-24 in [0, 1).
   Purposes: 0 the target row's own sample, 1 the acceptance test,
   2 the replacement draw; a caller picks any other value for its own draws
   (3 for the draft in the tests).
5. A draw from kept candidates with weights w_i is by inverse CDF in
   candidate order: the first i with u * sum(w) < w_0 + ... + w_i; the last
   kept candidate if rounding leaves none.
6. Row i of the verification (i = 0 is the committed token) samples the
   token at position pos0 + i.  Draft d_{i+1} is tested against row i with
   u from (pos0 + i, purpose 1): accepted iff u * q(d) < p(d), where p and q
   are the kept, renormalised lists (zero outside them).  At the first
   rejection, at row i, the replacement is drawn from r(t) = max(0, p_i(t) -
   q(t)) over row i's kept tokens with u from (pos0 + i, purpose 2); a zero
   residual mass (possible only through rounding) gives row i's own sample.
   With every draft accepted the bonus is row n-1's own sample.

Floating point decides integers here (the kept count, the drawn index, the
accept bit).  The functions return, beside each result, its margin: the
distance of the deciding quantity from its threshold.  A GPU computing in
FP32 may take the other side only where that margin is within FP32 rounding.
"""

import numpy as np

PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = 0xFFFFFFFF

PURPOSE_TARGET, PURPOSE_ACCEPT, PURPOSE_RESIDUAL = 0, 1, 2


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds on Python integers (SC'11 paper, section 4):
    a round multiplies words 0 and 2 by the two constants, and the new words
    are (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0));
    the key is bumped by the two Weyl constants before every round but the
    first."""
    c = [int(x) & _MASK32 for x in counter]
    k = [int(x) & _MASK32 for x in key]
    for r in range(10):
        if r:
            k = [(k[0] + PHILOX_W0) & _MASK32, (k[1] + PHILOX_W1) & _MASK32]
        p0 = PHILOX_M0 * c[0]
        p1 = PHILOX_M1 * c[2]
        c = [(p1 >> 32) ^ c[1] ^ k[0], p1 & _MASK32, (p0 >> 32) ^ c[3] ^ k[1], p0 & _MASK32]
    return c


def uniform(seed, position, purpose):
    """u in [0, 1) on a 2^-24 grid (reading 4)."""
    seed, position = int(seed), int(position)
    x = philox4x32_10([position & _MASK32, (position >> 32) & _MASK32, purpose, 0],
                      [seed & _MASK32, (seed >> 32) & _MASK32])[0]
    return (x >> 8) * 2.0 ** -24


def topk_ids(z, k):
    """Reading 1: the first min(k, V) token ids by (logit desc, id asc)."""
    z = np.asarray(z, dtype=np.float64)
    order = np.lexsort((np.arange(z.size), -z))
    return order[:min(int(k), z.size)]


def draw(weights, u):
    """Reading 5: (index, margin) of an inverse-CDF draw over weights >= 0."""
    w = np.asarray(weights, dtype=np.float64)
    cum = np.cumsum(w)
    tot = cum[-1]
    t = u * tot
    hit = np.nonzero(t < cum)[0]
    i = int(hit[0]) if hit.size else w.size - 1
    margin = float(np.min(np.abs(cum - t)) / tot) if tot > 0 else 0.0
    return i, margin


def sample_row(z, k, top_p, temperature, u):
    """Readings 1-3 and 5 for one row of logits.

    Returns dict: ids (the top-k in order), probs (renormalised over the kept
    prefix, zero beyond it), kept (m), token, and the margins of the top-p
    cut (topp_margin, over every candidate boundary) and of the draw
    (draw_margin)."""
    z = np.asarray(z, dtype=np.float64)
    ids = topk_ids(z, k)
    zs = z[ids]
    e = np.exp((zs - zs[0]) / temperature)
    p = e / e.sum()
    excl = np.concatenate([[0.0], np.cumsum(p)[:-1]])
    keep = (p > 0) & (excl < top_p)
    m = int(np.argmin(keep)) if not keep.all() else keep.size
    probs = np.zeros(ids.size)
    probs[:m] = p[:m] / p[:m].sum()
    j, dm = draw(e[:m], u)
    # the cut compares excl with top_p only where p_i > 0 (p_i = 0 is never kept)
    pos = np.nonzero(p[1:] > 0)[0] + 1
    tm = float(np.min(np.abs(excl[pos] - top_p))) if pos.size else np.inf
    return dict(ids=ids, probs=probs, kept=m, token=int(ids[j]), topp_margin=tm, draw_margin=dm)


def sample(logits, k, top_p, temperature, seed, pos0, purpose):
    """sample_row for every row r with u from (pos0 + r, purpose)."""
    return [sample_row(z, k, top_p, temperature, uniform(seed, pos0 + r, purpose))
            for r, z in enumerate(np.asarray(logits, dtype=np.float64))]


def _prob_of(ids, probs, count, t):
    hit = np.nonzero(np.asarray(ids[:count]) == t)[0]
    return float(probs[hit[0]]) if hit.size else 0.0


def residual(p_ids, p_probs, p_count, q_ids, q_probs, q_count):
    """max(0, p(t) - q(t)) for the target row's kept tokens t, in list order."""
    return np.array([max(0.0, float(p_probs[j]) - _prob_of(q_ids, q_probs, q_count, int(p_ids[j])))
                     for j in range(int(p_count))])


def accept(p_ids, p_probs, p_count, p_tokens, q_ids, q_probs, q_count, drafts, n, seed, pos0):
    """Reading 6.  p_*: the n target rows' kept lists and own samples; q_*:
    the n - 1 draft lists; drafts: d_1..d_{n-1}.  Returns (accepted count a,
    the a + 1 output tokens, the smallest margin of the decisions taken)."""
    return accept_with(p_ids, p_probs, p_count, p_tokens, q_ids, q_probs, q_count, drafts, n,
                       lambda i, purpose: uniform(seed, pos0 + i, purpose))


def accept_with(p_ids, p_probs, p_count, p_tokens, q_ids, q_probs, q_count, drafts, n, u_of):
    """accept() with the uniform for (row i, purpose) given by u_of(i, purpose)."""
    margin = np.inf
    for i in range(n - 1):
        d = int(drafts[i])
        pd = _prob_of(p_ids[i], p_probs[i], p_count[i], d)
        qd = _prob_of(q_ids[i], q_probs[i], q_count[i], d)
        u = u_of(i, PURPOSE_ACCEPT)
        margin = min(margin, abs(u * qd - pd))
        if u * qd < pd:
            continue
        r = residual(p_ids[i], p_probs[i], p_count[i], q_ids[i], q_probs[i], q_count[i])
        if r.sum() > 0:
            j, dm = draw(r, u_of(i, PURPOSE_RESIDUAL))
            margin = min(margin, dm)
            tok = int(p_ids[i][j])
        else:
            tok = int(p_tokens[i])
        return i, [int(x) for x in drafts[:i]] + [tok], margin
    return n - 1, [int(x) for x in drafts[:n - 1]] + [int(p_tokens[n - 1])], margin
