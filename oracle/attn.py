"""Verification attention in float64: the definition, its split form, the combine.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The definition (IQuestRT report, "Read only the KV tiles needed by the
current positions" and "Expose more parallelism in attention"): for live row
r and query head h, with KV head g = h // G and every stored value decoded
exactly to float64,

    s_j   = scale * <q_{r,h}, k_{g,j}>            for j in Vis(r)
    M     = max(max_j s_j, sigma_h)
    den   = sum_j exp(s_j - M) + exp(sigma_h - M)
    o     = sum_j exp(s_j - M) v_{g,j} / den
    lse   = M + ln(den)

The sink sigma_h has zero value: it enters the denominator only (same
section).  No sink means sigma_h = -inf.  An empty Vis(r) without a sink, and
every padding row, give o = 0 and lse = -inf.

The split form (same sections): the visible keys are partitioned into
contiguous runs; run s keeps m_s = max s_j over its keys, l_s = sum
exp(s_j - m_s) and the unnormalised O_s = sum exp(s_j - m_s) v_j; the combine
merges runs through their maxima and adds the sink once.

Reading: the sink is in the same post-scale natural-log units as s_j and is
not multiplied by scale.  Query head h uses KV head h // G (contiguous
groups).
"""

import numpy as np

from .masks import Problem, visible_matrix, union_extent_fast, split_key_ranges  # noqa: F401


class Cache:
    """Decoded float64 keys and values with their position-to-slot rule.

    k, v: float64 [Hkv, slots, D].  ring_slots = 0: position j lives in slot
    j; otherwise in slot j mod ring_slots.
    """

    def __init__(self, k, v, ring_slots=0):
        self.k = np.asarray(k, dtype=np.float64)
        self.v = np.asarray(v, dtype=np.float64)
        self.ring_slots = int(ring_slots)

    def slots(self, lo, hi):
        pos = np.arange(lo, hi, dtype=np.int64)
        return pos % self.ring_slots if self.ring_slots else pos


def _scores(p, q, cache, scale, g, G, lo, hi):
    """Masked scores [rows, G, hi-lo] for KV head g; invisible entries -inf."""
    sl = cache.slots(lo, hi)
    kg = cache.k[g][sl]                                  # [L, D]
    qg = q[:, g * G:(g + 1) * G, :]                      # [R, G, D]
    s = scale * np.einsum("rhd,jd->rhj", qg, kg)
    vis = visible_matrix(p, lo, hi)[:, None, :]
    return np.where(vis, s, -np.inf), sl


def verify_attn_ref(p, q, cache, scale, sink=None):
    """Brute-force definition.  q: float64 [R, Hq, D]; sink: [Hq] or None.

    Returns (o [R, Hq, D] float64, lse [R, Hq] float64).
    """
    q = np.asarray(q, dtype=np.float64)
    R, Hq, D = q.shape
    Hkv = cache.k.shape[0]
    G = Hq // Hkv
    lo, hi = union_extent_fast(p)
    o = np.zeros((R, Hq, D))
    lse = np.full((R, Hq), -np.inf)
    if hi <= lo:
        return o, lse
    sig = np.full(Hq, -np.inf) if sink is None else np.asarray(sink, np.float64)
    for g in range(Hkv):
        s, sl = _scores(p, q, cache, scale, g, G, lo, hi)
        vg = cache.v[g][sl]                              # [L, D]
        for r in range(p.live_rows):
            for jj in range(G):
                h = g * G + jj
                row = s[r, jj]
                M = max(np.max(row), sig[h])
                if M == -np.inf:
                    continue
                w = np.exp(row - M)                       # exp(-inf) = 0
                den = w.sum() + np.exp(sig[h] - M)
                o[r, h] = (w @ vg) / den
                lse[r, h] = M + np.log(den)
    return o, lse


def split_partials(p, q, cache, scale, splits):
    """Per-split (m, l, O) in natural-log units.

    Returns m, l: [S, R, Hq]; O: [S, R, Hq, D].  An empty run (or a row that
    sees none of its keys) has m = -inf, l = 0, O = 0.
    """
    q = np.asarray(q, dtype=np.float64)
    R, Hq, D = q.shape
    Hkv = cache.k.shape[0]
    G = Hq // Hkv
    lo, hi = union_extent_fast(p)
    ranges = split_key_ranges(lo, hi, splits)
    m = np.full((splits, R, Hq), -np.inf)
    l = np.zeros((splits, R, Hq))
    O = np.zeros((splits, R, Hq, D))
    for s_idx, (a, b) in enumerate(ranges):
        if b <= a:
            continue
        for g in range(Hkv):
            s, sl = _scores(p, q, cache, scale, g, G, a, b)
            vg = cache.v[g][sl]
            for r in range(p.live_rows):
                for jj in range(G):
                    h = g * G + jj
                    row = s[r, jj]
                    mx = np.max(row)
                    if mx == -np.inf:
                        continue
                    w = np.exp(row - mx)
                    m[s_idx, r, h] = mx
                    l[s_idx, r, h] = w.sum()
                    O[s_idx, r, h] = w @ vg
    return m, l, O


def combine(m, l, O, live_rows, sink=None):
    """LSE merge of split partials plus the sink, applied once.

    m, l: [S, R, Hq]; O: [S, R, Hq, D].  Padding rows (r >= live_rows) give
    o = 0 and lse = -inf.
    """
    S, R, Hq = m.shape
    D = O.shape[-1]
    sig = np.full(Hq, -np.inf) if sink is None else np.asarray(sink, np.float64)
    o = np.zeros((R, Hq, D))
    lse = np.full((R, Hq), -np.inf)
    for r in range(live_rows):
        for h in range(Hq):
            M = max(np.max(m[:, r, h]), sig[h])
            if M == -np.inf:
                continue
            w = np.exp(m[:, r, h] - M)
            den = (w * l[:, r, h]).sum() + np.exp(sig[h] - M)
            o[r, h] = (w[:, None] * O[:, r, h]).sum(axis=0) / den
            lse[r, h] = M + np.log(den)
    return o, lse


def verify_attn_ref_split(p, q, cache, scale, splits, sink=None):
    """Split form followed by the combine; must equal verify_attn_ref."""
    m, l, O = split_partials(p, q, cache, scale, splits)
    return combine(m, l, O, p.live_rows, sink)
