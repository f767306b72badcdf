"""Which keys each verification row sees, written out plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* IQuestRT report, "IQuestRT execution": one committed token plus three to
  seven drafts fill an eight-row kernel width; the remaining rows are padding.
* IQuestRT report, "Read only the KV tiles needed by the current positions":
  full attention reads the history up to the current positions with a causal
  mask at the boundary; the sliding-window ring is the 4,096-position window
  plus one 64-slot tile; the verification rows' KV is written before the read.
* "Qwen3.8-27B on one RTX 4090", "More tokens per round: verify trees": the
  tree is verified in one pass under a tree attention mask.

Readings where the pages leave a step open:
* Chain row r sits at position first_pos + r and sees keys 0..t (causal) or
  t-W+1..t clipped at 0 (window).
* A padding row sees no key and never widens the read extent.
* Tree node i's key sits at position prefix_len + i; row i sees the whole
  prefix [0, prefix_len) plus its ancestors and itself; parent -1 means the
  node hangs off the last committed token, which is already in the prefix.
* Ring slot of position p is p mod ring_slots.
* Splits are contiguous runs of 32-key chunks starting at the chunk holding
  the lowest visible key, balanced to within one chunk: with q = C // S and
  r = C % S (C chunks), split s takes q + 1 chunks if s < r and q chunks
  otherwise, in order.  (The pages fix the 64-slot tile of the read and the
  ring, not the unit a split boundary falls on.)
"""

import numpy as np

SPLIT_KEYS = 32  # keys per split granule

CAUSAL = "causal"
WINDOW = "window"
TREE = "tree"


class Problem:
    """Plain record of the row geometry (no arithmetic of the method)."""

    def __init__(self, mask, rows, live_rows, first_pos=0, prefix_len=0,
                 parent=None, window=0, ring_slots=0):
        self.mask = mask
        self.rows = int(rows)
        self.live_rows = int(live_rows)
        self.first_pos = int(first_pos)
        self.prefix_len = int(prefix_len)
        self.parent = None if parent is None else [int(x) for x in parent]
        self.window = int(window)
        self.ring_slots = int(ring_slots)


def tree_ancestors(parent):
    """Bit j of entry i is set iff node j is node i or one of its ancestors.

    Computed by walking parent links one at a time.
    """
    out = []
    for i in range(len(parent)):
        bits = 1 << i
        j = parent[i]
        steps = 0
        while j >= 0:
            bits |= 1 << j
            j = parent[j]
            steps += 1
            if steps > len(parent):
                raise ValueError("parent links form a cycle")
        out.append(bits)
    return out


def row_position(p, r):
    """Absolute position of chain row r (causal and window modes)."""
    return p.first_pos + r


def visible(p, r, j):
    """True iff row r attends to the key at absolute position j."""
    if r >= p.live_rows or j < 0:
        return False
    if p.mask == CAUSAL:
        return j <= row_position(p, r)
    if p.mask == WINDOW:
        t = row_position(p, r)
        return t - p.window < j <= t
    if p.mask == TREE:
        if j < p.prefix_len:
            return True
        i = j - p.prefix_len
        if i >= p.rows:
            return False
        return bool((tree_ancestors(p.parent)[r] >> i) & 1)
    raise ValueError(p.mask)


def visible_keys(p, r):
    """Sorted list of the positions row r sees, by enumeration over a bound."""
    if p.mask == TREE:
        bound = p.prefix_len + p.rows
    else:
        bound = p.first_pos + p.rows
    return [j for j in range(bound) if visible(p, r, j)]


def union_extent(p):
    """[lo, hi): smallest interval holding every key some live row sees."""
    keys = set()
    for r in range(p.live_rows):
        keys.update(visible_keys(p, r))
    if not keys:
        return 0, 0
    return min(keys), max(keys) + 1


def union_extent_fast(p):
    """Same as union_extent, from the interval end points (large positions)."""
    if p.live_rows == 0:
        return 0, 0
    if p.mask == CAUSAL:
        return 0, p.first_pos + p.live_rows
    if p.mask == WINDOW:
        lo = max(0, p.first_pos - p.window + 1)
        return lo, p.first_pos + p.live_rows
    if p.mask == TREE:
        return 0, p.prefix_len + p.live_rows
    raise ValueError(p.mask)


def visible_matrix(p, lo, hi):
    """Boolean [rows, hi-lo]: entry (r, j-lo) = visible(p, r, j).

    The same rules as visible(), broadcast over a range of positions.
    """
    j = np.arange(lo, hi, dtype=np.int64)[None, :]
    r = np.arange(p.rows, dtype=np.int64)[:, None]
    live = r < p.live_rows
    if p.mask == CAUSAL:
        t = p.first_pos + r
        vis = (j >= 0) & (j <= t)
    elif p.mask == WINDOW:
        t = p.first_pos + r
        vis = (j >= 0) & (j > t - p.window) & (j <= t)
    elif p.mask == TREE:
        anc = np.array(tree_ancestors(p.parent), dtype=np.int64)[:, None]
        i = j - p.prefix_len
        in_tree = (i >= 0) & (i < p.rows)
        bit = (anc >> np.clip(i, 0, 62)) & 1
        vis = (j >= 0) & ((j < p.prefix_len) | (in_tree & (bit == 1)))
    else:
        raise ValueError(p.mask)
    return vis & live


def split_key_ranges(lo, hi, splits):
    """Key range [a, b) of each split: contiguous 32-key chunks, balanced."""
    if hi <= lo:
        return [(0, 0)] * splits
    c_lo = lo // SPLIT_KEYS
    c_hi = -(-hi // SPLIT_KEYS)
    n = c_hi - c_lo
    out = []
    q, r = divmod(n, splits)
    for s in range(splits):
        a_c = c_lo + s * q + min(s, r)
        b_c = a_c + q + (1 if s < r else 0)
        a = max(lo, a_c * SPLIT_KEYS)
        b = min(hi, b_c * SPLIT_KEYS)
        out.append((a, b) if b > a else (a, a))
    return out


def ring_replay(ring_slots, events):
    """Replay writes into a ring; return the position label held by each slot.

    events: iterable of absolute positions written in order; slot p mod C
    receives label p.  Slots never written hold -1.
    """
    labels = [-1] * ring_slots
    for pos in events:
        labels[pos % ring_slots] = pos
    return labels
