"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Only random draws and fixed patterns live here: no attention, mask, ring or
codec arithmetic.  Values are drawn in FP32 on the CPU with a torch
Generator and rounded to bf16 (round to nearest even) where bf16 is asked for.
"""
import torch


def gen(seed):
    return torch.Generator().manual_seed(int(seed))


def normal_f32(shape, g):
    return torch.randn(shape, generator=g, dtype=torch.float32)


def normal_bf16(shape, g):
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def live_count(g, lo=4, hi=8):
    """Live rows of a chain step: uniform on lo..hi."""
    return int(torch.randint(lo, hi + 1, (1,), generator=g).item())


def random_tree(n, g):
    """Parents of an n-node draft tree: node 0 hangs off the committed token
    (-1); node i > 0 takes a parent uniform on 0..i-1."""
    par = [-1]
    for i in range(1, n):
        par.append(int(torch.randint(0, i, (1,), generator=g).item()))
    return par


def position_labels(positions, channels):
    """Integer labels of absolute positions, exact in bf16 (all < 64):
    base-64 digits, then residues mod 61, 59, 53, 47, 43, 41, 37, 31, 29,
    repeated to fill `channels`."""
    p = torch.as_tensor(positions, dtype=torch.int64)
    cols = [(p // 64 ** c) % 64 for c in range(3)]
    mods = [61, 59, 53, 47, 43, 41, 37, 31, 29]
    i = 0
    while len(cols) < channels:
        m = mods[i % len(mods)]
        cols.append((p * (1 + i // len(mods)) + i) % m)
        i += 1
    return torch.stack(cols[:channels], dim=-1).to(torch.float32)


def normal_bf16_device(shape, seed, device):
    """N(0,1) drawn on the GPU with a seeded device generator, rounded to bf16
    (for benchmark-sized caches that would be slow to draw on the CPU)."""
    g = torch.Generator(device=device).manual_seed(int(seed))
    return torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)


LOGIT_KINDS = ("lm", "flat", "bf16", "masked", "few", "equal", "spike")


def logits_f32(rows, vocab, g, kind="lm"):
    """FP32 logits [rows, vocab] of a few shapes a language-model head gives:
      lm      N(0, 2^2) plus 32 tokens per row raised by U(4, 12) (a peaked head);
      flat    N(0, 0.5^2) (a wide top-p set);
      bf16    lm rounded to bf16 (many equal logits);
      masked  -inf except 100 tokens drawn N(0, 1) (a constrained vocabulary);
      few     -inf except 5 tokens (fewer finite logits than a top-k of 20);
      equal   all zero (every logit tied);
      spike   N(0, 1) with one token at +60 (one token holds the mass)."""
    if kind == "equal":
        return torch.zeros((rows, vocab), dtype=torch.float32)
    if kind in ("lm", "bf16"):
        z = torch.randn((rows, vocab), generator=g) * 2.0
        n = min(32, vocab)
        for r in range(rows):
            idx = torch.randperm(vocab, generator=g)[:n]
            z[r, idx] += 4.0 + 8.0 * torch.rand(n, generator=g)
        return z.to(torch.bfloat16).float() if kind == "bf16" else z
    if kind == "flat":
        return torch.randn((rows, vocab), generator=g) * 0.5
    if kind in ("masked", "few"):
        n = min(100 if kind == "masked" else 5, vocab)
        z = torch.full((rows, vocab), float("-inf"))
        for r in range(rows):
            idx = torch.randperm(vocab, generator=g)[:n]
            z[r, idx] = torch.randn(n, generator=g)
        return z
    if kind == "spike":
        z = torch.randn((rows, vocab), generator=g)
        z[torch.arange(rows), torch.randint(0, vocab, (rows,), generator=g)] = 60.0
        return z
    raise ValueError(kind)
