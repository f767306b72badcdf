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
