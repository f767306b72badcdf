"""KV-cache codec of the quantized variant, written from the formats' definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Qwen3.8-27B on one RTX 4090", section "A cheaper cache and state": keys are
FP8 after a Hadamard rotation, values INT8.  Readings where the page is
silent:
* FP8 is the OCP E4M3FN format: 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, subnormals when the exponent field is 0, no infinities, and
  the two codes 0x7F / 0xFF are NaN; the largest finite value is 448.
  Encoding rounds to nearest, ties to even, and saturates at +-448.
* The rotation is the 128-point Walsh-Hadamard matrix in natural (Sylvester)
  order, H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]], divided by sqrt(128);
  the same rotation is applied to q so that scores are unchanged.
* Values: one FP32 scale per (token, KV head), s = max|v| / 127; codes are
  round-half-even of v / s clamped to [-127, 127]; s = 0 gives all-zero codes.
  Dequantisation is code * s.
* Where a code is decided from a rotated key, the rotation is taken in FP32
  (`wht_f32`, the precision a GPU encoder works in) so that both sides round
  the same value.
"""

import numpy as np


def e4m3_decode(codes):
    """Decode uint8 E4M3FN codes to float64 from the bit fields."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    mant = c & 0x7
    normal = sign * (1.0 + mant / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * (mant / 8.0) * np.exp2(-6.0)
    out = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (mant == 7), np.nan, out)


def e4m3_encode(x):
    """Nearest finite E4M3FN code, ties to the even code, saturating at 448.

    The positive finite codes 0x00..0x7E decode to increasing values, so the
    two candidates for |x| are its neighbours in that sorted list; the nearer
    one wins and an exact tie goes to the code whose last bit is 0.  The sign
    bit is copied from x, as in IEEE rounding (a negative value that rounds to
    zero gives -0, code 0x80).  NaN maps to 0x7F.
    """
    x = np.asarray(x, dtype=np.float64)
    pos_codes = np.arange(0x7F)                            # 0x00..0x7E
    pos_vals = e4m3_decode(pos_codes)
    assert np.all(np.diff(pos_vals) > 0)
    a = np.minimum(np.abs(np.nan_to_num(x)), 448.0)
    hi = np.clip(np.searchsorted(pos_vals, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = np.abs(a - pos_vals[lo])
    d_hi = np.abs(pos_vals[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    out = np.where(pick_hi, hi, lo).astype(np.int64)
    out = np.where(np.signbit(x), out | 0x80, out)
    return np.where(np.isnan(x), 0x7F, out).astype(np.uint8)


def hadamard(n):
    """Sylvester Hadamard matrix of order n (a power of two), entries +-1."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    if h.shape[0] != n:
        raise ValueError("order must be a power of two")
    return h


def wht(x):
    """Normalised rotation x -> H x / sqrt(n) along the last axis."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    return x @ hadamard(n).T / np.sqrt(n)


def wht_f32(x):
    """The normalised rotation as a GPU computes it in FP32: the fast
    Walsh-Hadamard transform in natural order, one butterfly stage per bit of
    the index from the lowest (width 1, 2, 4, ..., n/2), each stage replacing
    the pair (a, b) at indices (i, i + width) by (a + b, a - b) in float32,
    then a float32 multiply by float32(1/sqrt(n)).

    Rounding the rotated key to FP8 is decided on this FP32 value, so an
    encoder in FP32 and this function must agree bit for bit; the float64
    `wht` is the definition it approximates (to FP32 rounding).
    """
    y = np.array(x, dtype=np.float32, copy=True)
    n = y.shape[-1]
    if n & (n - 1):
        raise ValueError("length must be a power of two")
    width = 1
    while width < n:
        z = y.reshape(y.shape[:-1] + (n // (2 * width), 2, width))
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(y.shape)
        width *= 2
    return y * np.float32(1.0 / np.sqrt(n))


def encode_keys_f32(k):
    """E4M3FN codes of the FP32-rotated keys: e4m3_encode(wht_f32(k))."""
    return e4m3_encode(wht_f32(k).astype(np.float64))


def i8_encode(v):
    """Per-row INT8 codes and FP32 scale.  v: [..., D] -> (codes, scale[...])."""
    v = np.asarray(v, dtype=np.float64)
    amax = np.abs(v).max(axis=-1)
    scale = (amax / 127.0).astype(np.float32)
    s64 = scale.astype(np.float64)[..., None]
    safe = np.where(s64 == 0, 1.0, s64)
    q = np.clip(np.round(v / safe), -127, 127)             # np.round: half to even
    q = np.where(s64 == 0, 0, q)
    return q.astype(np.int8), scale


def i8_decode(codes, scale):
    """code * scale in float64 (exact)."""
    return np.asarray(codes, np.float64) * np.asarray(scale, np.float64)[..., None]
