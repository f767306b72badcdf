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
* A key's code is e4m3_encode(wht(k)), the rotation in float64.  An encoder
  that rotates in FP32 may round a value within FP32 error of an E4M3 rounding
  midpoint to the other neighbour; `e4m3_codes_acceptable` takes the
  definition's code wherever the FP32 error bound of the rotation
  (`wht_f32_error_bound`) keeps every midpoint away, and either neighbour
  elsewhere.
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


# FP32 rounding-error bound of an encoder's rotation, in units of 2^-24:
# every fast 128-point Walsh-Hadamard transform is seven levels of additions
# and subtractions, and the result is scaled by the FP32-rounded 1/sqrt(128)
# (before or after the levels).  The computed sum of n signed terms through a
# tree of depth d is within d*u*(1 + d*u)*sum|x| of the exact sum (u = 2^-24,
# the unit roundoff of round-to-nearest); the FP32 scale constant and the
# product's rounding add u*sum|x|/sqrt(n) and u*|y|.  The constants below
# cover those terms with margin.
WHT_F32_ERR_SUM = 9.0
WHT_F32_ERR_OUT = 2.0


def wht_f32_error_bound(x):
    """Upper bound on |fl32(H x / sqrt(n)) - H x / sqrt(n)| for any FP32
    encoder of the rotation (see the constants above), per output element:
    (9 * sum|x| / sqrt(n) + 2 |y|) * 2^-24, broadcast over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    y = wht(x)
    s = np.abs(x).sum(axis=-1, keepdims=True) / np.sqrt(n)
    return (WHT_F32_ERR_SUM * s + WHT_F32_ERR_OUT * np.abs(y)) * 2.0 ** -24 * (1 + 1e-9)


def e4m3_code_interval(y, bound):
    """Codes that an encoder may store for the exact value y when it rounds a
    value it computed within `bound` of y: (lo, hi) = (e4m3_encode(y - bound),
    e4m3_encode(y + bound)), and `decided` = no E4M3 rounding midpoint (and
    no zero) lies within the bound, so that the code is unique (lo == hi).
    Elsewhere every code whose value lies in [value(lo), value(hi)] is a
    correct rounding of some value in the interval."""
    y = np.asarray(y, dtype=np.float64)
    b = np.broadcast_to(np.asarray(bound, dtype=np.float64), y.shape)
    lo = e4m3_encode(y - b)
    hi = e4m3_encode(y + b)
    decided = (lo == hi) & ~((y - b <= 0) & (y + b >= 0))
    return lo, hi, decided


def e4m3_codes_acceptable(codes, y, bound):
    """Per element: True where `codes` is a correct E4M3FN code for an encoder
    whose rotated value lies within `bound` of the exact y (the definition's
    code where it is decided; a code between the interval's end codes
    elsewhere; 0x7F where y is NaN).  Returns (ok, decided)."""
    codes = np.asarray(codes, dtype=np.uint8)
    y = np.asarray(y, dtype=np.float64)
    lo, hi, decided = e4m3_code_interval(np.nan_to_num(y), bound)
    v = e4m3_decode(codes)
    inside = (v >= e4m3_decode(lo)) & (v <= e4m3_decode(hi))
    ok = np.where(decided, codes == lo, inside & ~np.isnan(v))
    nan = np.isnan(y)
    return np.where(nan, codes == 0x7F, ok), decided & ~nan


def _rne(x):
    """Round half to even (numpy's rounding of exact halves)."""
    return np.round(x)


def i8_encode(v):
    """Per-row INT8 codes and FP32 scale.  v: [..., D] -> (codes, scale[...]).

    s = max|v| / 127 rounded to FP32 (the float64 quotient of a value with at
    most 24 significant bits by 127 never lies on an FP32 rounding midpoint,
    so rounding it again to FP32 is the correctly rounded FP32 quotient);
    codes = round-half-even(v / s) clamped to [-127, 127].  v / s is taken in
    float64: for v with at most 24 significant bits and |v / s| <= 127.5 the
    float64 quotient lies on a half-integer only when the exact one does, so
    the rounding is that of the exact quotient.  s = 0 gives zero codes.  A
    row holding NaN or an infinity has a NaN or infinite scale and zero codes
    (its dequantised values are then NaN)."""
    v = np.asarray(v, dtype=np.float64)
    amax = np.abs(v).max(axis=-1)                          # NaN propagates
    with np.errstate(invalid="ignore", over="ignore"):
        scale = (amax / 127.0).astype(np.float32)
    s64 = scale.astype(np.float64)[..., None]
    usable = np.isfinite(s64) & (s64 != 0)
    safe = np.where(usable, s64, 1.0)
    with np.errstate(invalid="ignore"):
        q = np.clip(_rne(np.where(usable, v, 0.0) / safe), -127, 127)
    q = np.where(usable, q, 0)
    return q.astype(np.int8), scale


def i8_decode(codes, scale):
    """code * scale in float64 (exact)."""
    return np.asarray(codes, np.float64) * np.asarray(scale, np.float64)[..., None]
