"""Oracle key rotation: the normalized Walsh-Hadamard transform of a row.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Slow and literal.

Sources (page title, section):

* "Quantize What Counts: More for Keys, Less for Values", Technical Summary,
  "Results", rotation integration: rotating the keys alone (K4V2) brings
  accuracy close to K4V4, because the rotation spreads key outliers;
  rotating values adds little.
* "Statistical Inference and Quality Measures of KV Cache Quantisations
  Inspired by TurboQuant", the KQV scheme: a Walsh-Hadamard transform is
  applied before scalar quantization.

Readings where the pages leave a step open:

* the rotation is the Sylvester Walsh-Hadamard matrix of order d (a power
  of two) scaled by 1/sqrt(d), with no random sign flips, so it is
  orthonormal and its own inverse: q . k = (R q) . (R k);
* it is computed in float32 by the fast transform: stages h = 1, 2, 4, ...,
  d/2, each replacing the pair (x[i], x[i + h]) of every index i with bit h
  clear by (x[i] + x[i + h], x[i] - x[i + h]); then every element is
  multiplied by float32(1 / sqrt(d)); a float16 result is that float32
  value rounded to nearest even.  Each step is one IEEE float32 operation,
  so the result is fixed bit for bit.
"""
import numpy as np


def sylvester(d):
    """The d x d Sylvester Hadamard matrix (entries +1 / -1), d a power of two:
    H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def scale32(d):
    """float32(1 / sqrt(d)), the factor applied after the butterflies."""
    return np.float32(1.0 / np.sqrt(np.float64(d)))


def wht(x, out_dtype=np.float32):
    """Rotate the last axis of x (float16 or float32) as described above.

    Returns float32 or float16 (out_dtype)."""
    a = np.array(x, dtype=np.float32, copy=True)
    d = a.shape[-1]
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = 1
    while h < d:
        for i in range(d):
            if i & h:
                continue
            u = a[..., i].copy()
            v = a[..., i + h].copy()
            a[..., i] = u + v          # float32 + float32, rounded once
            a[..., i + h] = u - v
        h *= 2
    a = a * scale32(d)                 # float32 * float32, rounded once
    if out_dtype == np.float16:
        return a.astype(np.float16)    # round to nearest even
    if out_dtype != np.float32:
        raise TypeError("out_dtype is float32 or float16")
    return a
