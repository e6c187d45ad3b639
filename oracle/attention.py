"""Oracle of decode attention over a dequantized KV cache, in float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Sources (page title, section):

* "KV quantization axes ...", "Separate the two error paths": the key error
  enters through Q K^T / sqrt(D) and the softmax weights, the value error
  through the weighted sum; attention is a numerically stable softmax
  computed in float64, and quantized codes are restored to float64 before
  any multiplication.
* same page, "The hybrid wins one condition and loses others": the error
  measure is the L2 norm of (output - reference) over the L2 norm of the
  reference.

Readings where the pages leave a step open: query head h reads KV head h // (Hq/Hkv);
the scale is 1/sqrt(D); there is no mask (a decoding query sees every cached
token); the output is float32-comparable float64 [Hq][D].
"""

import numpy as np


def attention(q, k_hat, v_hat, sm_scale=None):
    """softmax(q K^T * sm_scale) V per query head, float64.

    q: [Hq][D]; k_hat, v_hat: [Hkv][N][D] (any float dtype; widened to fp64).
    Returns [Hq][D] float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k_hat, np.float64)
    v = np.asarray(v_hat, np.float64)
    hq, d = q.shape
    hkv, n, _ = k.shape
    if n == 0:
        raise ValueError("attention over an empty cache is undefined")
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    out = np.zeros((hq, d), np.float64)
    for h in range(hq):
        kvh = h // g
        s = (k[kvh] @ q[h]) * sm_scale          # scores, [N]
        p = np.exp(s - np.max(s))               # stable softmax numerator
        out[h] = (p @ v[kvh]) / np.sum(p)
    return out


def softmax_weights(q, k_hat, sm_scale=None):
    """The normalized softmax rows, [Hq][N] float64 (for invariant tests)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k_hat, np.float64)
    hq, d = q.shape
    hkv = k.shape[0]
    g = hq // hkv
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    rows = []
    for h in range(hq):
        s = (k[h // g] @ q[h]) * sm_scale
        p = np.exp(s - np.max(s))
        rows.append(p / np.sum(p))
    return np.stack(rows)


def relative_error(out, ref):
    """||out - ref||_2 / ||ref||_2 over the whole array, float64."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(out - ref) / np.linalg.norm(ref))


def max_row_relative_error(out, ref):
    """The largest per-row relative L2 error over the leading axes."""
    out = np.asarray(out, np.float64).reshape(-1, np.shape(out)[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    num = np.linalg.norm(out - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return float(np.max(num / den))
