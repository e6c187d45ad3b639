"""Oracle for MixKVQ channel salience and precision classes.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Source: "MixKVQ: Query-Aware Mixed-Precision KV Cache Quantization for
Long-Context Reasoning" (sciencestack.ai), Figure 3 caption: a key channel's
salience is the product of the query's average activation intensity on that
channel (I) and the channel's key scale (S); the channels with the highest
product are kept in BF16, the next ones in INT4, the rest in INT2.  Figure 4
caption: salience is refreshed every R tokens inside the window.

Readings where the pages leave a step open:

* I_d is the plain sum of |q| over the last W query rows and over the query
  heads that share the KV head (a sum, not a mean: dividing every channel by
  the same count cannot change the ranking).  Each |q| is a float16 value and
  at most a few thousand are summed, so the float64 sum is exact and its
  order is irrelevant.
* S_d is the largest |K[t, d]| over the G tokens of the group being flushed
  (the "key scale" up to the common factor 1/qmax).
* A_d = I_d * S_d in float64; channels are ranked by A descending, ties going
  to the lower channel index.
* Before any salience is set, I_d = 1 for every channel (ranking by key scale
  alone).
"""

import numpy as np

CLASS_BF16, CLASS_INT4, CLASS_INT2 = 0, 1, 2
CLASS_BITS = {CLASS_INT4: 4, CLASS_INT2: 2}


def intensity(q_win, n_kv_heads):
    """I[kvh][d] = sum over rows and grouped query heads of |q|, float64.

    q_win: [W][Hq][D] float16 (the last W query rows of one batch element).
    Query head h belongs to KV head h // (Hq // Hkv).
    """
    q = np.asarray(q_win)
    if q.dtype != np.float16:
        raise TypeError("query window is float16")
    w, hq, d = q.shape
    if hq % n_kv_heads:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // n_kv_heads
    out = np.zeros((n_kv_heads, d), np.float64)
    for kvh in range(n_kv_heads):
        acc = np.zeros(d, np.float64)
        for r in range(w):
            for h in range(kvh * g, (kvh + 1) * g):
                acc = acc + np.abs(q[r, h, :].astype(np.float64))
        out[kvh] = acc
    return out


def group_key_scale(k_group):
    """S_d = max over the group's tokens of |K[t, d]| (float32, exact)."""
    a = np.asarray(k_group).astype(np.float32)
    return np.max(np.abs(a), axis=0)


def classes(I, S, n_bf16, n_int4):
    """Precision class of each channel from A = I * S.

    Returns int array [D] with CLASS_BF16 / CLASS_INT4 / CLASS_INT2.
    """
    I = np.asarray(I, np.float64)
    S = np.asarray(S, np.float32).astype(np.float64)
    d = I.shape[0]
    if n_bf16 < 0 or n_int4 < 0 or n_bf16 + n_int4 > d:
        raise ValueError("class counts exceed D")
    A = I * S
    order = sorted(range(d), key=lambda c: (-A[c], c))
    cls = np.full(d, CLASS_INT2, np.int32)
    for rank, c in enumerate(order):
        if rank < n_bf16:
            cls[c] = CLASS_BF16
        elif rank < n_bf16 + n_int4:
            cls[c] = CLASS_INT4
    return cls
