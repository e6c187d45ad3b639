"""Oracle of decode attention over keys cached before the rotary embedding.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Slow and literal.

Sources (page title, section):

* "KVQuant: Towards 10 Million Context Length LLM Inference with KV Cache
  Quantization", summary and "Approach": keys are quantized per channel
  before the rotary position embedding is applied (pre-RoPE); the table of
  measured effects credits this with a perplexity gain at 3 bits.  The
  embedding is then applied to the dequantized keys when attention reads
  them.

Readings where the pages leave a step open (they give no formula for the
embedding itself):

* the embedding is the rotary form with frequencies
  theta_f = base ** (-2 f / D), f = 0 .. D/2 - 1 (base 10000 unless given);
  at position p, the channel pair (a, b) of frequency f is rotated by the
  angle p * theta_f:  (x_a, x_b) -> (x_a cos - x_b sin, x_a sin + x_b cos);
* two pair layouts: "half" pairs channel f with channel f + D/2 (the layout
  of the LLaMA-family checkpoints the KVQuant page evaluates), and
  "interleaved" pairs channel 2f with channel 2f + 1;
* every cached key (sink, quantized groups and tail alike) is stored before
  the rotation; token i of the cache order (sink, quantized, tail) sits at
  position pos0 + i; the decoding query is handed over already rotated at
  its own position, so only the keys are rotated here;
* everything is computed in float64 (angles, cosines, sines, products).
"""
import numpy as np

from . import attention as _attention

PAIRINGS = ("half", "interleaved")


def theta(d, base=10000.0):
    """Angle per position of every frequency, float64 [D/2]."""
    if d < 2 or d % 2:
        raise ValueError("the rotary embedding needs an even head_dim")
    f = np.arange(d // 2, dtype=np.float64)
    return np.float64(base) ** (-2.0 * f / d)


def pair_channels(d, pairing="half"):
    """(a, b): the two channels of every frequency f, int arrays [D/2]."""
    f = np.arange(d // 2)
    if pairing == "half":
        return f, f + d // 2
    if pairing == "interleaved":
        return 2 * f, 2 * f + 1
    raise ValueError("pairing is 'half' or 'interleaved'")


def rotate(x, positions, base=10000.0, pairing="half"):
    """Rotate rows of x [..., N, D] at positions [N] (integers); float64."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    a, b = pair_channels(d, pairing)
    ang = np.asarray(positions, np.float64)[:, None] * theta(d, base)[None, :]
    c, s = np.cos(ang), np.sin(ang)                   # [N][D/2]
    out = np.empty_like(x)
    out[..., a] = x[..., a] * c - x[..., b] * s
    out[..., b] = x[..., a] * s + x[..., b] * c
    return out


def attention(q, k_hat, v_hat, pos0=0, base=10000.0, pairing="half",
              sm_scale=None):
    """Attention of rotated queries q [Hq][D] over pre-RoPE dequantized keys
    k_hat [Hkv][N][D] (cache order) and values v_hat [Hkv][N][D]: each key
    is rotated at position pos0 + i first.  float64 [Hq][D]."""
    k = np.asarray(k_hat, np.float64)
    pos = pos0 + np.arange(k.shape[1])
    return _attention.attention(q, rotate(k, pos, base, pairing), v_hat,
                                sm_scale)
