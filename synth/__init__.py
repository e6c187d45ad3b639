"""Seeded synthetic inputs for the tests, the bench and the oracle checks.

This module holds random draws and the shapes of the workloads only -- none
of the quantization or attention arithmetic -- so both the oracle side and
the library side may use it.

The inputs copy the structures the pages name, not real model activations:
N(0,1) bodies, a few key channels with large magnitude (outlier channels),
and an attention-sink first token.  No dataset or trained weight is read.

Two generators:

* host draws with NumPy ``default_rng(seed)`` (PCG64), in the order
  q, K, V, outlier channel indices, outlier factors, drawn in float32 and then
  rounded to float16;
* a counter-based generator for caches too large to draw on the host: the
  SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014) applied to
  seed + (counter + 1) * 0x9E3779B97F4A7C15, i.e. the counter-th output of a
  SplitMix64 stream seeded with ``seed``; its four 16-bit lanes are summed
  (an Irwin-Hall approximation of a normal draw, integer-exact), centred,
  multiplied by one float32 constant and rounded to float16.  Every step is
  integer or a single correctly rounded float32 multiply, so any independent
  implementation of the same definition produces identical bytes.  The
  library carries its own device implementation (kvq_synth_normal_f16) for
  the bench; the tests compare the two byte for byte.
"""

import numpy as np

# ---------------------------------------------------------------------------
# host draws
# ---------------------------------------------------------------------------


def tiny_inputs(seed, n, d=32, n_query=8):
    """The small fp32 case: q [n_query][d], K [n][d], V [n][d] ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n_query, d), dtype=np.float32)
    k = rng.standard_normal((n, d), dtype=np.float32)
    v = rng.standard_normal((n, d), dtype=np.float32)
    return q, k, v


def tiny_condition(k, v, condition):
    """clean | kcol (K column 0 x40) | vrow (V row 0 x40), on copies."""
    k = k.copy()
    v = v.copy()
    if condition == "kcol":
        k[:, 0] *= np.float32(40.0)
    elif condition == "vrow":
        v[0, :] *= np.float32(40.0)
    elif condition != "clean":
        raise ValueError(condition)
    return k, v


def kv_inputs(seed, B, Hq, Hkv, N, D, outliers="per_head", n_out=4,
              out_factor=15.0, frac=0.02, fmin=10.0, fmax=30.0,
              sink_factor=None):
    """Decode-attention inputs: q fp16 [B][Hq][D], K, V fp16 [B][Hkv][N][D].

    outliers:
      "none"      clean N(0,1) keys;
      "per_head"  in every (batch, KV head) stream, ``n_out`` distinct random
                  key channels multiplied by ``out_factor``;
      "fraction"  round(frac * Hkv * D) distinct (KV head, channel) pairs,
                  shared by the batch, each multiplied by a factor drawn from
                  U[fmin, fmax].
    sink_factor: if set, token 0's K and V rows are multiplied by it.
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, N, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, N, D), dtype=np.float32)
    if outliers == "per_head":
        for b in range(B):
            for h in range(Hkv):
                ch = rng.choice(D, size=n_out, replace=False)
                k[b, h, :, ch] *= np.float32(out_factor)
    elif outliers == "fraction":
        n_pairs = int(round(frac * Hkv * D))
        pairs = rng.choice(Hkv * D, size=n_pairs, replace=False)
        factors = rng.uniform(fmin, fmax, size=n_pairs).astype(np.float32)
        for p, f in zip(pairs, factors):
            k[:, p // D, :, p % D] *= f
    elif outliers != "none":
        raise ValueError(outliers)
    if sink_factor is not None and N > 0:
        k[:, :, 0, :] *= np.float32(sink_factor)
        v[:, :, 0, :] *= np.float32(sink_factor)
    return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)


def query_window(seed, B, W, Hq, D):
    """The last W query rows for salience, fp16 [B][W][Hq][D] ~ N(0,1)."""
    rng = np.random.default_rng(seed + 1_000_003)
    return rng.standard_normal((B, W, Hq, D), dtype=np.float32).astype(
        np.float16)


# ---------------------------------------------------------------------------
# counter-based generator
# ---------------------------------------------------------------------------

GOLDEN_GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
TENSOR_K, TENSOR_V, TENSOR_Q = 0, 1, 2
# 1 / sqrt((2**32 - 1) / 3): the standard deviation of a sum of four
# independent uniform 16-bit integers is sqrt((2**32 - 1) / 3).
NORMAL_SCALE_F32 = np.float32(1.0 / np.sqrt((2.0 ** 32 - 1.0) / 3.0))


def _splitmix64_output(z):
    z = np.asarray(z, np.uint64)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
    return z ^ (z >> np.uint64(31))


def counter_index(tensor, layer, head, token, channel):
    """64-bit counter of one element (fields: 2+8+8+32+8 bits)."""
    t = np.asarray(token, np.uint64)
    c = np.asarray(channel, np.uint64)
    hi = np.uint64(((tensor * 256 + layer) * 256 + head))
    return ((hi << np.uint64(32)) + t) * np.uint64(256) + c


def counter_normal_f16(seed, tensor, layer, head, t0, n_tok, d):
    """fp16 [n_tok][d] block of the counter-based normal stream."""
    with np.errstate(over="ignore"):
        tok = np.arange(t0, t0 + n_tok, dtype=np.uint64)[:, None]
        ch = np.arange(d, dtype=np.uint64)[None, :]
        ctr = counter_index(tensor, layer, head, tok, ch)
        z = np.uint64(seed) + (ctr + np.uint64(1)) * np.uint64(GOLDEN_GAMMA)
        h = _splitmix64_output(z)
    lanes = [((h >> np.uint64(16 * i)) & np.uint64(0xFFFF)).astype(np.int64)
             for i in range(4)]
    s = lanes[0] + lanes[1] + lanes[2] + lanes[3] - 131070
    x = s.astype(np.float32) * NORMAL_SCALE_F32
    return x.astype(np.float16)


def counter_kv(seed, layer, Hkv, t0, n_tok, D, heads=None):
    """fp16 K, V [len(heads)][n_tok][D] for one layer of the counter stream."""
    heads = range(Hkv) if heads is None else heads
    k = np.stack([counter_normal_f16(seed, TENSOR_K, layer, h, t0, n_tok, D)
                  for h in heads])
    v = np.stack([counter_normal_f16(seed, TENSOR_V, layer, h, t0, n_tok, D)
                  for h in heads])
    return k, v


def counter_query(seed, layer, Hq, D):
    """fp16 q [Hq][D] for one layer (query head h uses head field h)."""
    return np.stack([counter_normal_f16(seed, TENSOR_Q, layer, h, 0, 1, D)[0]
                     for h in range(Hq)])


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

WORKLOADS = {
    # name: dict of shapes and cache parameters
    "tiny_int8": dict(B=1, Hq=8, Hkv=1, N=256, D=32, bits=8),
    "7b_layer_4k": dict(B=1, Hq=32, Hkv=32, N=4096, D=128, S=0, G=128,
                        Gv=32, R=128, k_bits=4, v_bits=2,
                        outliers="per_head", n_out=4, out_factor=15.0),
    "gqa_128k": dict(B=1, Hq=32, Hkv=8, N=131072, D=128, S=1, G=64, Gv=64,
                     R=64, k_bits=4, v_bits=2, outliers="fraction",
                     frac=0.02, fmin=10.0, fmax=30.0, sink_factor=20.0),
    # the same GQA layer with the bit widths swapped (the comparison run)
    "gqa_128k_k2v4": dict(B=1, Hq=32, Hkv=8, N=131072, D=128, S=1, G=64,
                          Gv=64, R=64, k_bits=2, v_bits=4, outliers="fraction",
                          frac=0.02, fmin=10.0, fmax=30.0, sink_factor=20.0),
    "mixkvq_32k": dict(B=8, Hq=40, Hkv=8, N=32768, D=128, S=0, G=128, Gv=64,
                       R=128, k_bits=2, v_bits=2, mixed=True, n_bf16=8,
                       n_int4=32, W=64, outliers="per_head", n_out=4,
                       out_factor=15.0),
    "1m_32layer": dict(B=1, Hq=32, Hkv=32, N=1048576, D=128, S=1, G=128,
                       Gv=32, R=128, k_bits=2, v_bits=2, layers=32,
                       chunk=4096),
    # the next rows on the 128K GQA layer: 3-bit codebook keys (per channel,
    # 128-token groups) and values (per token) with 1% per-vector outliers;
    # and the KQV scheme at a 4-bit budget (rotated keys at 4 bits, rotated
    # values at 3 bits plus the 1-bit sketch of m = 128 rows)
    "kvquant_3bit_1pct_128k": dict(B=1, Hq=32, Hkv=8, N=131072, D=128, G=128,
                                   Gv=128, k_bits=3, v_bits=3, k_nuq=True,
                                   v_nuq=True, n_out=1, outliers="fraction",
                                   frac=0.02, fmin=10.0, fmax=30.0,
                                   sink_factor=20.0),
    "kqv_4bit_128k": dict(B=1, Hq=32, Hkv=8, N=131072, D=128, G=128, Gv=32,
                          k_bits=4, v_bits=3, qjl_m=128, outliers="fraction",
                          frac=0.02, fmin=10.0, fmax=30.0, sink_factor=20.0),
}


# ---------------------------------------------------------------------------
# inputs of the non-uniform datatype and of the 1-bit residual sketch
# ---------------------------------------------------------------------------


def nuq_codebook(bits):
    """A synthetic non-uniform codebook of 2**bits levels in [-1, 1].

    The pages' codebooks come from a sensitivity-weighted k-means over real
    activations ("KVQuant ...", Approach), which needs model data; this one
    is built the way NormalFloat levels are (the page names NormalFloat as a
    basis): quantiles of N(0, 1), 2**(bits-1) positive and 2**(bits-1) - 1
    negative ones at evenly spaced probabilities in (0.5, 0.97], each side
    normalized so its outermost level is exactly +-1, plus an exact 0, every
    level rounded to fp16.  Returns float32 [2**bits], strictly ascending.
    """
    from scipy.stats import norm

    n = 1 << bits
    n_pos, n_neg = n // 2, n // 2 - 1
    pos = norm.ppf(np.linspace(0.5, 0.97, n_pos + 1)[1:])
    neg = norm.ppf(np.linspace(0.5, 0.97, n_neg + 1)[1:]) if n_neg else np.zeros(0)
    pos = pos / pos[-1]
    neg = -(neg / neg[-1]) if n_neg else neg
    levels = np.concatenate([neg[::-1], [0.0], pos]).astype(np.float16)
    return levels.astype(np.float32)


def jl_matrix(seed, m, d):
    """The Gaussian projection of the 1-bit sketch: float32 [m][d], i.i.d.
    N(0, 1) from default_rng(seed + 2_000_003)."""
    rng = np.random.default_rng(seed + 2_000_003)
    return rng.standard_normal((m, d), dtype=np.float32)
