"""Oracle codec: the symmetric absmax rule, its grouping axes, packing, dequant.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Slow and literal.

Sources (page title, section):

* "KV quantization axes: why Key and Value need separate reasoning"
  (huhohoo.com), section "What rows and columns mean": every scheme uses one
  symmetric rule -- the scale of a group is its largest magnitude divided by
  the largest code (127 for int8), the code is the rounded quotient clipped to
  the code range, and the reconstruction is code times scale.  The same
  section defines the three groupings: one scale for the whole matrix
  (tensor), one per row (token) and one per column (channel).
* same page, closing troubleshooting paragraph: token scales have shape (N,1)
  and channel scales (1,D); a group whose values are all zero uses scale 1;
  NaN or Inf inputs are refused.
* "KVQuant: Towards 10 Million Context Length LLM Inference with KV Cache
  Quantization", table "Measured effects reported in the paper": keys are
  quantized per channel and values per token.
* "MixKVQ: Query-Aware Mixed-Precision KV Cache Quantization ...", Figure 3:
  some key channels are kept in BF16.

Readings where the pages leave a step open:

* the largest code for b bits is qmax = 2**(b-1) - 1 (the page prints only
  the int8 value 127), so int2 codes are {-1, 0, 1};
* ``round`` is round-half-to-even (the page's NumPy ``round``/``rint``);
* the quotient x/scale and the scale m/qmax are IEEE float32 divisions (the
  page's source arrays are float32);
* a scale that underflows to 0 for a nonzero group is treated like a zero
  group (scale 1);
* codes are stored offset-binary, u = code + 2**(b-1), packed LSB-first into
  little-endian uint32 words, one row per token, floor(32/b) fields per word,
  unused high bits zero.
"""

import numpy as np

VALID_BITS = (8, 4, 3, 2)


class NonFiniteInput(ValueError):
    """The pages refuse NaN/Inf input; the oracle raises this."""


def qmax_for_bits(bits):
    """Largest code magnitude for a b-bit symmetric code: 2**(b-1) - 1."""
    if bits not in VALID_BITS:
        raise ValueError(f"bits must be one of {VALID_BITS}, got {bits}")
    return (1 << (bits - 1)) - 1


def _as_f32(x):
    a = np.asarray(x)
    if a.dtype not in (np.float16, np.float32):
        raise TypeError("codec input must be float16 or float32")
    a = a.astype(np.float32)  # float16 -> float32 is exact
    if not np.all(np.isfinite(a)):
        raise NonFiniteInput("NaN/Inf input is rejected")
    return a


def quantize_groups(x, bits):
    """Apply the rule independently to every row of x[..., n].

    The last axis holds one group.  Returns (codes int32 of x's shape,
    scales float32 of x.shape[:-1]).
    """
    qmax = qmax_for_bits(bits)
    v = _as_f32(x)
    if v.shape[-1] == 0:
        return (np.zeros(v.shape, np.int32),
                np.ones(v.shape[:-1], np.float32))
    m = np.max(np.abs(v), axis=-1).astype(np.float32)
    scale = (m / np.float32(qmax)).astype(np.float32)  # IEEE float32 division
    zero = (m == 0) | (scale == 0)  # zero group (or underflowed scale)
    scale = np.where(zero, np.float32(1.0), scale).astype(np.float32)
    q = (v / scale[..., None]).astype(np.float32)  # IEEE float32 quotient
    code = np.clip(np.rint(q), -qmax, qmax).astype(np.int32)
    return code, scale


def quantize_group(x, bits):
    """Quantize one group of values with the symmetric absmax rule.

    Returns (codes int32 array of x's shape, scale as np.float32).
    """
    a = np.asarray(x)
    codes, scales = quantize_groups(a.reshape(1, -1), bits)
    return codes.reshape(a.shape), np.float32(scales[0])


def quantize_matrix(x, bits, axis):
    """Quantize an N x D matrix with one of the page's three groupings.

    axis = "tensor": one scale, shape (1, 1)
    axis = "token":  one scale per row, shape (N, 1)
    axis = "channel": one scale per column, shape (1, D)
    Returns (codes int32 [N][D], scales float32 of the shape above).
    """
    a = _as_f32(x)
    n, d = a.shape
    codes = np.zeros((n, d), np.int32)
    if axis == "tensor":
        c, s = quantize_group(a, bits)
        return c, np.full((1, 1), s, np.float32)
    if axis == "token":
        scales = np.zeros((n, 1), np.float32)
        for t in range(n):
            codes[t, :], scales[t, 0] = quantize_group(a[t, :], bits)
        return codes, scales
    if axis == "channel":
        scales = np.zeros((1, d), np.float32)
        for c in range(d):
            codes[:, c], scales[0, c] = quantize_group(a[:, c], bits)
        return codes, scales
    raise ValueError(axis)


def quantize_k(k, bits, group_tok):
    """Per-channel key quantization, groups of ``group_tok`` consecutive tokens.

    k: [N][D] (float16/float32).  Returns codes int32 [N][D] and scales
    float32 [ceil(N/G)][D]; the last, partial group uses its own absmax.
    """
    a = _as_f32(k)
    n, d = a.shape
    if group_tok <= 0:
        raise ValueError("group_tok must be positive")
    n_groups = (n + group_tok - 1) // group_tok
    codes = np.zeros((n, d), np.int32)
    scales = np.zeros((n_groups, d), np.float32)
    for g in range(n_groups):
        t0, t1 = g * group_tok, min(n, (g + 1) * group_tok)
        # one group per channel: the channel's G values along the tokens
        c, s = quantize_groups(a[t0:t1, :].T, bits)
        codes[t0:t1, :] = c.T
        scales[g, :] = s
    return codes, scales


def quantize_v(v, bits, group_ch):
    """Per-token value quantization, groups of ``group_ch`` consecutive channels.

    v: [N][D].  Returns codes int32 [N][D] and scales float32 [N][D/Gv].
    """
    a = _as_f32(v)
    n, d = a.shape
    if group_ch <= 0 or d % group_ch:
        raise ValueError("group_ch must divide D")
    ng = d // group_ch
    c, s = quantize_groups(a.reshape(n, ng, group_ch), bits)
    return c.reshape(n, d), s.reshape(n, ng)


def fields_per_word(bits):
    return 32 // bits


def words_per_row(n_fields, bits):
    pw = fields_per_word(bits)
    return (n_fields + pw - 1) // pw


def pack_rows(codes, bits):
    """Pack signed codes [rows][fields] into uint32 words, offset binary.

    Field j of a row goes to word j // floor(32/b), at bit (j % floor(32/b))*b.
    """
    c = np.asarray(codes, np.int64)
    rows, nf = c.shape
    qmax = qmax_for_bits(bits)
    if np.any(np.abs(c) > qmax):
        raise ValueError("code out of range")
    u = (c + (1 << (bits - 1))).astype(np.uint64)
    pw = fields_per_word(bits)
    nw = words_per_row(nf, bits)
    out = np.zeros((rows, nw), np.uint64)
    for j in range(nf):
        out[:, j // pw] |= u[:, j] << np.uint64((j % pw) * bits)
    return out.astype(np.uint32)


def unpack_rows(words, bits, n_fields):
    """Inverse of pack_rows: uint32 [rows][words] -> signed codes int32."""
    w = np.asarray(words, np.uint64)
    pw = fields_per_word(bits)
    mask = np.uint64((1 << bits) - 1)
    out = np.zeros((w.shape[0], n_fields), np.int64)
    for j in range(n_fields):
        out[:, j] = (w[:, j // pw] >> np.uint64((j % pw) * bits)) & mask
    return (out - (1 << (bits - 1))).astype(np.int32)


def dequant(codes, scales_full):
    """x_hat = code * scale, in float64 (exact for these operands)."""
    return np.asarray(codes, np.float64) * np.asarray(scales_full, np.float64)


def dequant_f32(codes, scales_full):
    """The float32 reconstruction fl32(code * scale) (round to nearest even)."""
    return (np.asarray(codes, np.float32) *
            np.asarray(scales_full, np.float32)).astype(np.float32)


def expand_k_scales(scales, n_tok, group_tok):
    """[ceil(N/G)][D] -> [N][D]: token t uses the scale of group t // G."""
    idx = np.arange(n_tok) // group_tok
    return np.asarray(scales)[idx, :]


def expand_v_scales(scales, d, group_ch):
    """[N][D/Gv] -> [N][D]: channel c uses the scale of group c // Gv."""
    idx = np.arange(d) // group_ch
    return np.asarray(scales)[:, idx]


def f32_to_bf16_bits(x):
    """Round float32 to bfloat16, nearest-even, returning the uint16 pattern.

    Written from the format: bfloat16 keeps the upper 16 bits of the float32
    pattern; rounding to nearest-even adds 0x7FFF plus the lowest kept bit
    before truncation.  Finite inputs only.
    """
    a = np.asarray(x, np.float32)
    if not np.all(np.isfinite(a)):
        raise NonFiniteInput("NaN/Inf input is rejected")
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return (r & np.uint64(0xFFFF)).astype(np.uint16)


def bf16_bits_to_f32(b):
    """Exact widening of a bfloat16 pattern to float32."""
    return (np.asarray(b, np.uint32) << np.uint32(16)).view(np.float32)
