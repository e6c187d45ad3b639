"""Oracle of the non-uniform (codebook) datatype with dense-and-sparse outliers.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Source: "KVQuant: Towards 10 Million Context Length LLM Inference with KV
Cache Quantization" (atlas.scime.ai summary): the summary and "Approach"
(non-uniform nuqX datatypes; per-vector dense-and-sparse outlier isolation),
and the table "Measured effects reported in the paper" (1% outliers; per-vector
outlier thresholds beat a single per-matrix threshold; keys per channel,
values per token).

The page gives no formula, so the plainest readings are taken:

* a "vector" is what one scale covers: for keys one channel of a group of G
  consecutive tokens, for values one group of Gv channels of one token;
* per-vector isolation keeps the n_out entries of largest magnitude of each
  vector (ties to the lower index) exactly, in a sparse structure (their
  position in the vector and their fp16 value); 1% outliers of a 128-entry
  vector is round(1.28) = 1 entry;
* the dense part is the vector with those entries set to zero; its scale is
  its largest magnitude divided by the largest codebook magnitude (one IEEE
  float32 division; a zero dense part uses scale 1), and each entry's code
  is the index of the codebook level nearest to fl32(x / scale) (ties to the
  lower index);
* the reconstruction is dense + sparse: level[code] * scale everywhere,
  plus each kept outlier's value at its position (the codebook holds an
  exact 0, which every outlier position's dense entry quantizes to);
* the codebook (nuqX: 2**X levels, ascending, fp16-representable, with 0)
  is an input; the pages calibrate it by k-means on real activations, which
  is out of scope.
"""

import numpy as np

VALID_BITS = (2, 3, 4)


def check_codebook(lut, bits):
    lut = np.asarray(lut, np.float32)
    if bits not in VALID_BITS or lut.shape != (1 << bits,):
        raise ValueError("codebook must hold 2**bits levels, bits in (2, 3, 4)")
    if not np.all(np.diff(lut.astype(np.float64)) > 0):
        raise ValueError("codebook levels must be strictly ascending")
    if not np.any(lut == 0.0):
        raise ValueError("codebook must contain 0")
    if not np.array_equal(lut.astype(np.float16).astype(np.float32), lut):
        raise ValueError("codebook levels must be fp16 numbers")
    return lut


def nearest_level(q, lut):
    """Index of the level nearest to each float32 q (ties to the lower
    index): |q - level| is exact in float64 for these operands."""
    q = np.asarray(q, np.float32).astype(np.float64)
    d = np.abs(q[..., None] - np.asarray(lut, np.float64))
    return np.argmin(d, axis=-1).astype(np.int32)   # first minimum on ties


def select_outliers(x, n_out):
    """Positions of the n_out entries of largest |x| (ties to the lower
    index), ascending."""
    a = np.abs(np.asarray(x, np.float32).astype(np.float64))
    k = min(n_out, a.shape[0])
    order = sorted(range(a.shape[0]), key=lambda i: (-a[i], i))
    return np.array(sorted(order[:k]), np.int64)


def quantize_vector(x, lut, n_out):
    """One vector: (codes int32 [n], scale float32, outlier positions
    [n_out], outlier values float16 [n_out]).  Outlier slots past the
    vector's length (a vector shorter than n_out) are padding: position 0,
    value +0."""
    x = np.asarray(x)
    if x.dtype != np.float16:
        raise TypeError("the dense-and-sparse quantizer takes float16 input")
    xf = x.astype(np.float32)
    if not np.all(np.isfinite(xf)):
        raise ValueError("NaN/Inf input is rejected")
    idx = select_outliers(xf, n_out)
    dense = xf.copy()
    dense[idx] = 0.0
    m = np.float32(np.max(np.abs(dense))) if dense.size else np.float32(0)
    L = np.float32(np.max(np.abs(lut)))
    scale = np.float32(m / L)                       # IEEE float32 division
    if m == 0 or scale == 0:
        scale = np.float32(1.0)
    q = (dense / scale).astype(np.float32)          # IEEE float32 quotient
    codes = nearest_level(q, lut)
    out_pos = np.zeros(n_out, np.int64)
    out_val = np.zeros(n_out, np.float16)
    out_pos[:idx.size] = idx
    out_val[:idx.size] = x[idx]
    return codes, scale, out_pos, out_val


def dequant_vector(codes, scale, out_pos, out_val, lut):
    """dense + sparse in float64: level[code] * scale (exact: an fp16 level
    times a float32 scale), then each outlier value added at its position."""
    lut = np.asarray(lut, np.float64)
    x = lut[np.asarray(codes)] * np.float64(scale)
    for p, v in zip(out_pos, out_val):
        x[int(p)] += float(v)
    return x


def quantize_k(k, lut, group_tok, n_out):
    """Keys [N][D] fp16, one vector per (group of G tokens, channel).

    Returns codes int32 [N][D], scales float32 [ng][D], outlier positions
    (token within the group) [ng][D][n_out] and values fp16 [ng][D][n_out].
    """
    k = np.asarray(k)
    n, d = k.shape
    ng = (n + group_tok - 1) // group_tok
    codes = np.zeros((n, d), np.int32)
    scales = np.zeros((ng, d), np.float32)
    pos = np.zeros((ng, d, n_out), np.int64)
    val = np.zeros((ng, d, n_out), np.float16)
    for g in range(ng):
        t0, t1 = g * group_tok, min(n, (g + 1) * group_tok)
        for c in range(d):
            cc, s, p, v = quantize_vector(k[t0:t1, c], lut, n_out)
            codes[t0:t1, c], scales[g, c], pos[g, c], val[g, c] = cc, s, p, v
    return codes, scales, pos, val


def quantize_v(v, lut, group_ch, n_out):
    """Values [N][D] fp16, one vector per (token, group of Gv channels).

    Returns codes int32 [N][D], scales float32 [N][D/Gv], outlier positions
    (channel within the group) [N][D/Gv][n_out], values fp16 [N][D/Gv][n_out].
    """
    v = np.asarray(v)
    n, d = v.shape
    if d % group_ch:
        raise ValueError("Gv must divide D")
    ng = d // group_ch
    codes = np.zeros((n, d), np.int32)
    scales = np.zeros((n, ng), np.float32)
    pos = np.zeros((n, ng, n_out), np.int64)
    val = np.zeros((n, ng, n_out), np.float16)
    for t in range(n):
        for j in range(ng):
            sl = slice(j * group_ch, (j + 1) * group_ch)
            cc, s, p, vv = quantize_vector(v[t, sl], lut, n_out)
            codes[t, sl], scales[t, j], pos[t, j], val[t, j] = cc, s, p, vv
    return codes, scales, pos, val


def dequant_k(codes, scales, pos, val, lut, group_tok):
    """K_hat float64 [N][D] of quantize_k's outputs."""
    n, d = codes.shape
    out = np.zeros((n, d), np.float64)
    for g in range(scales.shape[0]):
        t0, t1 = g * group_tok, min(n, (g + 1) * group_tok)
        for c in range(d):
            out[t0:t1, c] = dequant_vector(codes[t0:t1, c], scales[g, c],
                                           pos[g, c], val[g, c], lut)
    return out


def dequant_v(codes, scales, pos, val, lut, group_ch):
    """V_hat float64 [N][D] of quantize_v's outputs."""
    n, d = codes.shape
    out = np.zeros((n, d), np.float64)
    for t in range(n):
        for j in range(d // group_ch):
            sl = slice(j * group_ch, (j + 1) * group_ch)
            out[t, sl] = dequant_vector(codes[t, sl], scales[t, j], pos[t, j],
                                        val[t, j], lut)
    return out


# ------------------------------------------------------------------ storage

def pack_codes(codes, bits):
    """Unsigned level indices [rows][n] -> uint32 words, LSB-first,
    floor(32/bits) fields per word, one row per token, unused bits zero."""
    c = np.asarray(codes, np.int64)
    if np.any(c < 0) or np.any(c >= (1 << bits)):
        raise ValueError("code out of range")
    per = 32 // bits
    rows, nf = c.shape
    nw = (nf + per - 1) // per
    out = np.zeros((rows, nw), np.uint64)
    for j in range(nf):
        out[:, j // per] |= c[:, j].astype(np.uint64) << np.uint64((j % per) * bits)
    return out.astype(np.uint32)


def pack_outliers(pos, val):
    """One uint32 per outlier slot: the position in bits 16..31, the fp16
    pattern of the value in bits 0..15."""
    p = np.asarray(pos, np.uint64)
    b = np.asarray(val, np.float16).view(np.uint16).astype(np.uint64)
    return ((p << np.uint64(16)) | b).astype(np.uint32)


def to_csr(pos, val, length):
    """The outliers of a stack of vectors ([..., n_out] positions and fp16
    values, `length` entries per vector) as CSR over the flattened vectors:
    (row_ptr, column, value) with the nonzero values only (padding slots and
    outliers whose value is 0 add nothing), columns ascending in each row."""
    p = np.asarray(pos).reshape(-1, np.shape(pos)[-1])
    v = np.asarray(val, np.float16).reshape(-1, np.shape(val)[-1])
    row_ptr, cols, vals = [0], [], []
    for r in range(p.shape[0]):
        entries = sorted((int(c), x) for c, x in zip(p[r], v[r]) if float(x) != 0.0)
        for c, x in entries:
            if c < 0 or c >= length:
                raise ValueError("outlier position outside the vector")
            cols.append(c)
            vals.append(x)
        row_ptr.append(len(cols))
    return (np.array(row_ptr, np.int64), np.array(cols, np.int64),
            np.array(vals, np.float16))


def from_csr(row_ptr, cols, vals, n_out):
    """CSR back to fixed-length rows of n_out slots (positions, fp16
    values): a row's entries in column order, then padding (0, +0)."""
    n_rows = len(row_ptr) - 1
    pos = np.zeros((n_rows, n_out), np.int64)
    val = np.zeros((n_rows, n_out), np.float16)
    for r in range(n_rows):
        k = row_ptr[r + 1] - row_ptr[r]
        if k > n_out:
            raise ValueError("row holds more than n_out entries")
        pos[r, :k] = cols[row_ptr[r]:row_ptr[r + 1]]
        val[r, :k] = vals[row_ptr[r]:row_ptr[r + 1]]
    return pos, val


def csr_to_dense(row_ptr, cols, vals, n_rows, length):
    """Dense float64 [n_rows][length] of a CSR matrix."""
    out = np.zeros((n_rows, length), np.float64)
    for r in range(n_rows):
        for i in range(row_ptr[r], row_ptr[r + 1]):
            out[r, cols[i]] += float(vals[i])
    return out
