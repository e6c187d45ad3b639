"""Oracle of the value-side 1-bit residual sketch (the KQV scheme).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Source: "Statistical Inference and Quality Measures of KV Cache
Quantisations Inspired by TurboQuant" (gist.science), Technical Summary:
"Quantization Schemes" (KQV: a Walsh-Hadamard transform on keys and
values; keys scalar-quantized with n bits; values with n - 1 bits plus a
1-bit QJL sketch of the residual), "1. Theoretical Proof of QJL Harm on
Keys" (the sketch is an unbiased estimator of the residual's inner
products, variance (pi/2) ||r||^2 / d) and "2. The K-V Asymmetry and Optimal
Scheme (KQV)" (values enter attention through a linear weighted sum, so the
unbiased sketch corrects their bias; it is never applied to keys).

Readings where the page leaves a step open:

* the scalar part is this build's symmetric absmax rule (oracle.codec) per
  token, in groups of Gv channels, with n - 1 bits;
* the sketch of a residual r (the rotated value minus its scalar
  reconstruction, both float32) is b_i = sign(<S_i, r>) (+1 at 0) for the m
  rows S_i of a Gaussian matrix S (an input, drawn once), stored with
  gamma = ||r||_2;
* the estimator of <y, r> is sqrt(pi/2) / m * gamma * <S y, b>, and the
  value the decode uses is x_hat + r_hat with
  r_hat = sqrt(pi/2) / m * gamma * S^T b, the estimator's linear form; its
  expectation over S is r (E[<s, y> sign(<s, r>)] = sqrt(2/pi) <y, r>/||r||
  for s ~ N(0, I));
* values are rotated by the normalized Walsh-Hadamard transform (its own
  inverse, oracle.rotation) before quantization, so the attention output is
  rotated back once at the end.
"""

import math

import numpy as np

from . import codec, rotation

C_QJL = math.sqrt(math.pi / 2.0)


def sketch(r, S):
    """Signs of S r (rows of r), +1 at exact zero; dot products in float64.
    r: [..., d] float32, S: [m][d] float32 -> int8 [..., m] of +-1."""
    dots = np.asarray(r, np.float64) @ np.asarray(S, np.float64).T
    return np.where(dots >= 0.0, 1, -1).astype(np.int8)


def estimate_inner(y, bits, gamma, S):
    """sqrt(pi/2)/m * gamma * <S y, b>: the estimate of <y, r>."""
    S = np.asarray(S, np.float64)
    m = S.shape[0]
    return C_QJL / m * float(gamma) * float((S @ np.asarray(y, np.float64)) @
                                            np.asarray(bits, np.float64))


def reconstruct(bits, gamma, S):
    """r_hat = sqrt(pi/2)/m * gamma * S^T b (rows of bits), float64."""
    S = np.asarray(S, np.float64)
    m = S.shape[0]
    b = np.asarray(bits, np.float64)
    return C_QJL / m * np.asarray(gamma, np.float64)[..., None] * (b @ S)


def quantize_v(v_rot, bits, group_ch, S):
    """Rotated values [N][D] (float32 or float16) -> scalar codes [N][D]
    (n - 1 = `bits` bits, symmetric absmax per (token, Gv channels)),
    scales [N][D/Gv], sketch bits int8 [N][m] and residual norms float32 [N].
    The residual is fl32(v - fl32(code * scale)) (exact: the two are within
    half a scale of each other, or the code is 0)."""
    v = np.asarray(v_rot).astype(np.float32)
    codes, scales = codec.quantize_v(v, bits, group_ch)
    xhat = codec.dequant_f32(codes, codec.expand_v_scales(scales, v.shape[1],
                                                          group_ch))
    r = (v - xhat).astype(np.float32)
    b = sketch(r, S)
    gamma = np.sqrt(np.sum(r.astype(np.float64) ** 2, axis=1)).astype(np.float32)
    return codes, scales, b, gamma, r


def dequant_v(codes, scales, b, gamma, S, group_ch):
    """V_hat (rotated domain) float64 [N][D] = x_hat + r_hat."""
    d = codes.shape[1]
    xhat = codec.dequant(codes, codec.expand_v_scales(scales, d, group_ch))
    return xhat + reconstruct(b, gamma, S)


def pack_signs(b):
    """Sketch bits [N][m] (+-1) -> uint32 [N][m/32]: bit i of word w is 1
    where b[32 w + i] = +1."""
    b = np.asarray(b)
    n, m = b.shape
    out = np.zeros((n, (m + 31) // 32), np.uint64)
    for i in range(m):
        out[:, i // 32] |= (b[:, i] > 0).astype(np.uint64) << np.uint64(i % 32)
    return out.astype(np.uint32)


def unrotate(out_rot):
    """Rows of an attention output computed on rotated values, turned back
    (float64 transform: H / sqrt(d) is its own inverse)."""
    x = np.asarray(out_rot, np.float64)
    d = x.shape[-1]
    H = rotation.sylvester(d).astype(np.float64) / math.sqrt(d)
    return x @ H
