"""Pins of the value-side 1-bit residual sketch oracle (CPU only).

Source: "Statistical Inference and Quality Measures of KV Cache
Quantisations Inspired by TurboQuant", Technical Summary: "Quantization
Schemes" (KQV), "1. Theoretical Proof of QJL Harm on Keys" (unbiased
estimator, variance (pi/2) ||r||^2 / d) and "2. The K-V Asymmetry and
Optimal Scheme (KQV)".
"""
import math

import numpy as np
import pytest

import synth
from oracle import attention, codec, qjl, rotation


def test_unbiased_with_the_pages_variance():
    """Over many independent Gaussian sketches of one residual r, the
    estimate of <y, r> averages to <y, r>, and its variance is
    ((pi/2) ||r||^2 ||y||^2 - <y, r>^2) / m; for a unit y orthogonal to r and
    m = d that is the page's (pi/2) ||r||^2 / d."""
    d = m = 64
    rng = np.random.default_rng(0)
    r = rng.standard_normal(d)
    y_par = rng.standard_normal(d)
    y_orth = y_par - (y_par @ r) / (r @ r) * r
    y_orth /= np.linalg.norm(y_orth)
    n = 4000
    for y in (y_par, y_orth):
        est = []
        for i in range(n):
            S = np.random.default_rng(1000 + i).standard_normal((m, d))
            b = qjl.sketch(r[None], S)[0]
            est.append(qjl.estimate_inner(y, b, np.linalg.norm(r), S))
        est = np.array(est)
        truth = float(y @ r)
        var = ((math.pi / 2) * (r @ r) * (y @ y) - truth ** 2) / m
        se = math.sqrt(var / n)
        assert abs(est.mean() - truth) < 4 * se, (est.mean(), truth, se)
        # sample variance within 10% (its own relative spread is ~2.2%)
        assert abs(est.var() / var - 1) < 0.1, (est.var(), var)
    var_orth = (math.pi / 2) * (r @ r) / d
    assert abs(((math.pi / 2) * (r @ r) * (y_orth @ y_orth) - (y_orth @ r) ** 2) / m
               - var_orth) < 1e-9


def test_sign_and_reconstruction_forms():
    d = 8
    r = np.array([1.5, -2.0, 0.0, 3.0, -0.25, 0.5, -1.0, 2.0], np.float32)
    # S = identity: the sketch is the sign pattern of r (+1 at 0)
    b = qjl.sketch(r[None], np.eye(d, dtype=np.float32))[0]
    assert b.tolist() == [1, -1, 1, 1, -1, 1, -1, 1]
    # the reconstruction is the estimator's linear form
    S = synth.jl_matrix(3, 16, d)
    b = qjl.sketch(r[None], S)
    g = np.float32(np.linalg.norm(r))
    rh = qjl.reconstruct(b, np.array([g]), S)[0]
    y = np.random.default_rng(2).standard_normal(d)
    assert math.isclose(float(y @ rh), qjl.estimate_inner(y, b[0], g, S),
                        rel_tol=1e-12)
    assert math.isclose(qjl.C_QJL, math.sqrt(math.pi / 2))


def test_packing_known_words():
    b = np.ones((1, 64), np.int8)
    b[0, 1] = b[0, 5] = -1
    b[0, 40] = -1
    w = qjl.pack_signs(b)
    assert w.tolist() == [[0xFFFFFFFF ^ 0x22, 0xFFFFFFFF ^ (1 << 8)]]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_residual_is_exact(bits):
    """x_hat + r reproduces the rotated value exactly (the float32
    subtraction is exact), and gamma is ||r|| rounded to float32."""
    rng = np.random.default_rng(bits)
    v = rng.standard_normal((40, 64)).astype(np.float16)
    vr = rotation.wht(v)
    S = synth.jl_matrix(1, 64, 64)
    codes, scales, b, gamma, r = qjl.quantize_v(vr, bits, 32, S)
    xhat = codec.dequant_f32(codes, codec.expand_v_scales(scales, 64, 32))
    assert np.array_equal(xhat.astype(np.float64) + r.astype(np.float64),
                          vr.astype(np.float64))
    assert np.array_equal(gamma, np.linalg.norm(r.astype(np.float64), axis=1)
                          .astype(np.float32))
    assert np.all(np.abs(r) <= np.repeat(scales, 32, axis=1) * (0.5 + 2.0 ** -20))
    assert set(np.unique(b).tolist()) <= {-1, 1}


def test_kqv_values_remove_the_scalar_bias():
    """The sketch's value reconstruction is unbiased, so over independent
    sketch matrices the attention output with values quantized to n - 1 = 2
    bits plus the sketch averages to the output of the exact rotated values,
    while the 2-bit scalar part alone keeps its deterministic error (the
    residual it drops).  (A single sketch adds variance: per token
    E||r_hat - r||^2 = (pi/2) ||r||^2 for m = d, which is the price the page
    says values can afford and keys cannot.)  The rotation back is exact."""
    d, n, hq, draws = 64, 512, 2, 200
    rng = np.random.default_rng(7)
    q = rng.standard_normal((hq, d)) / 4
    k = rng.standard_normal((1, n, d))
    v = rng.standard_normal((n, d)).astype(np.float16)
    vr = rotation.wht(v)
    ref = attention.attention(q, k, v.astype(np.float64)[None])
    mean_q = np.zeros_like(ref)
    for i in range(draws):
        S = synth.jl_matrix(100 + i, d, d)
        codes, scales, b, gamma, r = qjl.quantize_v(vr, 2, 32, S)
        vh_q = qjl.dequant_v(codes, scales, b, gamma, S, 32)
        mean_q += qjl.unrotate(attention.attention(q, k, vh_q[None])) / draws
    vh_s = codec.dequant(codes, codec.expand_v_scales(scales, d, 32))
    out_s = qjl.unrotate(attention.attention(q, k, vh_s[None]))
    e_mean = attention.relative_error(mean_q, ref)
    e_s = attention.relative_error(out_s, ref)
    assert e_mean < 0.25 * e_s, (e_mean, e_s)
    # unrotating the exact rotated values gives the values back
    assert np.allclose(qjl.unrotate(vr.astype(np.float64)),
                       v.astype(np.float64), atol=1e-6)
