"""Pins of the oracle key rotation (CPU only).

Reading under test ("Quantize What Counts: More for Keys, Less for Values",
rotation integration; "Statistical Inference and Quality Measures of KV
Cache Quantisations Inspired by TurboQuant", the KQV scheme): the
normalized Sylvester Walsh-Hadamard transform, computed in float32 by the
fast transform with stages h = 1, 2, 4, ...
"""
import struct

import numpy as np
import pytest

from oracle import codec, rotation


def f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def test_sylvester_is_hadamard():
    for d in (1, 2, 4, 8, 32, 128):
        h = rotation.sylvester(d)
        assert set(np.unique(h)) <= {-1, 1}
        assert np.array_equal(h @ h.T, d * np.eye(d, dtype=np.int64))
    # the order-4 matrix written out
    assert np.array_equal(rotation.sylvester(4), np.array(
        [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]]))
    with pytest.raises(ValueError):
        rotation.sylvester(12)


@pytest.mark.parametrize("d", [2, 8, 64, 128, 256])
def test_fast_transform_equals_matrix_on_exact_inputs(d):
    """Small integers keep every butterfly sum exact in float32, so the
    result is float32(1/sqrt(d)) times the exact product H x, rounded once
    (the matrix built from its recursive definition, in int64)."""
    rng = np.random.default_rng(d)
    x = rng.integers(-1000, 1001, size=(5, d))
    y = rotation.wht(x.astype(np.float32))
    hx = x @ rotation.sylvester(d).T
    c = f32(1.0 / np.sqrt(d))
    want = np.array([[f32(c * float(v)) for v in row] for row in hx],
                    dtype=np.float32)
    assert np.array_equal(y, want)


def test_rotation_is_orthonormal_and_involutive():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((7, 128)).astype(np.float32)
    k = rng.standard_normal((7, 128)).astype(np.float32)
    rq, rk = rotation.wht(q), rotation.wht(k)
    # dot products and norms are kept (float32 rounding only)
    np.testing.assert_allclose((rq.astype(np.float64) * rk).sum(1),
                               (q.astype(np.float64) * k).sum(1),
                               rtol=0, atol=1e-4)
    np.testing.assert_allclose(np.linalg.norm(rq, axis=1),
                               np.linalg.norm(q, axis=1), rtol=1e-5)
    # R R x = x
    np.testing.assert_allclose(rotation.wht(rq), q, rtol=0, atol=1e-5)


def test_one_outlier_spreads_evenly():
    """A single large channel becomes d equal magnitudes: the rotation's
    use against key outliers."""
    x = np.zeros(128, np.float32)
    x[17] = 64.0
    y = rotation.wht(x)
    assert np.all(np.abs(y) == np.float32(64.0) * rotation.scale32(128))
    # its sign pattern is row 17 of the Hadamard matrix
    assert np.array_equal(np.sign(y), rotation.sylvester(128)[:, 17])


def test_rotation_lowers_int4_key_error():
    """Per-channel int4 keys (one group of 128 tokens) where each token has
    one large channel, a different one per token: every channel's absmax is
    set by some outlier.  Rotating spreads each token's outlier over all
    channels at 1/sqrt(d) of its size, and the score error q.k halves (the
    K4 setting of the rotation-integration result)."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal(128).astype(np.float32)

    def score_err(keys, query):
        codes, scales = codec.quantize_matrix(keys, 4, "channel")
        kh = codes.astype(np.float64) * scales.astype(np.float64)
        return np.abs(kh @ query - keys.astype(np.float64) @ query).mean()

    for _ in range(3):
        k = rng.standard_normal((128, 128)).astype(np.float32)
        k[np.arange(128), rng.integers(0, 128, size=128)] *= 30.0
        assert score_err(rotation.wht(k), rotation.wht(q)) < 0.7 * score_err(k, q)


def test_float16_output_is_round_to_nearest_even():
    x = np.arange(128, dtype=np.float32) * np.float32(0.37)
    y32 = rotation.wht(x)
    y16 = rotation.wht(x, np.float16)
    assert np.array_equal(y16, y32.astype(np.float16))
    with pytest.raises(TypeError):
        rotation.wht(x, np.float64)
