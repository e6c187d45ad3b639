"""Pins of the oracle's rotary embedding of pre-RoPE keys (oracle/rope.py).

Each test fixes the oracle against something other than its own formula:
hand-computed frequencies, the polar form of a 2-D rotation, group laws of
rotations (identity, composition, orthogonality), the permutation that
relates the two pair layouts, an explicit block-rotation matrix, and the
relative-position property of attention with rotated queries and keys.
"""
import math

import numpy as np
import pytest

from oracle import attention, rope


def test_frequencies_by_hand():
    # base 10000: D = 4 gives 10000^0, 10000^-1/2; D = 8 adds the quarter powers
    assert np.array_equal(rope.theta(4), [1.0, 0.01])
    np.testing.assert_allclose(rope.theta(8), [1.0, 0.1, 0.01, 0.001], rtol=1e-15)
    np.testing.assert_allclose(rope.theta(2, base=500000.0), [1.0])
    # geometric: theta_f = theta_1 ** f
    t = rope.theta(128)
    np.testing.assert_allclose(t, t[1] ** np.arange(64), rtol=1e-13)
    with pytest.raises(ValueError):
        rope.theta(5)


@pytest.mark.parametrize("p", [0, 1, 3, 1000, 1 << 20])
def test_two_channels_polar_form(p):
    """D = 2 (theta_0 = 1): q . R(p) k = |q| |k| cos(p + phi_k - phi_q)."""
    rng = np.random.default_rng(p)
    q = rng.standard_normal(2)
    k = rng.standard_normal(2)
    rk = rope.rotate(k[None, :], [p])[0]
    want = (math.hypot(*q) * math.hypot(*k) *
            math.cos(p + math.atan2(k[1], k[0]) - math.atan2(q[1], q[0])))
    # the closed form rounds p + phi: allow for that at large p
    assert abs(q @ rk - want) <= 1e-12 * (1 + p) * (1 + abs(want))
    # a quarter turn is reached at no integer position; check the sign on a
    # position whose angle lies in (0, pi): the first channel turns towards
    # the second
    e = rope.rotate(np.array([[1.0, 0.0]]), [1])[0]
    assert e[0] == pytest.approx(math.cos(1.0)) and e[1] == pytest.approx(math.sin(1.0))
    assert e[1] > 0


@pytest.mark.parametrize("pairing", rope.PAIRINGS)
def test_group_laws(pairing):
    rng = np.random.default_rng(7)
    d = 64
    x = rng.standard_normal((5, d))
    # position 0 is the identity
    assert np.array_equal(rope.rotate(x, np.zeros(5)), x)
    # norms are kept (each pair is rotated)
    y = rope.rotate(x, [3, 77, 1000, 65535, 999999], pairing=pairing)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1),
                               rtol=1e-13)
    a, b = rope.pair_channels(d, pairing)
    np.testing.assert_allclose(np.hypot(y[:, a], y[:, b]), np.hypot(x[:, a], x[:, b]),
                               rtol=1e-12)
    # composition: rotating by m then by n equals rotating by m + n
    m = np.array([1, 5, 40, 123, 4000])
    n = np.array([2, 9, 11, 456, 77])
    z = rope.rotate(rope.rotate(x, m, pairing=pairing), n, pairing=pairing)
    np.testing.assert_allclose(z, rope.rotate(x, m + n, pairing=pairing), atol=1e-11)


def test_pairings_differ_by_a_channel_permutation():
    rng = np.random.default_rng(3)
    d = 32
    x = rng.standard_normal((4, d))
    pos = [0, 1, 17, 4095]
    # interleaved channel 2f <- half channel f, 2f + 1 <- f + d/2
    perm = np.empty(d, int)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    half = rope.rotate(x, pos, pairing="half")
    inter = rope.rotate(x[:, perm], pos, pairing="interleaved")
    np.testing.assert_allclose(inter, half[:, perm], rtol=0, atol=0)
    assert not np.allclose(rope.rotate(x, pos, pairing="interleaved"), half)


@pytest.mark.parametrize("pairing", rope.PAIRINGS)
def test_explicit_block_rotation_matrix(pairing):
    """Build R(p) entry by entry as a D x D matrix of 2 x 2 rotation blocks
    and apply it as a matrix-vector product."""
    d, p, base = 8, 13, 100.0
    a, b = rope.pair_channels(d, pairing)
    r = np.zeros((d, d))
    for f in range(d // 2):
        ang = p * base ** (-2.0 * f / d)
        r[a[f], a[f]] = math.cos(ang)
        r[a[f], b[f]] = -math.sin(ang)
        r[b[f], a[f]] = math.sin(ang)
        r[b[f], b[f]] = math.cos(ang)
    assert np.allclose(r @ r.T, np.eye(d), atol=1e-15)
    x = np.arange(1.0, d + 1.0)
    np.testing.assert_allclose(rope.rotate(x[None], [p], base, pairing)[0], r @ x,
                               rtol=1e-14)


@pytest.mark.parametrize("pairing", rope.PAIRINGS)
def test_relative_position_attention(pairing):
    """Scores depend only on the distance between query and key positions:
    rotating the query at position P and every key at its own position
    gives the attention of the query rotated at P - pos_i against the
    unrotated keys, computed here token by token."""
    rng = np.random.default_rng(11)
    hq, hkv, n, d = 4, 2, 9, 16
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    pos0, P = 1000, 1100
    qr = rope.rotate(q, np.full(hq, P), pairing=pairing)
    got = rope.attention(qr, k, v, pos0=pos0, pairing=pairing)
    g = hq // hkv
    for h in range(hq):
        s = np.array([rope.rotate(q[h][None], [P - (pos0 + i)], pairing=pairing)[0]
                      @ k[h // g, i] for i in range(n)]) / math.sqrt(d)
        w = np.exp(s - s.max())
        want = (w @ v[h // g]) / w.sum()
        np.testing.assert_allclose(got[h], want, rtol=1e-10, atol=1e-12)
    # the query and every key rotated by one common shift of positions:
    # plain attention of the unrotated pair (shift-invariance)
    shifted = rope.attention(rope.rotate(q, np.full(hq, P + 555), pairing=pairing),
                             k, v, pos0=pos0 + 555, pairing=pairing)
    np.testing.assert_allclose(shifted, got, atol=1e-11)


def test_pair_layouts_by_hand():
    a, b = rope.pair_channels(8, "half")
    assert list(a) == [0, 1, 2, 3] and list(b) == [4, 5, 6, 7]
    a, b = rope.pair_channels(8, "interleaved")
    assert list(a) == [0, 2, 4, 6] and list(b) == [1, 3, 5, 7]
    with pytest.raises(ValueError):
        rope.pair_channels(8, "neox")
