"""Pins of the oracle attention (closed forms, textbook routine, brute force).

Definition under test: "KV quantization axes ...", section "Separate the two
error paths" -- softmax(Q K^T / sqrt(D)) V with a stable float64 softmax.
"""
import math

import numpy as np
import torch

from oracle import attention


def test_rows_sum_to_one():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((6, 16))
    k = rng.standard_normal((3, 40, 16)) * 3
    w = attention.softmax_weights(q, k)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-12, rtol=0)
    assert np.all(w >= 0)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 8))
    k = rng.standard_normal((2, 1, 8))
    v = rng.standard_normal((2, 1, 8))
    out = attention.attention(q, k, v)
    for h in range(4):
        assert np.array_equal(out[h], v[h // 2, 0])


def test_zero_query_is_mean_of_values():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, 33, 8))
    v = rng.standard_normal((1, 33, 8))
    out = attention.attention(np.zeros((2, 8)), k, v)
    assert np.allclose(out, v[0].mean(axis=0), atol=1e-14, rtol=0)


def test_matches_torch_sdpa():
    """Against torch's scaled_dot_product_attention (float64, CPU)."""
    rng = np.random.default_rng(4)
    hq, hkv, n, d = 8, 2, 57, 32
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((hkv, n, d)) * 2
    v = rng.standard_normal((hkv, n, d))
    out = attention.attention(q, k, v)
    g = hq // hkv
    kt = torch.from_numpy(np.repeat(k, g, axis=0))
    vt = torch.from_numpy(np.repeat(v, g, axis=0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], kt, vt)[:, 0, :].numpy()
    assert np.allclose(out, ref, atol=1e-12, rtol=1e-12)


def test_brute_force_loops():
    rng = np.random.default_rng(5)
    hq, hkv, n, d = 4, 2, 5, 3
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    out = attention.attention(q, k, v)
    for h in range(hq):
        kv = h // (hq // hkv)
        s = [sum(q[h, c] * k[kv, t, c] for c in range(d)) / math.sqrt(d)
             for t in range(n)]
        e = [math.exp(x) for x in s]   # small scores: no shift needed
        z = sum(e)
        for c in range(d):
            ref = sum(e[t] * v[kv, t, c] for t in range(n)) / z
            assert abs(out[h, c] - ref) < 1e-13


def test_stable_for_large_scores():
    q = np.array([[1000.0, 0.0]])
    k = np.array([[[1.0, 0.0], [0.999, 0.0]]])
    v = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    out = attention.attention(q, k, v, sm_scale=1.0)
    # p = softmax([1000, 999]) -> weights 1/(1+e^-1), e^-1/(1+e^-1)
    a = 1.0 / (1.0 + math.exp(-1.0))
    assert np.allclose(out[0], [a, 1 - a], atol=1e-12)


def test_error_metrics():
    ref = np.array([[3.0, 4.0], [1.0, 0.0]])
    out = np.array([[3.0, 4.5], [1.0, 0.1]])
    assert math.isclose(attention.max_row_relative_error(out, ref), 0.1)
    assert math.isclose(attention.relative_error(out, ref),
                        math.sqrt(0.25 + 0.01) / math.sqrt(26.0))
