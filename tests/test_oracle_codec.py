"""Pins of the oracle codec against the pages and the mathematics (CPU only).

Rule under test: "KV quantization axes ...", section "What rows and columns
mean" (symmetric absmax rule and the three groupings) and the page's closing
troubleshooting paragraph (scale shapes, zero group, NaN/Inf rejected).
"""
import math
import os
import struct

import numpy as np
import pytest
import torch

from oracle import codec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    """Round a Python float (binary64) to binary32."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def scalar_rule(values, bits):
    """Brute force in pure Python, independent of NumPy.

    Division in binary64 followed by rounding to binary32 equals the
    correctly rounded binary32 quotient (53 >= 2*24+2, so the double
    rounding is innocuous); Python's round() is round-half-to-even.
    """
    qmax = 2 ** (bits - 1) - 1
    m = max(abs(float(v)) for v in values) if len(values) else 0.0
    scale = f32(f32(m) / qmax)
    if m == 0.0 or scale == 0.0:
        scale = 1.0
    codes = []
    for v in values:
        q = f32(float(v) / scale)
        codes.append(max(-qmax, min(qmax, round(q))))
    return codes, scale


@pytest.mark.parametrize("bits", [8, 4, 3, 2])
def test_brute_force_tiny_groupings(bits):
    rng = np.random.default_rng(bits)
    for n in range(1, 7):
        for d in range(1, 5):
            x = (rng.standard_normal((n, d)) * rng.uniform(0.01, 50)).astype(
                np.float32)
            for g in range(1, n + 1):
                codes, scales = codec.quantize_k(x, bits, g)
                for gi in range(scales.shape[0]):
                    for c in range(d):
                        col = x[gi * g:(gi + 1) * g, c]
                        ref_c, ref_s = scalar_rule(col.tolist(), bits)
                        assert scales[gi, c] == np.float32(ref_s)
                        assert codes[gi * g:(gi + 1) * g, c].tolist() == ref_c
            for gv in [v for v in range(1, d + 1) if d % v == 0]:
                codes, scales = codec.quantize_v(x, bits, gv)
                assert scales.shape == (n, d // gv)
                for t in range(n):
                    for j in range(d // gv):
                        row = x[t, j * gv:(j + 1) * gv]
                        ref_c, ref_s = scalar_rule(row.tolist(), bits)
                        assert scales[t, j] == np.float32(ref_s)
                        assert codes[t, j * gv:(j + 1) * gv].tolist() == ref_c


def test_scale_shapes_match_page():
    """Token scales are (N,1), channel scales (1,D), tensor one scale."""
    x = np.random.default_rng(0).standard_normal((7, 5)).astype(np.float32)
    assert codec.quantize_matrix(x, 8, "token")[1].shape == (7, 1)
    assert codec.quantize_matrix(x, 8, "channel")[1].shape == (1, 5)
    assert codec.quantize_matrix(x, 8, "tensor")[1].shape == (1, 1)
    # per-channel with G = N is the page's channel grouping
    c1, s1 = codec.quantize_matrix(x, 8, "channel")
    c2, s2 = codec.quantize_k(x, 8, 7)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    c3, s3 = codec.quantize_matrix(x, 8, "token")
    c4, s4 = codec.quantize_v(x, 8, 5)
    assert np.array_equal(c3, c4) and np.array_equal(s3, s4)


@pytest.mark.parametrize("bits", [8, 4, 3, 2])
def test_invariants(bits):
    qmax = codec.qmax_for_bits(bits)
    rng = np.random.default_rng(100 + bits)
    x = (rng.standard_normal((3000, 64)) *
         np.exp(rng.uniform(-8, 8, (3000, 1)))).astype(np.float32)
    codes, scales = codec.quantize_groups(x, bits)
    assert codes.min() >= -qmax and codes.max() <= qmax
    # every nonzero group reaches +-qmax exactly
    assert np.all(np.max(np.abs(codes), axis=1) == qmax)
    q = (x / scales[:, None]).astype(np.float32).astype(np.float64)
    # |fl32(x/scale) - code| <= 1/2 exactly (no clipping can be active
    # beyond rounding, since |x| <= m)
    assert np.all(np.abs(q - codes) <= 0.5)
    # reconstruction error: scale * (1/2 + qmax * 2**-23)
    err = np.abs(x.astype(np.float64) - codes * scales[:, None].astype(
        np.float64))
    bound = scales[:, None].astype(np.float64) * (0.5 + qmax * 2.0 ** -23)
    assert np.all(err <= bound)


@pytest.mark.parametrize("bits", [8, 4, 3, 2])
def test_exact_multiples_and_ties(bits):
    qmax = codec.qmax_for_bits(bits)
    s = 0.5  # scale = (qmax * 0.5) / qmax = 0.5 exactly
    ks = np.arange(-qmax, qmax + 1)
    x = (ks * s).astype(np.float32)
    codes, scale = codec.quantize_group(x, bits)
    assert scale == np.float32(0.5)
    assert codes.tolist() == ks.tolist()
    # ties k + 1/2 go to the even neighbour
    ties = np.array([qmax * s] + [(k + 0.5) * s for k in range(-qmax, qmax)],
                    np.float32)
    codes, scale = codec.quantize_group(ties, bits)
    want = [qmax] + [int(2 * round((k + 0.5) / 2)) for k in range(-qmax, qmax)]
    assert codes.tolist() == want
    for k, c in zip(range(-qmax, qmax), codes[1:]):
        assert c % 2 == 0 and abs(c - (k + 0.5)) == 0.5


def test_zero_group_and_nonfinite():
    codes, scale = codec.quantize_group(np.zeros(16, np.float32), 4)
    assert scale == 1.0 and np.all(codes == 0)
    codes, scale = codec.quantize_group(np.zeros(16, np.float16), 2)
    assert scale == 1.0 and np.all(codes == 0)
    for bad in (np.nan, np.inf, -np.inf):
        x = np.ones(8, np.float32)
        x[3] = bad
        with pytest.raises(codec.NonFiniteInput):
            codec.quantize_group(x, 8)
    # underflowing scale (m tiny): treated as a zero group
    tiny = np.array([1e-45, -1e-45, 0.0], np.float32)
    codes, scale = codec.quantize_group(tiny, 8)
    assert scale == 1.0 and np.all(codes == 0)


def test_f16_and_f32_inputs_agree():
    rng = np.random.default_rng(3)
    x16 = rng.standard_normal((40, 16)).astype(np.float16)
    for bits in (8, 4, 3, 2):
        a = codec.quantize_k(x16, bits, 8)
        b = codec.quantize_k(x16.astype(np.float32), bits, 8)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_adversarial_division_fixture():
    """Stored groups where reciprocal or float64 shortcuts change a code."""
    d = np.load(os.path.join(GOLDEN, "adversarial_groups.npz"))
    n_recip = n_f64 = 0
    for i in range(len(d["bits"])):
        bits, gl = int(d["bits"][i]), int(d["group_len"][i])
        x = d["x"][i, :gl]
        codes, scale = codec.quantize_group(x, bits)
        assert np.array_equal(codes, d["codes"][i, :gl].astype(np.int32))
        assert scale == d["scales"][i]
        qmax = codec.qmax_for_bits(bits)
        r = np.float32(1.0) / scale
        c_recip = np.clip(np.rint((x * r).astype(np.float32)), -qmax, qmax)
        c_f64 = np.clip(np.rint(x.astype(np.float64) / np.float64(scale)),
                        -qmax, qmax)
        n_recip += int(np.any(c_recip != codes))
        n_f64 += int(np.any(c_f64 != codes))
        assert np.any(c_recip != codes) or np.any(c_f64 != codes)
    assert n_recip > 0 and n_f64 > 0


@pytest.mark.parametrize("bits", [8, 4, 3, 2])
def test_packing_layout(bits):
    qmax = codec.qmax_for_bits(bits)
    pw = 32 // bits
    # hand-built row: field j holds code (j % (2*qmax+1)) - qmax
    nf = 3 * pw + 1
    codes = np.array([[(j % (2 * qmax + 1)) - qmax for j in range(nf)]])
    words = codec.pack_rows(codes, bits)
    assert words.shape == (1, 4)
    for j in range(nf):
        u = (int(words[0, j // pw]) >> ((j % pw) * bits)) & ((1 << bits) - 1)
        assert u == codes[0, j] + (1 << (bits - 1))
    # unused high bits and unused trailing fields are zero
    if 32 % bits:
        assert all((int(w) >> (pw * bits)) == 0 for w in words[0])
    assert (int(words[0, 3]) >> bits) == 0
    assert np.array_equal(codec.unpack_rows(words, bits, nf), codes)
    # a known word: int4 codes -7..0 -> u 1..8, nibble j at bits 4j
    if bits == 4:
        w = codec.pack_rows(np.array([[-7, -6, -5, -4, -3, -2, -1, 0]]), 4)
        assert int(w[0, 0]) == 0x87654321


def test_dequant_exact():
    rng = np.random.default_rng(5)
    codes = rng.integers(-127, 128, (50, 8))
    scales = rng.standard_normal((50, 8)).astype(np.float32)
    out = codec.dequant(codes, scales)
    for i in range(50):
        for j in range(8):
            # code (7 bits) * scale (24 bits) fits binary64 exactly
            assert out[i, j] == float(int(codes[i, j])) * float(scales[i, j])
    f = codec.dequant_f32(codes, scales)
    assert np.array_equal(f, (out.astype(np.float32)))


def test_bf16_rounding_matches_torch():
    """RNE float32 -> bfloat16 against torch's conversion (library routine)."""
    pats = [0x3F800000, 0x3F808000, 0x3F818000, 0x3F80FFFF, 0x3F7FFFFF,
            0x00000001, 0x80000001, 0x007FFFFF, 0x7F7F7FFF, 0xC0490FDB,
            0x3F8080000 & 0xFFFFFFFF, 0x477FE000, 0x33800000]
    rng = np.random.default_rng(11)
    x = np.concatenate([np.array(pats, np.uint32).view(np.float32),
                        rng.standard_normal(20000).astype(np.float32) * 50,
                        rng.standard_normal(2000).astype(np.float16).astype(
                            np.float32)])
    mine = codec.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(mine, ref.view(np.uint16))
    back = codec.bf16_bits_to_f32(mine)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).to(
        torch.float32).numpy())


def test_qmax_values():
    assert [codec.qmax_for_bits(b) for b in (8, 4, 3, 2)] == [127, 7, 3, 1]
    with pytest.raises(ValueError):
        codec.qmax_for_bits(5)
    assert math.isclose(codec.words_per_row(128, 3), 13)
