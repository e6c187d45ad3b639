"""Pins of the dense-and-sparse non-uniform quantizer oracle (CPU only).

Source: "KVQuant: Towards 10 Million Context Length LLM Inference with KV
Cache Quantization": summary and "Approach" (nuqX codebooks, per-vector
dense-and-sparse outlier isolation), table "Measured effects reported in the
paper" (1% outliers; per-vector thresholds beat one per-matrix threshold).
"""
import numpy as np
import pytest

import synth
from oracle import nuq


def brute_nearest(q, levels):
    """Pure Python: the first level at minimal distance (q, levels exact in
    binary64)."""
    best, best_d = 0, abs(float(q) - float(levels[0]))
    for j in range(1, len(levels)):
        d = abs(float(q) - float(levels[j]))
        if d < best_d:
            best, best_d = j, d
    return best


def brute_outliers(x, n_out):
    """Position i is an outlier iff fewer than n_out entries beat it
    (larger magnitude, or equal magnitude at a lower index)."""
    a = [abs(float(v)) for v in x]
    out = []
    for i in range(len(a)):
        beat = sum(1 for j in range(len(a)) if a[j] > a[i] or (a[j] == a[i] and j < i))
        if beat < n_out:
            out.append(i)
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebooks_are_valid_inputs(bits):
    lut = nuq.check_codebook(synth.nuq_codebook(bits), bits)
    assert lut[0] == -1.0 and lut[-1] == 1.0 and 0.0 in lut.tolist()
    gaps = np.diff(lut.astype(np.float64))
    assert gaps.max() / gaps.min() > 1.5          # genuinely non-uniform
    with pytest.raises(ValueError):
        nuq.check_codebook(np.array([-1, -0.5, 0.5, 1], np.float32), 2)  # no 0
    with pytest.raises(ValueError):
        nuq.check_codebook(np.array([-1, 0, 0.1, 1], np.float32), 2)     # not fp16


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_nearest_level_brute_force(bits):
    lut = synth.nuq_codebook(bits)
    rng = np.random.default_rng(bits)
    mids = ((lut[:-1].astype(np.float64) + lut[1:]) / 2).astype(np.float32)
    q = np.concatenate([rng.uniform(-1.2, 1.2, 500).astype(np.float32), lut,
                        mids, np.nextafter(mids, np.float32(2)),
                        np.nextafter(mids, np.float32(-2))])
    got = nuq.nearest_level(q, lut)
    for qi, g in zip(q, got):
        assert g == brute_nearest(qi, lut), qi
    # exact midpoints go to the lower level
    assert np.array_equal(nuq.nearest_level(mids, lut), np.arange(len(mids)))


def test_outlier_selection_brute_force():
    rng = np.random.default_rng(1)
    for n in (1, 2, 5, 17, 128):
        for n_out in (0, 1, 2, 3, 200):
            x = (rng.standard_normal(n) * 3).astype(np.float16)
            if n > 4:
                x[3] = -x[1]        # equal magnitudes: the lower index first
            got = nuq.select_outliers(x, n_out).tolist()
            assert got == brute_outliers(x, n_out)
    # all equal magnitudes: the lowest positions
    x = np.array([2, -2, 2, -2, 2], np.float16)
    assert nuq.select_outliers(x, 2).tolist() == [0, 1]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_vector_on_the_codebook_is_exact(bits):
    """A vector whose dense part lies on scale * levels (scale a power of
    two, the largest level present) reconstructs exactly, with the codes of
    those levels; the outliers come back exactly too."""
    lut = synth.nuq_codebook(bits)
    rng = np.random.default_rng(10 + bits)
    scale = np.float32(2.0 ** -3)
    codes = rng.integers(0, 1 << bits, 40)
    codes[7] = (1 << bits) - 1                      # the level 1.0
    x = (lut[codes] * scale).astype(np.float16)
    x[11] = np.float16(60.0)
    x[30] = np.float16(-45.5)                       # two spikes
    c, s, pos, val = nuq.quantize_vector(x, lut, 2)
    assert s == scale
    assert pos.tolist() == [11, 30] and val.tolist() == [60.0, -45.5]
    zero = int(np.argmin(np.abs(lut)))
    want = codes.copy()
    want[[11, 30]] = zero
    assert np.array_equal(c, want)
    assert np.array_equal(nuq.dequant_vector(c, s, pos, val, lut),
                          x.astype(np.float64))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_reconstruction_bound(bits):
    """Outliers are exact; every other entry is within half the largest
    codebook gap (times the scale) plus the float32 quotient's rounding."""
    lut = synth.nuq_codebook(bits)
    half_gap = float(np.max(np.diff(lut.astype(np.float64)))) / 2
    rng = np.random.default_rng(bits)
    for trial in range(30):
        x = (rng.standard_normal(64) * rng.uniform(0.01, 100)).astype(np.float16)
        x[rng.integers(0, 64)] *= np.float16(20)
        c, s, pos, val = nuq.quantize_vector(x, lut, 2)
        xh = nuq.dequant_vector(c, s, pos, val, lut)
        xf = x.astype(np.float64)
        mask = np.ones(64, bool)
        mask[pos] = False
        assert np.array_equal(xh[~mask], xf[~mask])
        bound = float(s) * (half_gap + 2.0 ** -23)
        assert np.all(np.abs(xh[mask] - xf[mask]) <= bound)
        # the outliers are the largest magnitudes
        assert np.min(np.abs(xf[~mask])) >= np.max(np.abs(xf[mask]))


def test_special_cases():
    lut = synth.nuq_codebook(3)
    zero = int(np.argmin(np.abs(lut)))
    x = (np.arange(10) - 4.5).astype(np.float16)
    # no outliers: the plain non-uniform code
    c, s, pos, val = nuq.quantize_vector(x, lut, 0)
    assert pos.size == 0 and s == np.float32(4.5)
    # every entry an outlier: exact, dense part zero with scale 1
    c, s, pos, val = nuq.quantize_vector(x, lut, 10)
    assert s == 1.0 and np.all(c == zero)
    assert np.array_equal(nuq.dequant_vector(c, s, pos, val, lut), x.astype(np.float64))
    # more slots than entries: padding (position 0, value +0) after them
    c, s, pos, val = nuq.quantize_vector(x[:3], lut, 5)
    assert pos.tolist() == [0, 1, 2, 0, 0]
    assert val.view(np.uint16).tolist()[3:] == [0, 0]
    assert np.array_equal(nuq.dequant_vector(c, s, pos, val, lut),
                          x[:3].astype(np.float64))
    # all zero: scale 1, zero codes
    c, s, pos, val = nuq.quantize_vector(np.zeros(8, np.float16), lut, 1)
    assert s == 1.0 and np.all(c == zero)
    with pytest.raises(ValueError):
        nuq.quantize_vector(np.array([1.0, np.inf], np.float16), lut, 1)


def test_key_and_value_grouping():
    """Keys: one vector per (group of G tokens, channel); values: per
    (token, group of Gv channels); checked against quantize_vector on the
    slices, with a partial last key group."""
    lut = synth.nuq_codebook(4)
    rng = np.random.default_rng(3)
    k = rng.standard_normal((21, 6)).astype(np.float16)
    c, s, p, v = nuq.quantize_k(k, lut, 8, 1)
    assert s.shape == (3, 6) and p.shape == (3, 6, 1)
    for g, (t0, t1) in enumerate(((0, 8), (8, 16), (16, 21))):
        for ch in range(6):
            cc, ss, pp, vv = nuq.quantize_vector(k[t0:t1, ch], lut, 1)
            assert np.array_equal(c[t0:t1, ch], cc) and s[g, ch] == ss
            assert p[g, ch].tolist() == pp.tolist()
    kh = nuq.dequant_k(c, s, p, v, lut, 8)
    assert kh.shape == (21, 6)
    vals = rng.standard_normal((5, 12)).astype(np.float16)
    c, s, p, v = nuq.quantize_v(vals, lut, 4, 1)
    assert s.shape == (5, 3) and p.shape == (5, 3, 1)
    for t in range(5):
        for j in range(3):
            cc, ss, pp, vv = nuq.quantize_vector(vals[t, 4 * j:4 * j + 4], lut, 1)
            assert np.array_equal(c[t, 4 * j:4 * j + 4], cc) and s[t, j] == ss
    vh = nuq.dequant_v(c, s, p, v, lut, 4)
    for t in range(5):
        for j in range(3):
            assert vh[t, 4 * j + p[t, j, 0]] == float(v[t, j, 0])


def test_packing_known_words():
    assert nuq.pack_codes(np.array([[1, 2, 3, 0, 3]]), 2).tolist() == \
        [[1 | (2 << 2) | (3 << 4) | (0 << 6) | (3 << 8)]]
    w = nuq.pack_codes(np.array([[7] * 11]), 3)
    assert w.tolist() == [[(1 << 30) - 1, 7]]            # 10 fields, then 1
    assert nuq.pack_codes(np.arange(16)[None] % 16, 4).tolist() == \
        [[0x76543210, 0xFEDCBA98]]
    assert nuq.pack_outliers(np.array([5]), np.array([1.0], np.float16)).tolist() == \
        [0x00053C00]
    assert nuq.pack_outliers(np.array([127]), np.array([-2.0], np.float16)).tolist() == \
        [0x007FC000]


def test_csr_round_trip():
    lut = synth.nuq_codebook(3)
    rng = np.random.default_rng(4)
    v = rng.standard_normal((30, 16)).astype(np.float16)
    v[3, :4] = 0                                     # a zero-valued outlier
    v[3, 4:] = 0
    c, s, p, val = nuq.quantize_v(v, lut, 16, 2)
    rp, cols, vals = nuq.to_csr(p, val, 16)
    assert rp.shape == (31,) and rp[-1] == cols.size
    assert np.all(np.diff(rp) <= 2) and rp[4] - rp[3] == 0
    dense = nuq.csr_to_dense(rp, cols, vals, 30, 16)
    for t in range(30):
        want = np.zeros(16)
        for pp, vv in zip(p[t, 0], val[t, 0]):
            want[pp] += float(vv)
        assert np.array_equal(dense[t], want)
    p2, v2 = nuq.from_csr(rp, cols, vals, 2)
    rp2, cols2, vals2 = nuq.to_csr(p2, v2, 16)
    assert np.array_equal(rp, rp2) and np.array_equal(cols, cols2) and \
        np.array_equal(vals.view(np.uint16), vals2.view(np.uint16))
    for t in range(30):
        if float(val[t, 0, 0]) != 0 and float(val[t, 0, 1]) != 0:
            assert p2[t].tolist() == p[t, 0].tolist()


def _matrix_threshold(x, n_total, lut):
    """One threshold for the whole matrix: the n_total largest magnitudes
    of x (rows are vectors) are kept exactly, each row's rest quantized."""
    flat = np.abs(x.astype(np.float64)).ravel()
    order = sorted(range(flat.size), key=lambda i: (-flat[i], i))[:n_total]
    keep = np.zeros(flat.size, bool)
    keep[order] = True
    keep = keep.reshape(x.shape)
    out = np.zeros(x.shape, np.float64)
    for r in range(x.shape[0]):
        dense = np.where(keep[r], np.float16(0), x[r]).astype(np.float16)
        c, s, p, v = nuq.quantize_vector(dense, lut, 0)
        out[r] = nuq.dequant_vector(c, s, p, v, lut)
        out[r][keep[r]] = x[r][keep[r]]
    return out


def test_per_vector_outliers_beat_none_and_per_matrix():
    """The page's ablations, on seeded vectors of very different overall
    magnitudes, each with one spike of ten times its own size: removing 1%
    outliers per vector lowers the reconstruction error (mean over vectors
    of the relative L2 error), and a per-vector threshold beats one
    threshold for the whole matrix with the same outlier count (which spends
    its outliers on the large vectors and leaves the spikes of the small
    ones in their dense part)."""
    lut = synth.nuq_codebook(3)
    errs = {"none": [], "vector": [], "matrix": []}
    for seed in (7, 19, 41):
        rng = np.random.default_rng(seed)
        x = rng.standard_normal((64, 128)).astype(np.float32)
        x *= (10.0 ** rng.uniform(0, 2, 64)).astype(np.float32)[:, None]
        spikes = rng.integers(0, 128, 64)
        x[np.arange(64), spikes] *= np.float32(10)
        x = x.astype(np.float16)
        ref = x.astype(np.float64)

        def row_err(rec):
            return float(np.mean(np.linalg.norm(rec - ref, axis=1) /
                                 np.linalg.norm(ref, axis=1)))
        for name, n_out in (("none", 0), ("vector", 1)):
            rec = np.stack([nuq.dequant_vector(*nuq.quantize_vector(x[r], lut, n_out), lut)
                            for r in range(64)])
            errs[name].append(row_err(rec))
        errs["matrix"].append(row_err(_matrix_threshold(x, 64, lut)))
    m = {k: float(np.mean(v)) for k, v in errs.items()}
    assert m["vector"] < 0.6 * m["none"], m
    assert m["vector"] < 0.8 * m["matrix"], m
