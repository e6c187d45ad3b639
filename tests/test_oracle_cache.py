"""Pins of the oracle cache and salience (invariants, brute force, special cases).

Cache: "MixKVQ ...", Figure 4 (full-precision buffer of R recent tokens in
front of per-channel keys and per-token values); "KVQuant ...", summary and
"Measured effects" table (fp16 first token).  Salience: "MixKVQ ...",
Figure 3 (A = I * S; BF16 / INT4 / INT2 key channels).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import attention, cache, codec, salience


def simulate_counts(n_tokens, S, R, G):
    """Token-by-token counter simulation of flush-on-overflow."""
    sink = quant = tail = 0
    for _ in range(n_tokens):
        if sink < S:
            sink += 1
            continue
        if tail == R:
            quant += G
            tail -= G
        tail += 1
    return sink, quant, tail


@pytest.mark.parametrize("S,R,G", [(0, 128, 128), (1, 64, 64), (1, 128, 32),
                                   (3, 96, 32), (0, 4, 2)])
def test_tail_closed_form(S, R, G):
    for n in list(range(0, 3 * R + 5)) + [4096, 131072, 1048576]:
        if n > 5000:
            # closed form only (simulation would be slow)
            npast = max(0, n - S)
            t = cache.tail_length(npast, R, G)
            assert 0 < t <= R and (npast - t) % G == 0
            continue
        s, q, t = simulate_counts(n, S, R, G)
        assert t == cache.tail_length(max(0, n - S), R, G)
        assert s + q + t == n


def test_workload_token_split():
    """Counts used by the workloads (sink, quantized, tail)."""
    want = {"7b_layer_4k": (0, 3968, 128), "gqa_128k": (1, 131008, 63),
            "mixkvq_32k": (0, 32640, 128), "1m_32layer": (1, 1048448, 127)}
    for name, (s, q, t) in want.items():
        w = synth.WORKLOADS[name]
        npast = w["N"] - w["S"]
        tl = cache.tail_length(npast, w["R"], w["G"])
        assert (min(w["S"], w["N"]), npast - tl, tl) == (s, q, t)


def make_cfg(**kw):
    base = dict(B=2, Hkv=2, D=32, S=1, R=16, G=8, Gv=16, k_bits=4, v_bits=2)
    base.update(kw)
    return cache.CacheConfig(**base)


def _equal_exports(a, b):
    assert a.keys() == b.keys()
    for key in a:
        assert a[key].dtype == b[key].dtype, key
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("mixed", [False, True])
def test_append_order_independent(mixed):
    cfg = make_cfg(mixed=mixed, n_bf16=3, n_int4=9, k_bits=2)
    q, k, v = synth.kv_inputs(3, 2, 4, 2, 77, 32)
    one = cache.Cache(cfg)
    for t in range(77):
        one.append(k[:, :, t:t + 1], v[:, :, t:t + 1])
    chunks = cache.Cache(cfg)
    for a, b in ((0, 5), (5, 6), (6, 40), (40, 77)):
        chunks.append(k[:, :, a:b], v[:, :, a:b])
    whole = cache.Cache(cfg)
    whole.append(k, v)
    _equal_exports(one.export(), chunks.export())
    _equal_exports(one.export(), whole.export())
    assert one.counts() == (1, 64, 12)


def test_groups_equal_stateless_quantizers():
    cfg = make_cfg(S=2)
    q, k, v = synth.kv_inputs(4, 2, 2, 2, 61, 32)
    c = cache.Cache(cfg)
    c.append(k, v)
    ns, nq, nt = c.counts()
    ex = c.export()
    for b in range(2):
        for h in range(2):
            assert np.array_equal(ex["sink_k"][b, h], k[b, h, :ns])
            assert np.array_equal(ex["tail_v"][b, h], v[b, h, ns + nq:])
            kc, ks = codec.quantize_k(k[b, h, ns:ns + nq], 4, 8)
            assert np.array_equal(ex["k_codes"][b, h], codec.pack_rows(kc, 4))
            assert np.array_equal(ex["k_scales"][b, h], ks)
            vc, vs = codec.quantize_v(v[b, h, ns:ns + nq], 2, 16)
            assert np.array_equal(ex["v_codes"][b, h], codec.pack_rows(vc, 2))
            assert np.array_equal(ex["v_scales"][b, h], vs)


def test_tail_only_cache_is_textbook_attention():
    cfg = make_cfg(S=1, R=64, G=32)
    q, k, v = synth.kv_inputs(5, 1, 4, 2, 50, 32)
    c = cache.Cache(make_cfg(B=1, S=1, R=64, G=32))
    c.append(k, v)
    assert c.counts() == (1, 0, 49)
    kh = np.stack([c.dequantized(0, h)[0] for h in range(2)])
    vh = np.stack([c.dequantized(0, h)[1] for h in range(2)])
    out = attention.attention(q[0].astype(np.float64), kh, vh)
    kt = torch.from_numpy(np.repeat(k[0].astype(np.float64), 2, axis=0))
    vt = torch.from_numpy(np.repeat(v[0].astype(np.float64), 2, axis=0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[0].astype(np.float64))[:, None, :], kt, vt)
    assert np.allclose(out, ref[:, 0].numpy(), atol=1e-12, rtol=1e-12)
    assert cfg.R == 64


def test_rejects_nonfinite_and_bad_config():
    c = cache.Cache(make_cfg())
    k = np.ones((2, 2, 3, 32), np.float16)
    k[1, 1, 2, 5] = np.inf
    with pytest.raises(codec.NonFiniteInput):
        c.append(k, np.ones_like(k))
    with pytest.raises(ValueError):
        make_cfg(R=12, G=8).check()
    with pytest.raises(ValueError):
        make_cfg(Gv=5).check()


# ---------------------------------------------------------------- salience

def test_intensity_is_exact_sum():
    qw = synth.query_window(9, 1, 64, 10, 16)[0]
    I = salience.intensity(qw, 2)
    for kvh in range(2):
        for d in range(16):
            exact = sum(Fraction(abs(float(qw[r, h, d])))
                        for r in range(64) for h in range(kvh * 5, kvh * 5 + 5))
            assert Fraction(I[kvh, d]) == exact


def test_class_counts_and_ties():
    rng = np.random.default_rng(0)
    I = rng.uniform(0, 10, 128)
    S = rng.uniform(0, 10, 128).astype(np.float32)
    cls = salience.classes(I, S, 8, 32)
    assert (np.sum(cls == 0), np.sum(cls == 1), np.sum(cls == 2)) == \
        (8, 32, 88)
    # all ties: lowest channels win
    cls = salience.classes(np.ones(128), np.ones(128, np.float32), 8, 32)
    assert np.all(cls[:8] == 0) and np.all(cls[8:40] == 1) and \
        np.all(cls[40:] == 2)


def test_query_awareness_special_case():
    """A channel with huge key scale but no query mass is not kept in BF16;
    a channel with moderate key scale and large query mass is."""
    D = 16
    I = np.full(D, 1.0)
    S = np.full(D, 1.0, np.float32)
    S[3] = 1000.0
    I[3] = 1e-6          # large S, tiny I -> A = 1e-3
    I[7] = 50.0
    S[7] = 2.0           # moderate S, large I -> A = 100
    cls = salience.classes(I, S, 1, 2)
    assert cls[7] == salience.CLASS_BF16
    assert cls[3] == salience.CLASS_INT2
    # ranking by S alone (I = 1) would have picked channel 3
    cls_s = salience.classes(np.ones(D), S, 1, 2)
    assert cls_s[3] == salience.CLASS_BF16


def test_mixed_group_contents():
    cfg = make_cfg(B=1, Hkv=1, S=0, R=8, G=8, mixed=True, n_bf16=4,
                   n_int4=8, k_bits=2)
    q, k, v = synth.kv_inputs(6, 1, 1, 1, 9, 32, n_out=3)
    c = cache.Cache(cfg)
    qw = synth.query_window(6, 1, 64, 1, 32)
    c.salience_select(qw)
    c.append(k, v)
    grp = c.streams[0][0].groups[0]
    kg = k[0, 0, :8]
    S = salience.group_key_scale(kg)
    A = c.I[0, 0] * S.astype(np.float64)
    top = sorted(range(32), key=lambda d: (-A[d], d))
    assert grp["ch_bf16"] == sorted(top[:4])
    assert grp["ch_int4"] == sorted(top[4:12])
    # bf16 channels round-trip through torch's bfloat16
    ref = torch.from_numpy(kg[:, grp["ch_bf16"]].astype(np.float32)).to(
        torch.bfloat16).to(torch.float32).numpy()
    kh, _ = c.dequantized(0, 0)
    assert np.array_equal(kh[:8][:, grp["ch_bf16"]], ref.astype(np.float64))
    # int channels: error within scale * (1/2 + qmax 2^-23)
    for name, bits in (("int4", 4), ("int2", 2)):
        ch = grp["ch_" + name]
        sc = grp[name + "_scales"].astype(np.float64)
        err = np.abs(kh[:8][:, ch] - kg[:, ch].astype(np.float64))
        qm = codec.qmax_for_bits(bits)
        assert np.all(err <= sc * (0.5 + qm * 2.0 ** -23))
    assert math.isclose(len(grp["ch_int2"]), 20)
