"""Pins of the oracle parts every attention parity test rests on (CPU only).

The dequantized cache (oracle.cache.Cache.dequantized) produces K_hat and
V_hat for every attention comparison, so it is checked here element by
element against a scalar loop written from the definitions alone, reading
the exported words bit by bit: "KV quantization axes: why Key and Value
need separate reasoning", section "What rows and columns mean" (x_hat =
code * scale, keys per channel, values per token); "MixKVQ: Query-Aware
Mixed-Precision KV Cache Quantization for Long-Context Reasoning",
Figure 3 (BF16 / INT4 / INT2 key channels) and Figure 4 (full-precision
tail); "KVQuant ...", summary (fp16 first token).  The byte model is pinned
to the counts the "KV quantization axes ..." page prints in "Scales occupy
bytes too" and to hand counts of the packed layout.
"""
import os
import struct
import sys

import numpy as np
import pytest

import synth
from oracle import bytes_model, cache, codec, salience

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def f16_value(bits16):
    """An fp16 pattern as a Python float (struct's 'e' format)."""
    return struct.unpack("<e", struct.pack("<H", int(bits16)))[0]


def bf16_value(bits16):
    """A bfloat16 pattern widened to binary32 (the top half of the word)."""
    return struct.unpack("<f", struct.pack("<I", int(bits16) << 16))[0]


def field(words, j, bits):
    """Signed code of field j of a packed row: offset binary, LSB-first,
    floor(32/bits) fields per little-endian 32-bit word."""
    per = 32 // bits
    w = int(words[j // per]) & 0xFFFFFFFF
    u = (w >> ((j % per) * bits)) & ((1 << bits) - 1)
    return u - (1 << (bits - 1))


def scalar_dequant(ex, cfg, b, h, k_in, v_in):
    """K_hat, V_hat of stream (b, h) as nested Python lists, token order
    sink, quantized groups, tail; fp16 rows taken from the inputs."""
    ns = ex["sink_k"].shape[2]
    nq = ex["v_codes"].shape[2]
    nt = ex["tail_k"].shape[2]
    D = cfg.D
    K, V = [], []
    for t in range(ns + nq + nt):
        if t < ns or t >= ns + nq:
            K.append([f16_value(np.float16(k_in[b, h, t, d]).view(np.uint16))
                      for d in range(D)])
            V.append([f16_value(np.float16(v_in[b, h, t, d]).view(np.uint16))
                      for d in range(D)])
            continue
        i = t - ns                      # quantized token index
        grp = i // cfg.G
        row_k = []
        if cfg.mixed:
            cls = ex["k_class"][b, h, grp]
            order = {0: [], 1: [], 2: []}
            for d in range(D):
                order[int(cls[d])].append(d)
            n4 = len(order[1])
            for d in range(D):
                c = int(cls[d])
                j = order[c].index(d)
                if c == 0:
                    row_k.append(bf16_value(ex["k_bf16"][b, h, i, j]))
                elif c == 1:
                    row_k.append(field(ex["k_int4"][b, h, i], j, 4) *
                                 float(ex["k_scales"][b, h, grp, j]))
                else:
                    row_k.append(field(ex["k_int2"][b, h, i], j, 2) *
                                 float(ex["k_scales"][b, h, grp, n4 + j]))
        else:
            for d in range(D):
                row_k.append(field(ex["k_codes"][b, h, i], d, cfg.k_bits) *
                             float(ex["k_scales"][b, h, grp, d]))
        K.append(row_k)
        V.append([field(ex["v_codes"][b, h, i], d, cfg.v_bits) *
                  float(ex["v_scales"][b, h, i, d // cfg.Gv])
                  for d in range(D)])
    return K, V


CASES = {
    # S = 2 sink tokens, three uniform key groups, a ragged tail
    "uniform_k4v2": dict(B=1, Hkv=2, D=16, S=2, R=8, G=8, Gv=4, k_bits=4,
                         v_bits=2, n=2 + 3 * 8 + 5),
    "uniform_k3v8": dict(B=2, Hkv=1, D=12, S=2, R=6, G=6, Gv=3, k_bits=3,
                         v_bits=8, n=2 + 3 * 6 + 4),
    "mixed": dict(B=1, Hkv=2, D=16, S=2, R=8, G=8, Gv=8, k_bits=2, v_bits=4,
                  mixed=True, n_bf16=2, n_int4=5, n=2 + 3 * 8 + 3),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_dequantized_equals_scalar_loop(name):
    kw = dict(CASES[name])
    n = kw.pop("n")
    cfg = cache.CacheConfig(**kw)
    q, k, v = synth.kv_inputs(31, cfg.B, cfg.Hkv, cfg.Hkv, n, cfg.D, n_out=2)
    c = cache.Cache(cfg)
    if cfg.mixed:
        c.salience_select(synth.query_window(31, cfg.B, 4, cfg.Hkv, cfg.D))
    c.append(k, v)
    ns, nq, nt = c.counts()
    assert (ns, nq // cfg.G) == (2, 3) and 0 < nt < cfg.G
    ex = c.export()
    for b in range(cfg.B):
        for h in range(cfg.Hkv):
            kh, vh = c.dequantized(b, h)
            K, V = scalar_dequant(ex, cfg, b, h, k, v)
            assert kh.shape == (n, cfg.D) and vh.shape == (n, cfg.D)
            assert kh.tolist() == K, "K_hat differs from the scalar loop"
            assert vh.tolist() == V, "V_hat differs from the scalar loop"
            # the rule's reconstruction bound holds on every quantized value
            qv = v[b, h, ns:ns + nq].astype(np.float64)
            vs = np.repeat(ex["v_scales"][b, h].astype(np.float64), cfg.Gv,
                           axis=1)
            qmax = codec.qmax_for_bits(cfg.v_bits)
            assert np.all(np.abs(vh[ns:ns + nq] - qv) <=
                          vs * (0.5 + qmax * 2.0 ** -23))


def test_expand_scales_index_tables():
    """Token t takes key-scale row t // G; channel c takes value-scale
    column c // Gv (hand-written tables for N = 7, G = 3 and D = 8,
    Gv = 2)."""
    ks = np.array([[10.0, 11.0], [20.0, 21.0], [30.0, 31.0]], np.float32)
    got = codec.expand_k_scales(ks, 7, 3)
    rows = [0, 0, 0, 1, 1, 1, 2]
    assert got.tolist() == [ks[r].tolist() for r in rows]
    vs = np.array([[1.0, 2.0, 3.0, 4.0], [5.0, 6.0, 7.0, 8.0]], np.float32)
    got = codec.expand_v_scales(vs, 8, 2)
    assert got.tolist() == [[1, 1, 2, 2, 3, 3, 4, 4], [5, 5, 6, 6, 7, 7, 8, 8]]
    # ragged: N = 5 with G = 4 -> rows 0,0,0,0,1; D = 6, Gv = 3 -> 0,0,0,1,1,1
    assert codec.expand_k_scales(ks[:2], 5, 4).tolist() == \
        [ks[0].tolist()] * 4 + [ks[1].tolist()]
    assert codec.expand_v_scales(vs[:, :2], 6, 3).tolist() == \
        [[1, 1, 1, 2, 2, 2], [5, 5, 5, 6, 6, 6]]


def test_group_key_scale_takes_magnitudes():
    """S_d is the largest |K[t, d]| of the group, also where the channel's
    values are all negative or its largest value is not its largest
    magnitude."""
    kg = np.array([[-3.0, 1.0, -0.25, 0.0],
                   [2.0, -0.5, -0.75, -0.0],
                   [-1.0, 0.75, -0.5, 0.0]], np.float16)
    S = salience.group_key_scale(kg)
    assert S.dtype == np.float32
    assert S.tolist() == [3.0, 1.0, 0.75, 0.0]
    # fp16 extremes widen exactly
    kg = np.array([[-65504.0, 2.0 ** -24], [1.0, -2.0 ** -24]], np.float16)
    assert salience.group_key_scale(kg).tolist() == [65504.0, 2.0 ** -24]


def test_cache_stream_bytes_page_counts():
    """int8 keys per channel (G = N) and values per token (Gv = D) at
    D = 32: the page's 4,480 B (N = 64) and 17,536 B (N = 256), which is
    2ND + 4D + 4N."""
    for n, want in ((64, 4480), (256, 17536)):
        got = bytes_model.cache_stream_bytes(0, n, 0, 32, 8, 8, n, 32)
        assert got == want == 2 * n * 32 + 4 * 32 + 4 * n


def test_cache_stream_bytes_hand_counts():
    # 4096-token 7B-style layer, one stream: 3,968 quantized tokens of
    # 16-word int4 key rows and 8-word int2 value rows, 31 key-scale rows of
    # 128 floats, 4 value scales per token, a 128-token fp16 tail of K and V
    assert bytes_model.cache_stream_bytes(0, 3968, 128, 128, 4, 2, 128, 32) \
        == 3968 * 64 + 31 * 128 * 4 + 3968 * 32 + 3968 * 4 * 4 + \
        128 * 128 * 2 * 2
    # 1M tokens, one stream: sink 1 + 1,048,448 quantized + tail 127
    assert bytes_model.cache_stream_bytes(1, 1048448, 127, 128, 2, 2, 128,
                                          32) == \
        1048448 * 32 + 8191 * 512 + 1048448 * 32 + 1048448 * 16 + 128 * 512
    # mixed keys, one stream of the 32K MixKVQ case: 8 bf16 channels
    # (16 B), 32 int4 (4 words), 88 int2 (6 words: 176 bits padded to 192),
    # per group 120 scales and a 128-byte class map; int2 values in 8 words,
    # 2 scales per token; 128 tail rows
    assert bytes_model.cache_stream_bytes(0, 32640, 128, 128, 0, 2, 128, 64,
                                          mixed=True, n_bf16=8,
                                          n_int4=32) == \
        32640 * (16 + 16 + 24) + 255 * (120 * 4 + 128) + 32640 * 32 + \
        32640 * 8 + 128 * 512
    # 3-bit rows: 10 fields per word, 13 words for 128 channels
    assert bytes_model.cache_stream_bytes(0, 64, 0, 128, 3, 3, 64, 128) == \
        64 * 52 + 128 * 4 + 64 * 52 + 64 * 4


def test_bench_byte_model_is_the_oracle_one():
    """bench.py counts the bytes of a decode call on its own (it may not
    import the oracle outside its CPU baseline); both counts agree."""
    sys.path.insert(0, ROOT)
    import bench

    class View:
        pass

    for kw in (dict(head_dim=128, n_quant=3968, n_sink=0, n_tail=128,
                    group_tok=128, group_ch=32, k_mixed=0, k_bits=4, v_bits=2,
                    batch=1, kv_heads=32, n_bf16=0, n_int4=0),
               dict(head_dim=128, n_quant=32640, n_sink=0, n_tail=128,
                    group_tok=128, group_ch=64, k_mixed=1, k_bits=0, v_bits=2,
                    batch=8, kv_heads=8, n_bf16=8, n_int4=32),
               dict(head_dim=128, n_quant=131008, n_sink=1, n_tail=63,
                    group_tok=64, group_ch=64, k_mixed=0, k_bits=2, v_bits=4,
                    batch=1, kv_heads=8, n_bf16=0, n_int4=0)):
        v = View()
        v.__dict__.update(kw)
        hq = 32
        per = bytes_model.cache_stream_bytes(
            v.n_sink, v.n_quant, v.n_tail, v.head_dim, v.k_bits, v.v_bits,
            v.group_tok, v.group_ch, mixed=bool(v.k_mixed), n_bf16=v.n_bf16,
            n_int4=v.n_int4)
        want = v.batch * v.kv_heads * per + v.batch * hq * v.head_dim * 2
        assert bench.stream_bytes(v, hq) == want
