"""GPU tests of the boundary: checkpoint re-attach, bytes around every output
buffer left untouched, and the binding's shape checks.

Re-attach: "KV quantization axes: why Key and Value need separate
reasoning", section "Reproduce" (the archived codes and scales are the whole
state and can be restored for audit); a cache buffer copied and bound again
with kvq_cache_init(n_tokens > 0) must behave exactly like the original.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import attention, cache as ocache, codec
from quantized_decode_attention_02_amd import kvq

pytestmark = pytest.mark.gpu
DEV = "cuda"
PAD = 4096          # canary bytes on each side of an output
CANARY = 0xA5


def say(*a):
    print(*a, flush=True)


def padded(nbytes, dtype, shape):
    """A device tensor of `shape` inside a byte buffer with PAD canary
    bytes before and after it; returns (flat bytes, tensor view)."""
    flat = torch.full((nbytes + 2 * PAD,), CANARY, dtype=torch.uint8, device=DEV)
    t = flat[PAD:PAD + nbytes].view(dtype).view(shape)
    return flat, t


def canaries_intact(flat, nbytes):
    h = flat.cpu().numpy()
    return bool(np.all(h[:PAD] == CANARY) and np.all(h[PAD + nbytes:] == CANARY))


def build(B=1, Hq=8, Hkv=2, N=1500, S=1, G=64, Gv=64, R=64, kb=4, vb=2,
          mixed=False, seed=7):
    q, k, v = synth.kv_inputs(seed, B, Hq, Hkv, N, 128, outliers="fraction",
                              frac=0.02, sink_factor=20.0)
    mk = dict(mixed=True, n_bf16=8, n_int4=32) if mixed else {}
    c = kvq.Cache(B, Hkv, 128, N + 256, kb, vb, G, Gv, R, S=S, **mk)
    if mixed:
        c.kvq_salience_select(torch.from_numpy(
            synth.query_window(seed, B, 64, Hq, 128)).to(DEV))
    c.kvq_append(torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV))
    return q, k, v, c


@pytest.mark.parametrize("mixed", [False, True])
def test_reattach_copied_buffer(mixed):
    say("re-attach", mixed)
    q, k, v, c = build(mixed=mixed, G=128 if mixed else 64,
                       R=128 if mixed else 64)
    n = c.n_tokens
    buf2 = c.buf.clone()
    mk = dict(mixed=True, n_bf16=8, n_int4=32) if mixed else {}
    cfg = c.cfg
    c2 = kvq.Cache(cfg.batch, cfg.kv_heads, cfg.head_dim, cfg.max_tokens,
                   cfg.k_bits, cfg.v_bits, cfg.group_tok, cfg.group_ch,
                   cfg.residual, S=cfg.sink, buf=buf2, n_tokens=n, **mk)
    assert c2.n_tokens == n
    v1, v2 = c.kvq_cache_view(), c2.kvq_cache_view()
    assert (v1.n_sink, v1.n_quant, v1.n_tail) == (v2.n_sink, v2.n_quant, v2.n_tail)
    qt = torch.from_numpy(q).to(DEV)
    for flags in (kvq.KVQ_DECODE_AUTO, kvq.KVQ_DECODE_GENERIC):
        a = kvq.kvq_decode_attention(v1, qt, flags=flags)
        b = kvq.kvq_decode_attention(v2, qt, flags=flags)
        assert torch.equal(a, b)
    # both keep going identically: more tokens, a flush included
    rng = np.random.default_rng(3)
    kn = rng.standard_normal((1, 2, 200, 128)).astype(np.float16)
    vn = rng.standard_normal((1, 2, 200, 128)).astype(np.float16)
    for cc in (c, c2):
        cc.kvq_append(torch.from_numpy(kn).to(DEV), torch.from_numpy(vn).to(DEV))
        assert cc.kvq_cache_check() == kvq.KVQ_OK
    e1 = kvq.kvq_export(c.kvq_cache_view())
    e2 = kvq.kvq_export(c2.kvq_cache_view())
    for key in e1:
        assert torch.equal(e1[key], e2[key]), key
    a = kvq.kvq_decode_attention(c.kvq_cache_view(), qt)
    b = kvq.kvq_decode_attention(c2.kvq_cache_view(), qt)
    assert torch.equal(a, b)


def test_reattach_rejects_more_tokens_than_capacity():
    q, k, v, c = build()
    cfg = c.cfg
    with pytest.raises(kvq.KvqError) as e:
        kvq.Cache(cfg.batch, cfg.kv_heads, cfg.head_dim, cfg.max_tokens,
                  cfg.k_bits, cfg.v_bits, cfg.group_tok, cfg.group_ch,
                  cfg.residual, S=cfg.sink, buf=c.buf.clone(),
                  n_tokens=cfg.max_tokens + 1)
    assert e.value.status == kvq.KVQ_E_ARG


@pytest.mark.parametrize("mixed", [False, True])
def test_decode_writes_only_its_outputs(mixed):
    """Output rows and the workspace's used prefix are the only bytes a
    decode call writes (both kernels, the rotary form too)."""
    say("canary decode", mixed)
    q, k, v, c = build(mixed=mixed, G=128 if mixed else 64,
                       R=128 if mixed else 64)
    view = c.kvq_cache_view()
    B, Hq, D = q.shape
    qt = torch.from_numpy(q).to(DEV)
    ref = kvq.kvq_decode_attention(view, qt, flags=kvq.KVQ_DECODE_GENERIC)
    ob = B * Hq * D * 4
    for call in ("plain", "rope"):
        for flags in (kvq.KVQ_DECODE_AUTO, kvq.KVQ_DECODE_GENERIC):
            for splits in (0, 5):
                ws_bytes = kvq.kvq_decode_workspace_bytes(view, Hq, splits)
                fo, out = padded(ob, torch.float32, (B, Hq, D))
                fw, ws = padded(ws_bytes, torch.uint8, (ws_bytes,))
                if call == "plain":
                    kvq.kvq_decode_attention(view, qt, n_splits=splits,
                                             flags=flags, workspace=ws, out=out)
                else:
                    kvq.kvq_decode_attention_rope(view, qt, n_splits=splits,
                                                  flags=flags, workspace=ws,
                                                  out=out)
                torch.cuda.synchronize()
                assert canaries_intact(fo, ob), (call, flags, splits)
                assert canaries_intact(fw, ws_bytes), (call, flags, splits)
                assert torch.isfinite(out).all()
                if call == "plain":
                    err = attention.max_row_relative_error(
                        out.cpu().numpy(), ref.cpu().numpy().astype(np.float64))
                    assert err <= 2e-3


def test_quantizers_and_dequant_write_only_their_outputs():
    L = kvq.lib()
    rng = np.random.default_rng(5)
    n_mats, n_tok, d = 3, 75, 96
    x = torch.from_numpy(rng.standard_normal((n_mats, n_tok, d)).astype(
        np.float16)).to(DEV)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for bits in (8, 4, 3, 2):
        w = kvq.kvq_words(d, bits)
        for axis, group in ((kvq.KVQ_PER_CHANNEL, 16), (kvq.KVQ_PER_TOKEN, 32)):
            ns = (n_tok + group - 1) // group * d if axis == kvq.KVQ_PER_CHANNEL \
                else n_tok * (d // group)
            cb, sb = n_mats * n_tok * w * 4, n_mats * ns * 4
            fc, codes = padded(cb, torch.int32, (n_mats, n_tok, w))
            fs, scales = padded(sb, torch.float32, (n_mats, ns))
            fn = L.kvq_quantize_k if axis == kvq.KVQ_PER_CHANNEL else L.kvq_quantize_v
            st = fn(ctypes.c_void_p(x.data_ptr()), kvq.KVQ_F16, n_mats, n_tok, d,
                    bits, group, ctypes.c_void_p(codes.data_ptr()),
                    ctypes.c_void_p(scales.data_ptr()), None, s)
            assert st == kvq.KVQ_OK
            ob = n_mats * n_tok * d * 4
            fo, out = padded(ob, torch.float32, (n_mats, n_tok, d))
            st = L.kvq_dequant(ctypes.c_void_p(codes.data_ptr()),
                               ctypes.c_void_p(scales.data_ptr()), n_mats, n_tok,
                               d, bits, axis, group, ctypes.c_void_p(out.data_ptr()), s)
            assert st == kvq.KVQ_OK
            torch.cuda.synchronize()
            for f, nb in ((fc, cb), (fs, sb), (fo, ob)):
                assert canaries_intact(f, nb), (bits, axis)
            # and the values are the oracle's
            xm = x[1].cpu().numpy()
            if axis == kvq.KVQ_PER_CHANNEL:
                rc, rs = codec.quantize_k(xm, bits, group)
            else:
                rc, rs = codec.quantize_v(xm, bits, group)
            assert np.array_equal(codes[1].cpu().numpy().view(np.uint32),
                                  codec.pack_rows(rc, bits))
            assert np.array_equal(scales[1].cpu().numpy(), rs.reshape(-1))


def test_append_stays_inside_the_cache_buffer():
    """kvq_append and kvq_salience_select write nothing past
    kvq_cache_bytes (the buffer is handed over with canaries behind it)."""
    cfg = dict(B=2, Hkv=2, D=128, G=128, Gv=64, R=128, S=1)
    for mixed in (False, True):
        mk = dict(mixed=True, n_bf16=8, n_int4=32) if mixed else {}
        probe = kvq.Cache(2, 2, 128, 900, 2, 2, 128, 64, 128, S=1, **mk)
        nb = probe.buf.numel()
        flat = torch.full((nb + PAD,), CANARY, dtype=torch.uint8, device=DEV)
        c = kvq.Cache(2, 2, 128, 900, 2, 2, 128, 64, 128, S=1,
                      buf=flat[:nb], **mk)
        if mixed:
            c.kvq_salience_select(torch.from_numpy(
                synth.query_window(1, 2, 64, 10, 128)).to(DEV))
        q, k, v = synth.kv_inputs(1, 2, 10, 2, 900, 128)
        for a, b in ((0, 1), (1, 300), (300, 301), (301, 900)):
            c.kvq_append(torch.from_numpy(np.ascontiguousarray(k[:, :, a:b])).to(DEV),
                         torch.from_numpy(np.ascontiguousarray(v[:, :, a:b])).to(DEV))
        assert c.kvq_cache_check() == kvq.KVQ_OK
        assert np.all(flat[nb:].cpu().numpy() == CANARY), mixed
        assert cfg["D"] == 128


def test_binding_checks_shapes():
    q, k, v, c = build()
    view = c.kvq_cache_view()
    qt = torch.from_numpy(q).to(DEV)
    bad = [
        lambda: kvq.kvq_decode_attention(view, qt[:, :, :64].contiguous()),
        lambda: kvq.kvq_decode_attention(view, torch.cat([qt, qt])),
        lambda: kvq.kvq_decode_attention(view, qt, out=torch.empty(
            (1, 8, 64), dtype=torch.float32, device=DEV)),
        lambda: kvq.kvq_decode_attention(view, qt, out=torch.empty(
            (1, 8, 128), dtype=torch.float16, device=DEV)),
        lambda: kvq.kvq_decode_attention(view, qt, workspace=torch.empty(
            16, dtype=torch.uint8, device=DEV)),
        lambda: kvq.kvq_decode_attention_rope(view, qt[0]),
        lambda: c.kvq_append(torch.zeros((1, 2, 3, 64), dtype=torch.float16,
                                         device=DEV),
                             torch.zeros((1, 2, 3, 64), dtype=torch.float16,
                                         device=DEV)),
        lambda: c.kvq_append(torch.zeros((1, 2, 3, 128), dtype=torch.float16,
                                         device=DEV),
                             torch.zeros((1, 2, 4, 128), dtype=torch.float16,
                                         device=DEV)),
        lambda: c.kvq_append(torch.zeros((2, 2, 3, 128), dtype=torch.float16,
                                         device=DEV),
                             torch.zeros((2, 2, 3, 128), dtype=torch.float16,
                                         device=DEV)),
    ]
    n0 = c.n_tokens
    for i, f in enumerate(bad):
        with pytest.raises(kvq.KvqError) as e:
            f()
        assert e.value.status == kvq.KVQ_E_ARG, i
    assert c.n_tokens == n0
    # the cache is untouched and still decodes like the oracle
    oc = ocache.Cache(ocache.CacheConfig(B=1, Hkv=2, D=128, S=1, R=64, G=64,
                                         Gv=64, k_bits=4, v_bits=2))
    oc.append(k, v)
    kh = np.stack([oc.dequantized(0, h)[0] for h in range(2)])
    vh = np.stack([oc.dequantized(0, h)[1] for h in range(2)])
    ref = attention.attention(q[0].astype(np.float64), kh, vh)
    out = kvq.kvq_decode_attention(view, qt)[0].cpu().numpy()
    assert attention.max_row_relative_error(out, ref) <= 2e-3
