"""The no-allocation decode entry point (kvq_decode_attention_noalloc)
against kvq_decode_attention on the same views: two calls in a row, the
second on a smaller cache, and a request beyond the fixed scratch."""
import numpy as np
import pytest
import torch

import synth
from oracle import attention, cache as ocache
from quantized_decode_attention_02_amd import kvq

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def make(B, Hq, Hkv, N, G, Gv, kb, vb, S, seed, mixed=False):
    q, k, v = synth.kv_inputs(seed, B, Hq, Hkv, N, 128, outliers="fraction",
                              frac=0.02, sink_factor=20.0)
    mk = dict(mixed=True, n_bf16=8, n_int4=32) if mixed else {}
    c = kvq.Cache(B, Hkv, 128, N + 8, kb, vb, G, Gv, G, S=S, **mk)
    if mixed:
        c.kvq_salience_select(torch.from_numpy(
            synth.query_window(seed, B, 64, Hq, 128)).to(DEV))
    c.kvq_append(torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV))
    assert c.kvq_cache_check() == kvq.KVQ_OK
    oc = ocache.Cache(ocache.CacheConfig(B=B, Hkv=Hkv, D=128, S=S, R=G, G=G,
                                         Gv=Gv, k_bits=kb, v_bits=vb, **mk))
    if mixed:
        oc.salience_select(synth.query_window(seed, B, 64, Hq, 128))
    oc.append(k, v)
    return q, c, oc


def oracle_out(q, oc, Hkv):
    outs = []
    for b in range(q.shape[0]):
        kh = np.stack([oc.dequantized(b, h)[0] for h in range(Hkv)])
        vh = np.stack([oc.dequantized(b, h)[1] for h in range(Hkv)])
        outs.append(attention.attention(q[b].astype(np.float64), kh, vh))
    return np.stack(outs)


# (B, Hq, Hkv, N, G, Gv, k_bits, v_bits, S, mixed): the first call of each
# pair on the larger cache, the second on a smaller one
PAIRS = [
    ((1, 32, 8, 20000, 64, 64, 4, 2, 1, False),
     (1, 8, 2, 700, 64, 64, 4, 2, 1, False)),
    ((2, 10, 2, 4000, 128, 64, 2, 2, 0, True),
     (1, 5, 1, 300, 128, 64, 2, 2, 0, True)),
    ((1, 4, 4, 9000, 128, 32, 2, 2, 1, False),
     (1, 2, 2, 130, 128, 32, 2, 4, 1, False)),
]


@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_matches_workspace_entry(pair):
    for i, cfg in enumerate(PAIRS[pair]):
        B, Hq, Hkv, N, G, Gv, kb, vb, S, mixed = cfg
        say("noalloc", pair, i, cfg)
        q, c, oc = make(B, Hq, Hkv, N, G, Gv, kb, vb, S, 11 + i, mixed)
        view = c.kvq_cache_view()
        qt = torch.from_numpy(q).to(DEV)
        ref = oracle_out(q, oc, Hkv)
        for flags in (kvq.KVQ_DECODE_AUTO, kvq.KVQ_DECODE_GENERIC):
            for splits in (0, 3):
                a = kvq.kvq_decode_attention(view, qt, n_splits=splits, flags=flags)
                out = torch.full_like(a, float("nan"))
                kvq.kvq_decode_attention_noalloc(view, qt, out, n_splits=splits,
                                                 flags=flags)
                torch.cuda.synchronize()
                assert torch.equal(out, a), (flags, splits)
                err = attention.max_row_relative_error(out.cpu().numpy(), ref)
                assert err <= 2e-3, err


def test_noalloc_rejects_requests_beyond_its_scratch():
    q, c, oc = make(1, 32, 8, 2000, 64, 64, 4, 2, 1, 5)
    view = c.kvq_cache_view()
    qt = torch.from_numpy(q).to(DEV)
    out = torch.zeros((1, 32, 128), dtype=torch.float32, device=DEV)
    # 32 heads x 16384 partials x 130 floats > 16 MiB
    need = kvq.kvq_decode_workspace_bytes(view, 32, 16384)
    assert need > kvq.NOALLOC_SCRATCH_BYTES
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attention_noalloc(view, qt, out, n_splits=16384)
    assert e.value.status == kvq.KVQ_E_SCRATCH
    assert torch.count_nonzero(out).item() == 0
    # the largest split count that fits still runs, and agrees
    a = kvq.kvq_decode_attention(view, qt, n_splits=900)
    kvq.kvq_decode_attention_noalloc(view, qt, out, n_splits=900)
    assert torch.equal(out, a)
