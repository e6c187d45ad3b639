"""The C-ABI library loads, exports every symbol include/kvq.h declares, and
rejects bad arguments on the host before touching the GPU (CPU only)."""
import ctypes
import os
import re

import pytest

from quantized_decode_attention_02_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = kvq.lib()
    names = declared_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(L, n), n
    assert sorted(kvq.EXPORTED) == names


def test_words_and_strerror():
    assert kvq.kvq_words(128, 4) == 16
    assert kvq.kvq_words(128, 2) == 8
    assert kvq.kvq_words(128, 3) == 13
    assert kvq.kvq_words(32, 8) == 8
    assert kvq.kvq_words(5, 7) == -1
    assert kvq.strerror(kvq.KVQ_E_NONFINITE) == "NaN/Inf input rejected"


def _cfg(**kw):
    base = dict(batch=1, kv_heads=32, head_dim=128, k_bits=4, v_bits=2,
                group_tok=128, group_ch=32, residual=128, sink=0, k_mixed=0,
                n_bf16=0, n_int4=0, max_tokens=4096)
    base.update(kw)
    return kvq.CacheCfg(**base)


def test_cache_bytes_covers_the_payload():
    L = kvq.lib()
    c = _cfg()
    nbytes = L.kvq_cache_bytes(ctypes.byref(c))
    # payload of a full cache: 3968 quantized tokens + 128 tail per head
    payload = 32 * (3968 * (64 + 32 + 16) + 31 * 128 * 4 + 128 * 512)
    assert payload <= nbytes <= payload * 1.1


@pytest.mark.parametrize("bad", [dict(k_bits=5), dict(residual=100),
                                 dict(group_ch=48), dict(head_dim=300),
                                 dict(k_mixed=1, n_bf16=100, n_int4=40),
                                 dict(batch=0)])
def test_cache_bytes_rejects_bad_config(bad):
    c = _cfg(**bad)
    assert kvq.lib().kvq_cache_bytes(ctypes.byref(c)) == 0


def test_host_argument_errors_enqueue_nothing():
    L = kvq.lib()
    p = ctypes.c_void_p(256)
    # bad bit width / group / dtype: rejected before any HIP call
    assert L.kvq_quantize_k(p, 1, 1, 4, 8, 5, 2, p, p, None, None) == \
        kvq.KVQ_E_ARG
    assert L.kvq_quantize_v(p, 1, 1, 4, 8, 4, 3, p, p, None, None) == \
        kvq.KVQ_E_ARG
    assert L.kvq_quantize_k(p, 7, 1, 4, 8, 4, 2, p, p, None, None) == \
        kvq.KVQ_E_ARG
    # empty input is a successful no-op
    assert L.kvq_quantize_k(p, 1, 0, 4, 8, 4, 2, p, p, None, None) == \
        kvq.KVQ_OK
    assert L.kvq_dequant(p, p, 1, 4, 8, 4, 9, 2, p, None) == kvq.KVQ_E_ARG
    c = _cfg()
    h = ctypes.c_void_p()
    # misaligned buffer
    assert L.kvq_cache_init(ctypes.byref(c), ctypes.c_void_p(100), 1 << 30,
                            0, ctypes.byref(h), None) == kvq.KVQ_E_ARG
    # too small
    assert L.kvq_cache_init(ctypes.byref(c), ctypes.c_void_p(256), 16, 0,
                            ctypes.byref(h), None) == kvq.KVQ_E_ARG
    assert L.kvq_synth_normal_f16(p, 1, 9, 0, 0, 1, 0, 1, 8, 8, None) == \
        kvq.KVQ_E_ARG
    # rotation: d must be a power of two in 1..256, dtypes f16/f32, and an
    # in-place call keeps its dtype; zero rows is a successful no-op
    for d in (0, 3, 96, 512):
        assert L.kvq_hadamard(p, kvq.KVQ_F16, p, kvq.KVQ_F16, 4, d, None) == \
            kvq.KVQ_E_ARG
    assert L.kvq_hadamard(p, 7, p, kvq.KVQ_F16, 4, 64, None) == kvq.KVQ_E_ARG
    assert L.kvq_hadamard(p, kvq.KVQ_F16, p, kvq.KVQ_F32, 4, 64, None) == \
        kvq.KVQ_E_ARG
    assert L.kvq_hadamard(ctypes.c_void_p(257), kvq.KVQ_F32, p, kvq.KVQ_F32,
                          4, 64, None) == kvq.KVQ_E_ARG
    assert L.kvq_hadamard(None, kvq.KVQ_F16, p, kvq.KVQ_F16, 0, 64, None) == \
        kvq.KVQ_OK


def test_view_validation_and_empty_decode():
    L = kvq.lib()
    v = kvq.KvView()
    v.batch, v.kv_heads, v.head_dim = 1, 1, 32
    # an empty view: decode is an argument error, workspace query too for a
    # head count that does not divide
    assert L.kvq_decode_workspace_bytes(ctypes.byref(v), 3, 0) > 0
    p = ctypes.c_void_p(256)
    assert L.kvq_decode_attention(ctypes.byref(v), p, 1, 3, 0.1, p, 0, 0, p,
                                  1 << 20, None) == kvq.KVQ_E_ARG
    v2 = kvq.KvView()
    v2.batch, v2.kv_heads, v2.head_dim = 1, 2, 32
    assert L.kvq_decode_workspace_bytes(ctypes.byref(v2), 3, 0) == 0
    # quantized tokens but no code arrays
    v.n_quant, v.group_tok, v.group_ch, v.k_bits, v.v_bits = 64, 64, 32, 4, 2
    assert L.kvq_decode_workspace_bytes(ctypes.byref(v), 1, 0) == 0


def test_rope_decode_argument_errors():
    """Every argument error of kvq_decode_attention_rope returns before any
    launch (so this runs without a GPU)."""
    L = kvq.lib()
    p = ctypes.c_void_p(256)
    v = kvq.KvView()
    v.batch, v.kv_heads, v.head_dim = 1, 1, 32
    v.n_sink, v.sink_k, v.sink_v, v.sink_stride = 1, 256, 256, 32
    ws = 1 << 20

    def call(rope, view=v, hq=1, sm=0.1):
        return L.kvq_decode_attention_rope(
            ctypes.byref(view), None if rope is None else ctypes.byref(rope), p, kvq.KVQ_F16,
            hq, sm, p, 0, 0, p, ws, None)

    def rope(**kw):
        r = kvq.Rope(base=10000.0, pairing=kvq.KVQ_ROPE_HALF, reserved=0, pos0=0)
        for k, x in kw.items():
            setattr(r, k, x)
        return r

    assert call(None) == kvq.KVQ_E_ARG
    for bad in ({"base": 0.0}, {"base": -2.0}, {"base": float("nan")},
                {"base": float("inf")}, {"pairing": 2}, {"pos0": -1},
                {"pos0": 1 << 40}):
        assert call(rope(**bad)) == kvq.KVQ_E_ARG, bad
    assert call(rope(), sm=0.0) == kvq.KVQ_E_ARG
    two = kvq.KvView()
    two.batch, two.kv_heads, two.head_dim = 1, 2, 32
    two.n_sink, two.sink_k, two.sink_v, two.sink_stride = 1, 256, 256, 32
    assert call(rope(), view=two, hq=3) == kvq.KVQ_E_ARG  # Hq not a multiple of Hkv
    odd = kvq.KvView()
    odd.batch, odd.kv_heads, odd.head_dim = 1, 1, 33
    odd.n_sink, odd.sink_k, odd.sink_v, odd.sink_stride = 1, 256, 256, 33
    assert call(rope(), view=odd) == kvq.KVQ_E_ARG       # odd head_dim
    empty = kvq.KvView()
    empty.batch, empty.kv_heads, empty.head_dim = 1, 1, 32
    assert call(rope(), view=empty) == kvq.KVQ_E_ARG     # no tokens


def test_struct_layouts_match_the_header(tmp_path):
    """The ctypes mirrors of the C structs have the header's size and field
    offsets (a small C program built with gcc prints them)."""
    import shutil
    import subprocess
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    structs = {"kvq_cache_cfg": kvq.CacheCfg, "kvq_kv_view": kvq.KvView,
               "kvq_ext_view": kvq.ExtView, "kvq_rope": kvq.Rope,
               "kvq_export_bufs": kvq.ExportBufs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"',
             "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    got = {}
    for line in out.splitlines():
        c, f, n = line.split()
        got[(c, f)] = int(n)
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)
