"""Thin ctypes binding of libkvq.so (same names as the C ABI in include/kvq.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libkvq.so.  PyTorch supplies device memory (tensors) and the current HIP
stream.  If the library is missing the import of this module still works,
but every call raises -- there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK, KVQ_E_ARG, KVQ_E_CAPACITY, KVQ_E_NONFINITE, KVQ_E_HIP, \
    KVQ_E_POISONED, KVQ_E_UNSUPPORTED, KVQ_E_SCRATCH = range(8)
NOALLOC_SCRATCH_BYTES = 16 << 20  # KVQ_NOALLOC_SCRATCH_BYTES
KVQ_F32, KVQ_F16 = 0, 1
KVQ_PER_CHANNEL, KVQ_PER_TOKEN = 0, 1
KVQ_V_ROWS, KVQ_V_TILE32 = 0, 1
KVQ_DECODE_AUTO, KVQ_DECODE_GENERIC = 0, 1
KVQ_ROPE_HALF, KVQ_ROPE_INTERLEAVED = 0, 1

EXPORTED = [
    "kvq_words", "kvq_quantize_k", "kvq_quantize_v", "kvq_dequant",
    "kvq_cache_bytes", "kvq_cache_init", "kvq_cache_free", "kvq_cache_tokens",
    "kvq_append", "kvq_salience_select", "kvq_cache_check", "kvq_cache_view",
    "kvq_export", "kvq_decode_workspace_bytes", "kvq_decode_attention",
    "kvq_poll_error", "kvq_strerror", "kvq_fill_u32", "kvq_synth_normal_f16", "kvq_stream_read",
    "kvq_hadamard", "kvq_decode_attention_rope", "kvq_decode_attention_noalloc",
    "kvq_quantize_nuq_k", "kvq_quantize_nuq_v", "kvq_quantize_v_qjl",
    "kvq_decode_ext_workspace_bytes", "kvq_decode_attention_ext",
]

_c_i32, _c_i64, _c_u64, _c_p, _c_f = (ctypes.c_int32, ctypes.c_int64,
                                      ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_float)


class CacheCfg(ctypes.Structure):
    _fields_ = [("batch", _c_i32), ("kv_heads", _c_i32), ("head_dim", _c_i32),
                ("k_bits", _c_i32), ("v_bits", _c_i32), ("group_tok", _c_i32),
                ("group_ch", _c_i32), ("residual", _c_i32), ("sink", _c_i32),
                ("k_mixed", _c_i32), ("n_bf16", _c_i32), ("n_int4", _c_i32),
                ("max_tokens", _c_i64)]


class Rope(ctypes.Structure):
    _fields_ = [("base", ctypes.c_double), ("pairing", _c_i32),
                ("reserved", _c_i32), ("pos0", _c_i64)]


class KvView(ctypes.Structure):
    _fields_ = [("batch", _c_i32), ("kv_heads", _c_i32), ("head_dim", _c_i32),
                ("k_bits", _c_i32), ("v_bits", _c_i32), ("group_tok", _c_i32),
                ("group_ch", _c_i32), ("k_mixed", _c_i32), ("n_bf16", _c_i32),
                ("n_int4", _c_i32), ("v_layout", _c_i32), ("residual", _c_i32),
                ("n_sink", _c_i64), ("n_quant", _c_i64), ("n_tail", _c_i64),
                ("sink_k", _c_p), ("sink_v", _c_p), ("sink_stride", _c_i64),
                ("tail_k", _c_p), ("tail_v", _c_p), ("tail_stride", _c_i64),
                ("k_codes", _c_p), ("k_codes_stride", _c_i64),
                ("k_scales", _c_p), ("k_scales_stride", _c_i64),
                ("k_gmax", _c_p), ("k_gmax_stride", _c_i64),
                ("k_pos", _c_p), ("k_pos_stride", _c_i64),
                ("k_bf16", _c_p), ("k_bf16_stride", _c_i64),
                ("k_int4", _c_p), ("k_int4_stride", _c_i64),
                ("k_int2", _c_p), ("k_int2_stride", _c_i64),
                ("v_codes", _c_p), ("v_codes_stride", _c_i64),
                ("v_scales", _c_p), ("v_scales_stride", _c_i64),
                ("err_flag", _c_p)]


class ExtView(ctypes.Structure):
    _fields_ = [("batch", _c_i32), ("kv_heads", _c_i32), ("head_dim", _c_i32),
                ("reserved0", _c_i32), ("n_tok", _c_i64),
                ("k_bits", _c_i32), ("group_tok", _c_i32), ("k_nuq", _c_i32),
                ("k_n_out", _c_i32),
                ("k_codes", _c_p), ("k_codes_stride", _c_i64),
                ("k_scales", _c_p), ("k_scales_stride", _c_i64),
                ("k_outliers", _c_p), ("k_outliers_stride", _c_i64),
                ("k_lut", _c_f * 16),
                ("v_bits", _c_i32), ("group_ch", _c_i32), ("v_nuq", _c_i32),
                ("v_n_out", _c_i32),
                ("v_codes", _c_p), ("v_codes_stride", _c_i64),
                ("v_scales", _c_p), ("v_scales_stride", _c_i64),
                ("v_outliers", _c_p), ("v_outliers_stride", _c_i64),
                ("v_lut", _c_f * 16),
                ("v_qjl", _c_i32), ("qjl_m", _c_i32), ("v_rotated", _c_i32),
                ("reserved1", _c_i32),
                ("v_sketch", _c_p), ("v_sketch_stride", _c_i64),
                ("v_rnorm", _c_p), ("v_rnorm_stride", _c_i64),
                ("jl", _c_p)]


class ExportBufs(ctypes.Structure):
    _fields_ = [(n, _c_p) for n in (
        "sink_k", "sink_v", "tail_k", "tail_v", "k_codes", "k_scales",
        "k_class", "k_bf16", "k_int4", "k_int2", "v_codes", "v_scales")]


class KvqError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


_lib = None


def lib():
    """The loaded libkvq.so; raises if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "'python -m quantized_decode_attention_02_amd.build'")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "kvq_words": (_c_i32, [_c_i32, _c_i32]),
        "kvq_quantize_k": (_c_i32, [_c_p, _c_i32, _c_i64, _c_i64, _c_i32,
                                    _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p]),
        "kvq_quantize_v": (_c_i32, [_c_p, _c_i32, _c_i64, _c_i64, _c_i32,
                                    _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p]),
        "kvq_dequant": (_c_i32, [_c_p, _c_p, _c_i64, _c_i64, _c_i32, _c_i32,
                                 _c_i32, _c_i32, _c_p, _c_p]),
        "kvq_cache_bytes": (ctypes.c_size_t, [ctypes.POINTER(CacheCfg)]),
        "kvq_cache_init": (_c_i32, [ctypes.POINTER(CacheCfg), _c_p,
                                    ctypes.c_size_t, _c_i64,
                                    ctypes.POINTER(_c_p), _c_p]),
        "kvq_cache_free": (None, [_c_p]),
        "kvq_cache_tokens": (_c_i64, [_c_p]),
        "kvq_append": (_c_i32, [_c_p, _c_p, _c_p, _c_i32, _c_i64, _c_p]),
        "kvq_salience_select": (_c_i32, [_c_p, _c_p, _c_i32, _c_i32, _c_i32,
                                         _c_p]),
        "kvq_cache_check": (_c_i32, [_c_p, _c_p]),
        "kvq_cache_view": (_c_i32, [_c_p, ctypes.POINTER(KvView)]),
        "kvq_export": (_c_i32, [ctypes.POINTER(KvView),
                                ctypes.POINTER(ExportBufs), _c_p]),
        "kvq_decode_workspace_bytes": (ctypes.c_size_t, [
            ctypes.POINTER(KvView), _c_i32, _c_i32]),
        "kvq_decode_attention": (_c_i32, [
            ctypes.POINTER(KvView), _c_p, _c_i32, _c_i32, _c_f, _c_p, _c_i32,
            _c_i32, _c_p, ctypes.c_size_t, _c_p]),
        "kvq_quantize_nuq_k": (_c_i32, [_c_p, _c_i64, _c_i64, _c_i32, _c_i32,
                                        _c_i32, _c_p, _c_i32, _c_p, _c_p, _c_p,
                                        _c_p, _c_p]),
        "kvq_quantize_nuq_v": (_c_i32, [_c_p, _c_i64, _c_i64, _c_i32, _c_i32,
                                        _c_i32, _c_p, _c_i32, _c_p, _c_p, _c_p,
                                        _c_p, _c_p]),
        "kvq_quantize_v_qjl": (_c_i32, [_c_p, _c_i32, _c_i64, _c_i64, _c_i32,
                                        _c_i32, _c_i32, _c_p, _c_i32, _c_p, _c_p,
                                        _c_p, _c_p, _c_p, _c_p]),
        "kvq_decode_ext_workspace_bytes": (ctypes.c_size_t, [
            ctypes.POINTER(ExtView), _c_i32, _c_i32]),
        "kvq_decode_attention_ext": (_c_i32, [
            ctypes.POINTER(ExtView), _c_p, _c_i32, _c_i32, _c_f, _c_p, _c_i32,
            _c_p, ctypes.c_size_t, _c_p]),
        "kvq_decode_attention_noalloc": (_c_i32, [
            ctypes.POINTER(KvView), _c_p, _c_i32, _c_i32, _c_f, _c_p, _c_i32,
            _c_i32, _c_p]),
        "kvq_decode_attention_rope": (_c_i32, [
            ctypes.POINTER(KvView), ctypes.POINTER(Rope), _c_p, _c_i32, _c_i32, _c_f, _c_p,
            _c_i32, _c_i32, _c_p, ctypes.c_size_t, _c_p]),
        "kvq_poll_error": (_c_i32, [_c_p, _c_p]),
        "kvq_strerror": (ctypes.c_char_p, [_c_i32]),
        "kvq_fill_u32": (_c_i32, [_c_p, ctypes.c_uint32, _c_i64, _c_p]),
        "kvq_stream_read": (_c_i32, [_c_p, _c_i64, _c_p, _c_p]),
        "kvq_hadamard": (_c_i32, [_c_p, _c_i32, _c_p, _c_i32, _c_i64, _c_i32, _c_p]),
        "kvq_synth_normal_f16": (_c_i32, [_c_p, _c_u64, _c_i32, _c_i32,
                                          _c_i32, _c_i32, _c_i64, _c_i64,
                                          _c_i32, _c_i64, _c_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def strerror(status):
    try:
        return lib().kvq_strerror(status).decode()
    except RuntimeError:
        return f"status {status}"


def _check(status, where):
    if status != KVQ_OK:
        raise KvqError(status, where)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dtype(t):
    if t.dtype == torch.float16:
        return KVQ_F16
    if t.dtype == torch.float32:
        return KVQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("device tensors must be contiguous CUDA tensors")


def _need_shape(t, shape, where, what):
    """Raise KvqError(KVQ_E_ARG) unless t has exactly `shape`."""
    if tuple(t.shape) != tuple(shape):
        raise KvqError(KVQ_E_ARG, f"{where}: {what} has shape "
                       f"{tuple(t.shape)}, expected {tuple(shape)}")


def _need_bytes(t, n, where, what):
    if t.numel() * t.element_size() < n:
        raise KvqError(KVQ_E_ARG, f"{where}: {what} holds "
                       f"{t.numel() * t.element_size()} bytes, needs {n}")


def kvq_words(n_fields, bits):
    return lib().kvq_words(n_fields, bits)


def kvq_quantize_k(k, bits, group_tok, err=None):
    """k: [n_mats][n_tok][d] -> (codes int32 [.., words], scales f32, err)."""
    _need_cuda(k)
    n_mats, n_tok, d = k.shape
    w = kvq_words(d, bits)
    ng = (n_tok + group_tok - 1) // group_tok if group_tok > 0 else 0
    codes = torch.empty((n_mats, n_tok, max(w, 0)), dtype=torch.int32,
                        device=k.device)
    scales = torch.empty((n_mats, ng, d), dtype=torch.float32, device=k.device)
    if err is None:
        err = torch.zeros(1, dtype=torch.int32, device=k.device)
    _check(lib().kvq_quantize_k(_ptr(k), _dtype(k), n_mats, n_tok, d, bits,
                                group_tok, _ptr(codes), _ptr(scales),
                                _ptr(err), _stream()), "kvq_quantize_k")
    return codes, scales, err


def kvq_quantize_v(v, bits, group_ch, err=None):
    """v: [n_mats][n_tok][d] -> (codes, scales [.., d/Gv], err)."""
    _need_cuda(v)
    n_mats, n_tok, d = v.shape
    w = kvq_words(d, bits)
    ng = d // group_ch if group_ch > 0 else 0
    codes = torch.empty((n_mats, n_tok, max(w, 0)), dtype=torch.int32,
                        device=v.device)
    scales = torch.empty((n_mats, n_tok, ng), dtype=torch.float32,
                         device=v.device)
    if err is None:
        err = torch.zeros(1, dtype=torch.int32, device=v.device)
    _check(lib().kvq_quantize_v(_ptr(v), _dtype(v), n_mats, n_tok, d, bits,
                                group_ch, _ptr(codes), _ptr(scales),
                                _ptr(err), _stream()), "kvq_quantize_v")
    return codes, scales, err


def kvq_hadamard(x, out=None, out_dtype=None):
    """Rotate the last axis of x (float16/float32 device tensor) by the
    normalized Walsh-Hadamard transform; out (optional, may be x) or a new
    tensor of out_dtype (default: x's dtype)."""
    _need_cuda(x)
    d = x.shape[-1]
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    _need_cuda(out)
    if out.shape != x.shape:
        raise ValueError("out must have the shape of x")
    n_rows = x.numel() // d if d else 0
    _check(lib().kvq_hadamard(_ptr(x), _dtype(x), _ptr(out), _dtype(out),
                              n_rows, d, _stream()), "kvq_hadamard")
    return out


def kvq_dequant(codes, scales, n_tok, d, bits, axis, group):
    _need_cuda(codes, scales)
    n_mats = codes.shape[0]
    out = torch.empty((n_mats, n_tok, d), dtype=torch.float32,
                      device=codes.device)
    _check(lib().kvq_dequant(_ptr(codes), _ptr(scales), n_mats, n_tok, d,
                             bits, axis, group, _ptr(out), _stream()),
           "kvq_dequant")
    return out


def kvq_poll_error(err):
    return lib().kvq_poll_error(_ptr(err), _stream())


def kvq_synth_normal_f16(out, seed, tensor, layer, head0, n_heads, t0, n_tok,
                         d, head_stride=None):
    _need_cuda(out)
    if head_stride is None:
        head_stride = n_tok * d
    _check(lib().kvq_synth_normal_f16(_ptr(out), seed, tensor, layer, head0,
                                      n_heads, t0, n_tok, d, head_stride,
                                      _stream()), "kvq_synth_normal_f16")
    return out


STREAM_READ_BLOCKS = 8192  # workgroups of kvq_stream_read


def kvq_stream_read(buf, sink):
    """One launch of the plain streaming-read kernel over the bytes of buf
    (a device tensor); sink: device tensor of at least STREAM_READ_BLOCKS
    int32 (one XOR word per workgroup)."""
    _need_cuda(buf)
    _need_cuda(sink)
    n = buf.numel() * buf.element_size()
    if sink.numel() * sink.element_size() < STREAM_READ_BLOCKS * 4:
        raise ValueError(f"sink needs {STREAM_READ_BLOCKS} words")
    _check(lib().kvq_stream_read(_ptr(buf), n - n % 16, _ptr(sink), _stream()),
           "kvq_stream_read")


class Cache:
    """A kvq_cache bound to one torch-allocated device buffer."""

    def __init__(self, B, Hkv, D, max_tokens, k_bits, v_bits, G, Gv, R, S=0,
                 mixed=False, n_bf16=0, n_int4=0, device="cuda", buf=None,
                 n_tokens=0):
        """A new empty cache in a fresh buffer, or (buf, n_tokens > 0) one
        re-attached to a device buffer that already holds n_tokens tokens
        (a copy of another cache's buffer, e.g. restored from a
        checkpoint)."""
        self.cfg = CacheCfg(batch=B, kv_heads=Hkv, head_dim=D, k_bits=k_bits,
                            v_bits=v_bits, group_tok=G, group_ch=Gv,
                            residual=R, sink=S, k_mixed=int(mixed),
                            n_bf16=n_bf16, n_int4=n_int4,
                            max_tokens=max_tokens)
        nbytes = lib().kvq_cache_bytes(ctypes.byref(self.cfg))
        if nbytes == 0:
            raise KvqError(KVQ_E_ARG, "kvq_cache_bytes")
        if buf is None:
            buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _need_cuda(buf)
        _need_bytes(buf, nbytes, "kvq_cache_init", "buf")
        self.buf = buf
        h = ctypes.c_void_p()
        _check(lib().kvq_cache_init(ctypes.byref(self.cfg), _ptr(self.buf),
                                    buf.numel() * buf.element_size(),
                                    n_tokens, ctypes.byref(h), _stream()),
               "kvq_cache_init")
        self.handle = h
        self.mixed = mixed

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.kvq_cache_free(h)
            self.handle = None

    @property
    def n_tokens(self):
        return lib().kvq_cache_tokens(self.handle)

    def kvq_append(self, k_new, v_new):
        _need_cuda(k_new, v_new)
        c = self.cfg
        if k_new.dim() != 4:
            raise KvqError(KVQ_E_ARG, "kvq_append: k_new must be [B][Hkv][n][D]")
        n_new = k_new.shape[2]
        _need_shape(k_new, (c.batch, c.kv_heads, n_new, c.head_dim),
                    "kvq_append", "k_new")
        _need_shape(v_new, tuple(k_new.shape), "kvq_append", "v_new")
        if v_new.dtype != k_new.dtype:
            raise KvqError(KVQ_E_ARG, "kvq_append: k_new and v_new dtypes differ")
        _check(lib().kvq_append(self.handle, _ptr(k_new), _ptr(v_new),
                                _dtype(k_new), n_new, _stream()),
               "kvq_append")

    def kvq_salience_select(self, q_win):
        _need_cuda(q_win)
        if q_win.dim() != 4 or q_win.shape[0] != self.cfg.batch or \
                q_win.shape[3] != self.cfg.head_dim:
            raise KvqError(KVQ_E_ARG, "kvq_salience_select: q_win must be "
                           "[B][w_rows][Hq][D]")
        _, w, hq, _ = q_win.shape
        _check(lib().kvq_salience_select(self.handle, _ptr(q_win),
                                         _dtype(q_win), w, hq, _stream()),
               "kvq_salience_select")

    def kvq_cache_check(self):
        return lib().kvq_cache_check(self.handle, _stream())

    def kvq_cache_view(self):
        v = KvView()
        _check(lib().kvq_cache_view(self.handle, ctypes.byref(v)),
               "kvq_cache_view")
        return v


def kvq_export(view):
    """Canonical dense device copies of a view (dict of torch tensors)."""
    B, H, D = view.batch, view.kv_heads, view.head_dim
    ns, nq, nt = view.n_sink, view.n_quant, view.n_tail
    dev = torch.device("cuda")
    ng = nq // view.group_tok if view.group_tok > 0 else 0
    t = {
        "sink_k": torch.empty((B, H, ns, D), dtype=torch.float16, device=dev),
        "sink_v": torch.empty((B, H, ns, D), dtype=torch.float16, device=dev),
        "tail_k": torch.empty((B, H, nt, D), dtype=torch.float16, device=dev),
        "tail_v": torch.empty((B, H, nt, D), dtype=torch.float16, device=dev),
        "v_codes": torch.empty((B, H, nq, kvq_words(D, view.v_bits)),
                               dtype=torch.int32, device=dev),
        "v_scales": torch.empty((B, H, nq, D // view.group_ch),
                                dtype=torch.float32, device=dev),
    }
    if view.k_mixed:
        nb, n4 = view.n_bf16, view.n_int4
        n2 = D - nb - n4
        t["k_class"] = torch.empty((B, H, ng, D), dtype=torch.uint8,
                                   device=dev)
        t["k_bf16"] = torch.empty((B, H, nq, nb), dtype=torch.int16,
                                  device=dev)
        t["k_int4"] = torch.empty((B, H, nq, kvq_words(n4, 4)),
                                  dtype=torch.int32, device=dev)
        t["k_int2"] = torch.empty((B, H, nq, kvq_words(n2, 2)),
                                  dtype=torch.int32, device=dev)
        t["k_scales"] = torch.empty((B, H, ng, n4 + n2), dtype=torch.float32,
                                    device=dev)
    else:
        t["k_codes"] = torch.empty((B, H, nq, kvq_words(D, view.k_bits)),
                                   dtype=torch.int32, device=dev)
        t["k_scales"] = torch.empty((B, H, ng, D), dtype=torch.float32,
                                    device=dev)
    bufs = ExportBufs(**{k: (v.data_ptr() if v.numel() else None)
                         for k, v in t.items()})
    _check(lib().kvq_export(ctypes.byref(view), ctypes.byref(bufs), _stream()),
           "kvq_export")
    return t


def kvq_decode_workspace_bytes(view, n_q_heads, n_splits=0):
    return lib().kvq_decode_workspace_bytes(ctypes.byref(view), n_q_heads,
                                            n_splits)


def _decode_args(where, view, q, n_splits, workspace, out):
    """Shape checks shared by the decode calls; returns (hq, sm default,
    workspace, out)."""
    _need_cuda(q)
    if q.dim() != 3:
        raise KvqError(KVQ_E_ARG, f"{where}: q must be [B][Hq][D]")
    B, hq, D = q.shape
    if B != view.batch or D != view.head_dim:
        raise KvqError(KVQ_E_ARG, f"{where}: q is [{B}][{hq}][{D}], the view "
                       f"holds batch {view.batch}, head_dim {view.head_dim}")
    ws_bytes = kvq_decode_workspace_bytes(view, hq, n_splits)
    if ws_bytes == 0:
        raise KvqError(KVQ_E_ARG, "kvq_decode_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    _need_cuda(workspace)
    _need_bytes(workspace, ws_bytes, where, "workspace")
    if out is None:
        out = torch.empty((B, hq, D), dtype=torch.float32, device=q.device)
    _need_cuda(out)
    _need_shape(out, (B, hq, D), where, "out")
    if out.dtype != torch.float32:
        raise KvqError(KVQ_E_ARG, f"{where}: out must be float32")
    return hq, 1.0 / D ** 0.5, workspace, out


def kvq_decode_attention(view, q, sm_scale=None, n_splits=0,
                         flags=KVQ_DECODE_AUTO, workspace=None, out=None):
    """q: [B][Hq][D] f16/f32 -> out [B][Hq][D] float32."""
    hq, sm0, workspace, out = _decode_args("kvq_decode_attention", view, q,
                                           n_splits, workspace, out)
    if sm_scale is None:
        sm_scale = sm0
    _check(lib().kvq_decode_attention(
        ctypes.byref(view), _ptr(q), _dtype(q), hq, sm_scale, _ptr(out),
        n_splits, flags, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream()),
        "kvq_decode_attention")
    return out


def kvq_decode_attention_noalloc(view, q, out, sm_scale=None, n_splits=0,
                                 flags=KVQ_DECODE_AUTO):
    """kvq_decode_attention with the split partials in the library's fixed
    scratch: q [B][Hq][D] f16/f32, out [B][Hq][D] float32 (the caller's);
    nothing is allocated."""
    _need_cuda(q, out)
    if q.dim() != 3 or q.shape[0] != view.batch or q.shape[2] != view.head_dim:
        raise KvqError(KVQ_E_ARG, "kvq_decode_attention_noalloc: q must be "
                       "[B][Hq][D] of the view")
    _need_shape(out, tuple(q.shape), "kvq_decode_attention_noalloc", "out")
    if out.dtype != torch.float32:
        raise KvqError(KVQ_E_ARG, "kvq_decode_attention_noalloc: out must be float32")
    hq, D = q.shape[1], q.shape[2]
    if sm_scale is None:
        sm_scale = 1.0 / D ** 0.5
    _check(lib().kvq_decode_attention_noalloc(
        ctypes.byref(view), _ptr(q), _dtype(q), hq, sm_scale, _ptr(out),
        n_splits, flags, _stream()), "kvq_decode_attention_noalloc")
    return out


def kvq_decode_attention_rope(view, q, base=10000.0, pairing="half", pos0=0,
                              sm_scale=None, n_splits=0, flags=KVQ_DECODE_AUTO,
                              workspace=None, out=None):
    """Decode over keys cached before the rotary embedding: cache-order
    token i is rotated at position pos0 + i.  q: [B][Hq][D] f16/f32, already
    rotated at its own position -> out [B][Hq][D] float32."""
    hq, sm0, workspace, out = _decode_args("kvq_decode_attention_rope", view,
                                           q, n_splits, workspace, out)
    if sm_scale is None:
        sm_scale = sm0
    pr = {"half": KVQ_ROPE_HALF, "interleaved": KVQ_ROPE_INTERLEAVED}.get(pairing, -1)
    rope = Rope(base=base, pairing=pr, reserved=0, pos0=pos0)
    _check(lib().kvq_decode_attention_rope(
        ctypes.byref(view), ctypes.byref(rope), _ptr(q), _dtype(q), hq, sm_scale, _ptr(out),
        n_splits, flags, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream()),
        "kvq_decode_attention_rope")
    return out


def stateless_view(k_codes, k_scales, v_codes, v_scales, B, Hkv, D, k_bits,
                   v_bits, G, Gv, n_tok):
    """A view over kvq_quantize_k/v outputs ([B*Hkv][n_tok][..] arrays)."""
    v = KvView()
    v.batch, v.kv_heads, v.head_dim = B, Hkv, D
    v.k_bits, v.v_bits, v.group_tok, v.group_ch = k_bits, v_bits, G, Gv
    v.v_layout = KVQ_V_ROWS
    v.n_quant = n_tok
    v.k_codes, v.k_codes_stride = k_codes.data_ptr(), k_codes[0].numel()
    v.k_scales, v.k_scales_stride = k_scales.data_ptr(), k_scales[0].numel()
    v.v_codes, v.v_codes_stride = v_codes.data_ptr(), v_codes[0].numel()
    v.v_scales, v.v_scales_stride = v_scales.data_ptr(), v_scales[0].numel()
    return v


_STREAM_ARRAYS = [
    ("sink_k", "sink_stride", 2), ("sink_v", "sink_stride", 2),
    ("tail_k", "tail_stride", 2), ("tail_v", "tail_stride", 2),
    ("k_codes", "k_codes_stride", 4), ("k_scales", "k_scales_stride", 4),
    ("k_gmax", "k_gmax_stride", 4), ("k_pos", "k_pos_stride", 1),
    ("k_bf16", "k_bf16_stride", 2), ("k_int4", "k_int4_stride", 4),
    ("k_int2", "k_int2_stride", 4), ("v_codes", "v_codes_stride", 4),
    ("v_scales", "v_scales_stride", 4),
]


def stream_view(view, b, kvh):
    """A one-stream (batch 1, one KV head) view of stream (b, kvh)."""
    v = KvView()
    ctypes.memmove(ctypes.byref(v), ctypes.byref(view), ctypes.sizeof(KvView))
    s = b * view.kv_heads + kvh
    v.batch, v.kv_heads = 1, 1
    for name, stride, size in _STREAM_ARRAYS:
        p = getattr(view, name)
        if p:
            setattr(v, name, p + s * getattr(view, stride) * size)
    return v


# --------------------------------------------------------------------------
# extended formats: codebook datatype with dense-and-sparse outliers, value
# residual sketch, and their decode
# --------------------------------------------------------------------------

def _host_lut(lut, bits):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(lut, dtype=np.float32))
    if a.shape != (1 << bits,):
        raise KvqError(KVQ_E_ARG, "codebook must hold 2**bits levels")
    return a, a.ctypes.data_as(ctypes.c_void_p)


def kvq_quantize_nuq_k(k, bits, group_tok, lut, n_out, err=None):
    """k: [n_mats][n_tok][d] float16 -> (codes int32 [n_mats][n_tok][words],
    scales f32 [n_mats][ng][d], outliers int32 [n_mats][ng][d][n_out], err)."""
    _need_cuda(k)
    if k.dtype != torch.float16 or k.dim() != 3:
        raise KvqError(KVQ_E_ARG, "kvq_quantize_nuq_k: k must be float16 [n_mats][n_tok][d]")
    n_mats, n_tok, d = k.shape
    ng = (n_tok + group_tok - 1) // group_tok if group_tok > 0 else 0
    codes = torch.empty((n_mats, n_tok, max(kvq_words(d, bits), 0)),
                        dtype=torch.int32, device=k.device)
    scales = torch.empty((n_mats, ng, d), dtype=torch.float32, device=k.device)
    outl = torch.empty((n_mats, ng, d, max(n_out, 0)), dtype=torch.int32, device=k.device)
    if err is None:
        err = torch.zeros(1, dtype=torch.int32, device=k.device)
    keep, lp = _host_lut(lut, bits)
    _check(lib().kvq_quantize_nuq_k(_ptr(k), n_mats, n_tok, d, bits, group_tok, lp,
                                    n_out, _ptr(codes), _ptr(scales),
                                    _ptr(outl) if outl.numel() else None,
                                    _ptr(err), _stream()), "kvq_quantize_nuq_k")
    return codes, scales, outl, err


def kvq_quantize_nuq_v(v, bits, group_ch, lut, n_out, err=None):
    """v: [n_mats][n_tok][d] float16 -> (codes, scales [..][d/Gv],
    outliers int32 [n_mats][n_tok][d/Gv][n_out], err)."""
    _need_cuda(v)
    if v.dtype != torch.float16 or v.dim() != 3:
        raise KvqError(KVQ_E_ARG, "kvq_quantize_nuq_v: v must be float16 [n_mats][n_tok][d]")
    n_mats, n_tok, d = v.shape
    ng = d // group_ch if group_ch > 0 else 0
    codes = torch.empty((n_mats, n_tok, max(kvq_words(d, bits), 0)),
                        dtype=torch.int32, device=v.device)
    scales = torch.empty((n_mats, n_tok, ng), dtype=torch.float32, device=v.device)
    outl = torch.empty((n_mats, n_tok, ng, max(n_out, 0)), dtype=torch.int32, device=v.device)
    if err is None:
        err = torch.zeros(1, dtype=torch.int32, device=v.device)
    keep, lp = _host_lut(lut, bits)
    _check(lib().kvq_quantize_nuq_v(_ptr(v), n_mats, n_tok, d, bits, group_ch, lp,
                                    n_out, _ptr(codes), _ptr(scales),
                                    _ptr(outl) if outl.numel() else None,
                                    _ptr(err), _stream()), "kvq_quantize_nuq_v")
    return codes, scales, outl, err


def kvq_quantize_v_qjl(v, bits, group_ch, jl, err=None):
    """v: [n_mats][n_tok][d] f16/f32 (already rotated), jl [m][d] f32 ->
    (codes, scales, sketch int32 [n_mats][n_tok][m/32], rnorm f32
    [n_mats][n_tok], err)."""
    _need_cuda(v, jl)
    if v.dim() != 3 or jl.dim() != 2 or jl.dtype != torch.float32 or \
            jl.shape[1] != v.shape[2]:
        raise KvqError(KVQ_E_ARG, "kvq_quantize_v_qjl: v [n_mats][n_tok][d], jl [m][d] f32")
    n_mats, n_tok, d = v.shape
    m = jl.shape[0]
    ng = d // group_ch if group_ch > 0 else 0
    codes = torch.empty((n_mats, n_tok, max(kvq_words(d, bits), 0)),
                        dtype=torch.int32, device=v.device)
    scales = torch.empty((n_mats, n_tok, ng), dtype=torch.float32, device=v.device)
    sketch = torch.empty((n_mats, n_tok, max(m // 32, 0)), dtype=torch.int32, device=v.device)
    rnorm = torch.empty((n_mats, n_tok), dtype=torch.float32, device=v.device)
    if err is None:
        err = torch.zeros(1, dtype=torch.int32, device=v.device)
    _check(lib().kvq_quantize_v_qjl(_ptr(v), _dtype(v), n_mats, n_tok, d, bits, group_ch,
                                    _ptr(jl), m, _ptr(codes), _ptr(scales), _ptr(sketch),
                                    _ptr(rnorm), _ptr(err), _stream()), "kvq_quantize_v_qjl")
    return codes, scales, sketch, rnorm, err


def ext_view(B, Hkv, D, n_tok, keys, values, k_bits, v_bits, G, Gv, k_lut=None,
             v_lut=None, sketch=None, rnorm=None, jl=None, v_rotated=False):
    """A kvq_ext_view over quantizer outputs ([B*Hkv][...] arrays).

    keys:   (codes, scales) symmetric, or (codes, scales, outliers) with
            k_lut for the codebook datatype;
    values: (codes, scales) or (codes, scales, outliers) with v_lut;
    sketch, rnorm, jl: the residual sketch of the values (optional)."""
    v = ExtView()
    v.batch, v.kv_heads, v.head_dim, v.n_tok = B, Hkv, D, n_tok
    v.k_bits, v.group_tok, v.v_bits, v.group_ch = k_bits, G, v_bits, Gv
    kc, ks = keys[0], keys[1]
    v.k_codes, v.k_codes_stride = kc.data_ptr(), kc[0].numel()
    v.k_scales, v.k_scales_stride = ks.data_ptr(), ks[0].numel()
    if k_lut is not None:
        v.k_nuq = 1
        v.k_lut[:1 << k_bits] = [float(x) for x in k_lut]
        if len(keys) > 2 and keys[2].numel():
            v.k_n_out = keys[2].shape[-1]
            v.k_outliers, v.k_outliers_stride = keys[2].data_ptr(), keys[2][0].numel()
    vc, vs = values[0], values[1]
    v.v_codes, v.v_codes_stride = vc.data_ptr(), vc[0].numel()
    v.v_scales, v.v_scales_stride = vs.data_ptr(), vs[0].numel()
    if v_lut is not None:
        v.v_nuq = 1
        v.v_lut[:1 << v_bits] = [float(x) for x in v_lut]
        if len(values) > 2 and values[2].numel():
            v.v_n_out = values[2].shape[-1]
            v.v_outliers, v.v_outliers_stride = values[2].data_ptr(), values[2][0].numel()
    if sketch is not None:
        v.v_qjl, v.qjl_m = 1, jl.shape[0]
        v.v_sketch, v.v_sketch_stride = sketch.data_ptr(), sketch[0].numel()
        v.v_rnorm, v.v_rnorm_stride = rnorm.data_ptr(), rnorm[0].numel()
        v.jl = jl.data_ptr()
    v.v_rotated = int(bool(v_rotated))
    return v


def kvq_decode_ext_workspace_bytes(view, n_q_heads, n_splits=0):
    return lib().kvq_decode_ext_workspace_bytes(ctypes.byref(view), n_q_heads, n_splits)


def kvq_decode_attention_ext(view, q, sm_scale=None, n_splits=0, workspace=None, out=None):
    """q: [B][Hq][D] f16/f32 -> out [B][Hq][D] float32."""
    _need_cuda(q)
    if q.dim() != 3 or q.shape[0] != view.batch or q.shape[2] != view.head_dim:
        raise KvqError(KVQ_E_ARG, "kvq_decode_attention_ext: q must be [B][Hq][D] of the view")
    B, hq, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / D ** 0.5
    ws_bytes = kvq_decode_ext_workspace_bytes(view, hq, n_splits)
    if ws_bytes == 0:
        raise KvqError(KVQ_E_ARG, "kvq_decode_ext_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    _need_cuda(workspace)
    _need_bytes(workspace, ws_bytes, "kvq_decode_attention_ext", "workspace")
    if out is None:
        out = torch.empty((B, hq, D), dtype=torch.float32, device=q.device)
    _need_cuda(out)
    _need_shape(out, (B, hq, D), "kvq_decode_attention_ext", "out")
    _check(lib().kvq_decode_attention_ext(
        ctypes.byref(view), _ptr(q), _dtype(q), hq, sm_scale, _ptr(out), n_splits,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()),
        "kvq_decode_attention_ext")
    return out
