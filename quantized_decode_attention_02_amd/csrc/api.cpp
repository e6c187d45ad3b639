// Host side of libkvq: argument validation, cache layout planning, the flush
// plan of kvq_append, path and split selection of the decode.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <math.h>
#include <string.h>

#include "kvq_internal.h"

using namespace kvq;

struct kvq_cache {
  kvq_cache_cfg cfg;
  char* base;
  size_t bytes;
  CacheDev dev;
  int64_t nq_cap;      // quantized-token capacity (multiple of 32)
  int64_t n_tokens, n_sink, n_quant, n_tail;
  int poisoned;
};

namespace {

bool bits_ok(int b) { return b == 8 || b == 4 || b == 3 || b == 2; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int64_t tail_len(int64_t npast, int64_t R, int64_t G) {
  if (npast <= R) return npast;
  return R - G + ((npast - R - 1) % G) + 1;
}

kvq_status hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_E_HIP; }

bool cfg_ok(const kvq_cache_cfg* c) {
  if (!c) return false;
  if (c->batch < 1 || c->kv_heads < 1 || c->head_dim < 1 || c->head_dim > kMaxD) return false;
  if (!bits_ok(c->v_bits)) return false;
  if (!c->k_mixed && !bits_ok(c->k_bits)) return false;
  if (c->group_tok < 1 || c->residual < c->group_tok || c->residual % c->group_tok) return false;
  if (c->group_ch < 1 || c->head_dim % c->group_ch) return false;
  if (c->sink < 0 || c->max_tokens < 0) return false;
  if (c->k_mixed) {
    if (c->n_bf16 < 0 || c->n_int4 < 0 || c->n_bf16 + c->n_int4 > c->head_dim) return false;
  }
  return true;
}

// Lays the cache out in one buffer; fills c when non-null.  Every array is
// 256-byte aligned and every per-stream stride a multiple of 64 bytes.
size_t plan(const kvq_cache_cfg* cfg, char* base, kvq_cache* c) {
  const int64_t ns = (int64_t)cfg->batch * cfg->kv_heads;
  const int D = cfg->head_dim, G = cfg->group_tok, R = cfg->residual;
  const int64_t npast = cfg->max_tokens > cfg->sink ? cfg->max_tokens - cfg->sink : 0;
  const int64_t nq = npast > R ? npast - tail_len(npast, R, G) : 0;
  const int64_t nq_cap = round_up(nq, 32);
  const int64_t ng = nq / G;
  size_t off = 0;
  auto take = [&](int64_t per_stream_bytes, int64_t* stride_elems, int elem) -> char* {
    int64_t per = round_up(per_stream_bytes, 64);
    if (stride_elems) *stride_elems = per / elem;
    char* p = base ? base + off : nullptr;
    off += (size_t)round_up(per * ns, 256);
    return p;
  };
  CacheDev d{};
  d.B = cfg->batch; d.H = cfg->kv_heads; d.D = D;
  d.k_bits = cfg->k_mixed ? 0 : cfg->k_bits; d.v_bits = cfg->v_bits;
  d.G = G; d.Gv = cfg->group_ch; d.R = R; d.S = cfg->sink;
  d.mixed = cfg->k_mixed; d.n_bf16 = cfg->k_mixed ? cfg->n_bf16 : 0;
  d.n_int4 = cfg->k_mixed ? cfg->n_int4 : 0;
  d.v_layout = v_tile_ok(D, cfg->v_bits, G) ? KVQ_V_TILE32 : KVQ_V_ROWS;
  d.err = (uint32_t*)(base ? base + off : nullptr);
  off += 256;
  int64_t dummy;
  // salience intensity: dense [streams][D] float64
  d.I = (double*)(base ? base + off : nullptr);
  off += (size_t)round_up(ns * D * 8, 256);
  d.sink_k = (uint16_t*)take((int64_t)cfg->sink * D * 2, &d.s_sink, 2);
  d.sink_v = (uint16_t*)take((int64_t)cfg->sink * D * 2, &dummy, 2);
  d.tail_k = (uint16_t*)take((int64_t)R * D * 2, &d.s_tail, 2);
  d.tail_v = (uint16_t*)take((int64_t)R * D * 2, &dummy, 2);
  if (!cfg->k_mixed) {
    d.k_codes = (uint32_t*)take(nq_cap * words_of(D, cfg->k_bits) * 4, &d.s_k_codes, 4);
    d.k_scales = (float*)take(ng * D * 4, &d.s_k_scales, 4);
  } else {
    const int nb = cfg->n_bf16, n4 = cfg->n_int4, n2 = D - nb - n4;
    d.k_pos = (uint8_t*)take(ng * D, &d.s_k_pos, 1);
    d.k_scales = (float*)take(ng * (n4 + n2) * 4, &d.s_k_scales, 4);
    d.k_bf16 = (uint16_t*)take(nq_cap * nb * 2, &d.s_k_bf16, 2);
    d.k_int4 = (uint32_t*)take(nq_cap * words_of(n4, 4) * 4, &d.s_k_int4, 4);
    d.k_int2 = (uint32_t*)take(nq_cap * words_of(n2, 2) * 4, &d.s_k_int2, 4);
  }
  d.k_gmax = (float*)take(ng * 4, &d.s_k_gmax, 4);
  d.v_codes = (uint32_t*)take(nq_cap * words_of(D, cfg->v_bits) * 4, &d.s_v_codes, 4);
  d.v_scales = (float*)take(nq_cap * (D / cfg->group_ch) * 4, &d.s_v_scales, 4);
  if (c) {
    c->dev = d;
    c->nq_cap = nq_cap;
  }
  return off;
}

bool view_ok(const kvq_kv_view* v) {
  if (!v) return false;
  if (v->batch < 1 || v->kv_heads < 1 || v->head_dim < 1 || v->head_dim > kMaxD) return false;
  if (v->n_sink < 0 || v->n_quant < 0 || v->n_tail < 0) return false;
  if (v->n_sink > 0 && (!v->sink_k || !v->sink_v)) return false;
  if (v->n_tail > 0 && (!v->tail_k || !v->tail_v || v->residual < v->n_tail)) return false;
  if (v->n_quant > 0) {
    if (v->group_tok < 1 || v->group_ch < 1 || v->head_dim % v->group_ch) return false;
    if (!bits_ok(v->v_bits) || !v->v_codes || !v->v_scales) return false;
    if (v->v_layout == KVQ_V_TILE32) {
      if (!v_tile_ok(v->head_dim, v->v_bits, v->group_tok) || v->n_quant % 32) return false;
    } else if (v->v_layout != KVQ_V_ROWS) {
      return false;
    }
    if (v->k_mixed) {
      if (v->n_bf16 < 0 || v->n_int4 < 0 || v->n_bf16 + v->n_int4 > v->head_dim) return false;
      if (!v->k_pos || !v->k_scales) return false;
      if (v->n_bf16 && !v->k_bf16) return false;
      if (v->n_int4 && !v->k_int4) return false;
      if (v->head_dim - v->n_bf16 - v->n_int4 && !v->k_int2) return false;
      if (v->n_quant % v->group_tok) return false;
    } else {
      if (!bits_ok(v->k_bits) || !v->k_codes || !v->k_scales) return false;
    }
  }
  return true;
}

int generic_parts(const kvq_kv_view* v, int n_splits) {
  const int64_t N = v->n_sink + v->n_quant + v->n_tail;
  if (n_splits > 0) return n_splits;
  const int64_t streams = (int64_t)v->batch * v->kv_heads;
  int64_t p = (1024 + streams - 1) / streams;
  int64_t by_len = (N + 63) / 64;
  if (p > by_len) p = by_len;
  if (p < 1) p = 1;
  if (p > 4096) p = 4096;
  return (int)p;
}

// Split count of the general kernel's rotary form (32-token chunks, small
// LDS footprint): about 4096 workgroups, at least 32 tokens each.
int rope_generic_parts(const kvq_kv_view* v, int n_splits) {
  const int64_t N = v->n_sink + v->n_quant + v->n_tail;
  if (n_splits > 0) return n_splits;
  const int64_t streams = (int64_t)v->batch * v->kv_heads;
  int64_t p = (4096 + streams - 1) / streams;
  int64_t by_len = (N + 31) / 32;
  if (p > by_len) p = by_len;
  if (p < 1) p = 1;
  if (p > 4096) p = 4096;
  return (int)p;
}

size_t generic_lds(int g, int D) {
  return sizeof(float) * ((size_t)g * D * 2 + (size_t)g * 128 + 3 * (size_t)g);
}

}  // namespace

extern "C" {

int kvq_words(int n_fields, int bits) {
  if (!bits_ok(bits) || n_fields < 0) return -1;
  return words_of(n_fields, bits);
}

const char* kvq_strerror(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_E_ARG: return "invalid argument";
    case KVQ_E_CAPACITY: return "cache capacity exceeded";
    case KVQ_E_NONFINITE: return "NaN/Inf input rejected";
    case KVQ_E_HIP: return "HIP runtime error";
    case KVQ_E_POISONED: return "cache poisoned by an earlier NaN/Inf input";
    case KVQ_E_UNSUPPORTED: return "unsupported configuration";
    case KVQ_E_SCRATCH: return "decode partials exceed the fixed scratch of the no-allocation entry point";
  }
  return "unknown status";
}

kvq_status kvq_quantize_k(const void* k, int dtype, int64_t n_mats, int64_t n_tok,
                          int d, int bits, int group_tok, uint32_t* codes,
                          float* scales, uint32_t* err_flag, void* stream) {
  if (dtype != KVQ_F32 && dtype != KVQ_F16) return KVQ_E_ARG;
  if (n_mats < 0 || n_tok < 0 || d < 1 || d > kMaxD || !bits_ok(bits) || group_tok < 1)
    return KVQ_E_ARG;
  if (n_mats == 0 || n_tok == 0) return KVQ_OK;
  if (!k || !codes || !scales || !aligned(codes, 4) || !aligned(scales, 4) ||
      !aligned(k, dtype == KVQ_F32 ? 4 : 2) || (err_flag && !aligned(err_flag, 4)))
    return KVQ_E_ARG;
  if ((n_tok + group_tok - 1) / group_tok > 0x7FFFFFFF || n_mats > 65535) return KVQ_E_UNSUPPORTED;
  return hip_status(launch_quantize_k(k, dtype == KVQ_F16, n_mats, n_tok, d, bits,
                                      group_tok, codes, scales, err_flag, (hipStream_t)stream));
}

kvq_status kvq_quantize_v(const void* v, int dtype, int64_t n_mats, int64_t n_tok,
                          int d, int bits, int group_ch, uint32_t* codes,
                          float* scales, uint32_t* err_flag, void* stream) {
  if (dtype != KVQ_F32 && dtype != KVQ_F16) return KVQ_E_ARG;
  if (n_mats < 0 || n_tok < 0 || d < 1 || d > kMaxD || !bits_ok(bits) || group_ch < 1 ||
      d % group_ch)
    return KVQ_E_ARG;
  if (n_mats == 0 || n_tok == 0) return KVQ_OK;
  if (!v || !codes || !scales || !aligned(codes, 4) || !aligned(scales, 4) ||
      !aligned(v, dtype == KVQ_F32 ? 4 : 2))
    return KVQ_E_ARG;
  if ((n_tok + 31) / 32 > 0x7FFFFFFF || n_mats > 65535) return KVQ_E_UNSUPPORTED;
  return hip_status(launch_quantize_v(v, dtype == KVQ_F16, n_mats, n_tok, d, bits,
                                      group_ch, codes, scales, err_flag, (hipStream_t)stream));
}

kvq_status kvq_dequant(const uint32_t* codes, const float* scales, int64_t n_mats,
                       int64_t n_tok, int d, int bits, int axis, int group,
                       float* out, void* stream) {
  if (n_mats < 0 || n_tok < 0 || d < 1 || d > kMaxD || !bits_ok(bits) || group < 1)
    return KVQ_E_ARG;
  if (axis != KVQ_PER_CHANNEL && axis != KVQ_PER_TOKEN) return KVQ_E_ARG;
  if (axis == KVQ_PER_TOKEN && d % group) return KVQ_E_ARG;
  if (n_mats == 0 || n_tok == 0) return KVQ_OK;
  if (!codes || !scales || !out || !aligned(codes, 4) || !aligned(scales, 4) || !aligned(out, 4))
    return KVQ_E_ARG;
  return hip_status(launch_dequant(codes, scales, n_mats, n_tok, d, bits, axis, group,
                                   out, (hipStream_t)stream));
}

size_t kvq_cache_bytes(const kvq_cache_cfg* cfg) {
  if (!cfg_ok(cfg)) return 0;
  return plan(cfg, nullptr, nullptr);
}

kvq_status kvq_cache_init(const kvq_cache_cfg* cfg, void* dev_buf, size_t bytes,
                          int64_t n_tokens, kvq_cache** out, void* stream) {
  if (!out) return KVQ_E_ARG;
  *out = nullptr;
  if (!cfg_ok(cfg) || !dev_buf || !aligned(dev_buf, 256)) return KVQ_E_ARG;
  if (bytes < plan(cfg, nullptr, nullptr)) return KVQ_E_ARG;
  if (n_tokens < 0 || n_tokens > cfg->max_tokens) return KVQ_E_ARG;
  kvq_cache* c = (kvq_cache*)calloc(1, sizeof(kvq_cache));
  if (!c) return KVQ_E_ARG;
  c->cfg = *cfg;
  c->base = (char*)dev_buf;
  c->bytes = bytes;
  plan(cfg, c->base, c);
  const int64_t S = cfg->sink, R = cfg->residual, G = cfg->group_tok;
  c->n_tokens = n_tokens;
  c->n_sink = n_tokens < S ? n_tokens : S;
  const int64_t npast = n_tokens - c->n_sink;
  c->n_tail = tail_len(npast, R, G);
  c->n_quant = npast - c->n_tail;
  hipStream_t s = (hipStream_t)stream;
  if (n_tokens == 0) {
    hipError_t e = launch_fill_u32(c->dev.err, 0u, 1, s);
    if (e == hipSuccess)
      e = launch_fill_f64(c->dev.I, 1.0, (int64_t)cfg->batch * cfg->kv_heads * cfg->head_dim, s);
    if (e != hipSuccess) {
      free(c);
      return KVQ_E_HIP;
    }
  }
  *out = c;
  return KVQ_OK;
}

void kvq_cache_free(kvq_cache* c) { free(c); }

int64_t kvq_cache_tokens(const kvq_cache* c) { return c ? c->n_tokens : -1; }

kvq_status kvq_append(kvq_cache* c, const void* k_new, const void* v_new, int dtype,
                      int64_t n_new, void* stream) {
  if (!c) return KVQ_E_ARG;
  if (c->poisoned) return KVQ_E_POISONED;
  if (dtype != KVQ_F16 || n_new < 0) return KVQ_E_ARG;
  if (n_new == 0) return KVQ_OK;
  if (!k_new || !v_new || !aligned(k_new, 2) || !aligned(v_new, 2)) return KVQ_E_ARG;
  if (c->n_tokens + n_new > c->cfg.max_tokens) return KVQ_E_CAPACITY;
  const int64_t S = c->cfg.sink, R = c->cfg.residual, G = c->cfg.group_tok;
  const int64_t take = (S - c->n_sink) < n_new ? (S - c->n_sink) : n_new;
  const int64_t m = n_new - take;
  const int64_t nq_old = c->n_quant, nt_old = c->n_tail;
  const int64_t total = nt_old + m;
  const int64_t F = total > R ? (total - R + G - 1) / G : 0;
  if (nq_old + F * G > c->nq_cap) return KVQ_E_CAPACITY;
  hipStream_t s = (hipStream_t)stream;
  const uint16_t* kin = (const uint16_t*)k_new;
  const uint16_t* vin = (const uint16_t*)v_new;
  // 1. quantize the flushed groups (reads ring rows and input rows)
  hipError_t e = launch_flush(c->dev, kin, vin, n_new, take, nq_old, nt_old, F, s);
  // 2. then write sink rows and the surviving new tail rows
  const int64_t skip = F * G > nt_old ? F * G - nt_old : 0;  // new tokens flushed
  const int64_t in_lo = take + skip, in_hi = n_new;
  const int64_t p_lo = nq_old + nt_old + skip;
  if (e == hipSuccess)
    e = launch_append_rows(c->dev, kin, vin, n_new, c->n_sink, take, in_lo, in_hi, p_lo, s);
  if (e != hipSuccess) return KVQ_E_HIP;
  c->n_sink += take;
  c->n_quant = nq_old + F * G;
  c->n_tail = total - F * G;
  c->n_tokens += n_new;
  return KVQ_OK;
}

kvq_status kvq_salience_select(kvq_cache* c, const void* q_win, int dtype, int w_rows,
                               int n_q_heads, void* stream) {
  if (!c) return KVQ_E_ARG;
  if (c->poisoned) return KVQ_E_POISONED;
  if (!c->cfg.k_mixed || dtype != KVQ_F16 || w_rows < 0 || n_q_heads < 1 ||
      n_q_heads % c->cfg.kv_heads)
    return KVQ_E_ARG;
  if (w_rows > 0 && (!q_win || !aligned(q_win, 2))) return KVQ_E_ARG;
  // a window row of 32 channels of a KV head's query heads is staged in
  // 64 KB of LDS
  if ((int64_t)(n_q_heads / c->cfg.kv_heads) * 32 * 2 > 65536) return KVQ_E_UNSUPPORTED;
  return hip_status(launch_salience(c->dev, (const uint16_t*)q_win, w_rows, n_q_heads,
                                    (hipStream_t)stream));
}

kvq_status kvq_cache_check(kvq_cache* c, void* stream) {
  if (!c) return KVQ_E_ARG;
  kvq_status st = kvq_poll_error(c->dev.err, stream);
  if (st == KVQ_E_NONFINITE) c->poisoned = 1;
  if (st == KVQ_OK && c->poisoned) return KVQ_E_POISONED;
  return st;
}

kvq_status kvq_cache_view(const kvq_cache* c, kvq_kv_view* v) {
  if (!c || !v) return KVQ_E_ARG;
  if (c->poisoned) return KVQ_E_POISONED;
  const CacheDev& d = c->dev;
  memset(v, 0, sizeof(*v));
  v->batch = d.B; v->kv_heads = d.H; v->head_dim = d.D;
  v->k_bits = d.k_bits; v->v_bits = d.v_bits; v->group_tok = d.G; v->group_ch = d.Gv;
  v->k_mixed = d.mixed; v->n_bf16 = d.n_bf16; v->n_int4 = d.n_int4;
  v->v_layout = d.v_layout; v->residual = d.R;
  v->n_sink = c->n_sink; v->n_quant = c->n_quant; v->n_tail = c->n_tail;
  v->sink_k = d.sink_k; v->sink_v = d.sink_v; v->sink_stride = d.s_sink;
  v->tail_k = d.tail_k; v->tail_v = d.tail_v; v->tail_stride = d.s_tail;
  v->k_codes = d.k_codes; v->k_codes_stride = d.s_k_codes;
  v->k_scales = d.k_scales; v->k_scales_stride = d.s_k_scales;
  v->k_gmax = d.k_gmax; v->k_gmax_stride = d.s_k_gmax;
  v->k_pos = d.k_pos; v->k_pos_stride = d.s_k_pos;
  v->k_bf16 = d.k_bf16; v->k_bf16_stride = d.s_k_bf16;
  v->k_int4 = d.k_int4; v->k_int4_stride = d.s_k_int4;
  v->k_int2 = d.k_int2; v->k_int2_stride = d.s_k_int2;
  v->v_codes = d.v_codes; v->v_codes_stride = d.s_v_codes;
  v->v_scales = d.v_scales; v->v_scales_stride = d.s_v_scales;
  v->err_flag = d.err;
  return KVQ_OK;
}

kvq_status kvq_export(const kvq_kv_view* v, const kvq_export_bufs* out, void* stream) {
  if (!view_ok(v) || !out) return KVQ_E_ARG;
  return hip_status(launch_export(*v, *out, (hipStream_t)stream));
}

size_t kvq_decode_workspace_bytes(const kvq_kv_view* v, int n_q_heads, int n_splits) {
  if (!view_ok(v) || n_q_heads < 1 || n_q_heads % v->kv_heads || n_splits < 0 ||
      n_splits > 16384)
    return 0;
  int parts = generic_parts(v, n_splits);
  if (mfma_decode_eligible(*v, n_q_heads)) {
    int pm = mfma_decode_parts(*v, n_q_heads, n_splits);
    if (pm > parts) parts = pm;
  }
  if (rope_fast_eligible(*v, n_q_heads)) {
    int pr = rope_fast_parts(*v, n_q_heads, n_splits) + rope_fp16_parts(*v);
    if (pr > parts) parts = pr;
  }
  if (v->head_dim % 2 == 0) {
    int pg = rope_generic_parts(v, n_splits);
    if (pg > parts) parts = pg;
  }
  return (size_t)v->batch * n_q_heads * parts * (v->head_dim + 2) * sizeof(float);
}

kvq_status kvq_decode_attention(const kvq_kv_view* v, const void* q, int dtype,
                                int n_q_heads, float sm_scale, float* out, int n_splits,
                                int flags, void* workspace, size_t ws_bytes, void* stream) {
  return kvq::decode_attention_impl(v, q, dtype, n_q_heads, sm_scale, out, n_splits, flags,
                                    workspace, ws_bytes, stream);
}

}  // extern "C"

namespace kvq {

kvq_status decode_attention_impl(const kvq_kv_view* v, const void* q, int dtype, int n_q_heads,
                                 float sm_scale, float* out, int n_splits, int flags,
                                 void* workspace, size_t ws_bytes, void* stream) {
  if (!view_ok(v) || !q || !out || !workspace) return KVQ_E_ARG;
  if (dtype != KVQ_F16 && dtype != KVQ_F32) return KVQ_E_ARG;
  if (n_q_heads < 1 || n_q_heads % v->kv_heads || n_splits < 0 || n_splits > 16384)
    return KVQ_E_ARG;
  if (flags != KVQ_DECODE_AUTO && flags != KVQ_DECODE_GENERIC) return KVQ_E_ARG;
  if (!aligned(q, dtype == KVQ_F32 ? 4 : 2) || !aligned(out, 4) || !aligned(workspace, 4))
    return KVQ_E_ARG;
  if (!(sm_scale > 0.0f) || !__builtin_isfinite(sm_scale)) return KVQ_E_ARG;
  const int64_t N = v->n_sink + v->n_quant + v->n_tail;
  if (N == 0) return KVQ_E_ARG;
  if (ws_bytes < kvq_decode_workspace_bytes(v, n_q_heads, n_splits)) return KVQ_E_ARG;
  if ((int64_t)v->batch * n_q_heads > 0x7FFFFFFF || v->batch > 65535) return KVQ_E_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  float* partials = (float*)workspace;
  const int g = n_q_heads / v->kv_heads;
  hipError_t e;
  int parts;
  if (flags == KVQ_DECODE_AUTO && aligned(q, 16) && mfma_decode_eligible(*v, n_q_heads)) {
    parts = mfma_decode_parts(*v, n_q_heads, n_splits);
    e = launch_decode_mfma(*v, q, dtype == KVQ_F16, n_q_heads, sm_scale, partials, parts, s);
  } else {
    const size_t lds = generic_lds(g, v->head_dim);
    if (lds > 160 * 1024) return KVQ_E_UNSUPPORTED;
    parts = generic_parts(v, n_splits);
    e = launch_decode_generic(*v, q, dtype == KVQ_F16, n_q_heads, sm_scale, partials,
                              parts, s);
  }
  if (e == hipSuccess) e = launch_merge(partials, v->batch, n_q_heads, v->head_dim, parts, out, s);
  return hip_status(e);
}

}  // namespace kvq

extern "C" {

kvq_status kvq_decode_attention_rope(const kvq_kv_view* v, const kvq_rope* rope, const void* q,
                                     int dtype, int n_q_heads, float sm_scale, float* out,
                                     int n_splits, int flags, void* workspace, size_t ws_bytes,
                                     void* stream) {
  if (!view_ok(v) || !rope || !q || !out || !workspace) return KVQ_E_ARG;
  if (dtype != KVQ_F16 && dtype != KVQ_F32) return KVQ_E_ARG;
  if (n_q_heads < 1 || n_q_heads % v->kv_heads || n_splits < 0 || n_splits > 16384)
    return KVQ_E_ARG;
  if (flags != KVQ_DECODE_AUTO && flags != KVQ_DECODE_GENERIC) return KVQ_E_ARG;
  if (!aligned(q, dtype == KVQ_F32 ? 4 : 2) || !aligned(out, 4) || !aligned(workspace, 4))
    return KVQ_E_ARG;
  if (!(sm_scale > 0.0f) || !__builtin_isfinite(sm_scale)) return KVQ_E_ARG;
  if (v->head_dim % 2) return KVQ_E_ARG;
  if (!(rope->base > 0.0) || !__builtin_isfinite(rope->base)) return KVQ_E_ARG;
  if (rope->pairing != KVQ_ROPE_HALF && rope->pairing != KVQ_ROPE_INTERLEAVED) return KVQ_E_ARG;
  const int64_t N = v->n_sink + v->n_quant + v->n_tail;
  if (N == 0) return KVQ_E_ARG;
  if (rope->pos0 < 0 || rope->pos0 > ((int64_t)1 << 40) - N) return KVQ_E_ARG;
  if (ws_bytes < kvq_decode_workspace_bytes(v, n_q_heads, n_splits)) return KVQ_E_ARG;
  if ((int64_t)v->batch * n_q_heads > 0x7FFFFFFF || v->batch > 65535) return KVQ_E_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  float* partials = (float*)workspace;
  RopeDev rd{};
  rd.base = rope->base;
  rd.interleaved = rope->pairing == KVQ_ROPE_INTERLEAVED;
  rd.pos0 = rope->pos0;
  for (int f = 0; f < v->head_dim / 2; ++f)
    rd.phi[f] = pow(rope->base, -2.0 * f / v->head_dim) * 0.15915494309189533577;  // / (2 pi)
  hipError_t e;
  int parts;
  if (flags == KVQ_DECODE_AUTO && rope_fast_eligible(*v, n_q_heads)) {
    const int pf = rope_fast_parts(*v, n_q_heads, n_splits);
    parts = pf + rope_fp16_parts(*v);
    e = launch_decode_rope(*v, q, dtype == KVQ_F16, n_q_heads, sm_scale, rd, partials, pf, s);
  } else {
    // the rotary form of the general kernel: 32-token chunks, their keys
    // and values staged in LDS
    const size_t g = n_q_heads / v->kv_heads, D = v->head_dim;
    const size_t lds = sizeof(float) * (g * D * 2 + g * 32 + 3 * g + D * (1 + 32));
    if (lds > 160 * 1024) return KVQ_E_UNSUPPORTED;
    parts = rope_generic_parts(v, n_splits);
    e = launch_decode_generic_range(*v, q, dtype == KVQ_F16, n_q_heads, sm_scale, partials, 0,
                                    N, parts, 0, parts, &rd, s);
  }
  if (e == hipSuccess) e = launch_merge(partials, v->batch, n_q_heads, v->head_dim, parts, out, s);
  return hip_status(e);
}

}  // extern "C"

namespace {

// fp16 numbers: at most 11 significant bits, within the fp16 range.
bool fp16_exact(float x) {
  const double a = fabs((double)x);
  if (a == 0.0) return true;
  if (!(a <= 65504.0)) return false;
  if (a < 6.103515625e-05) {  // subnormal: a multiple of 2^-24
    const double t = a * 16777216.0;
    return t == rint(t);
  }
  int e;
  const double m = frexp(a, &e);
  return m * 2048.0 == rint(m * 2048.0);
}

// Host codebook -> kernel arguments; false if it is not a valid one
// (2^bits strictly ascending fp16 numbers including 0, every midpoint of
// neighbours a float32 number).
bool make_lut(const float* lut, int bits, ExtLut* out) {
  if (!lut || bits < 2 || bits > 4) return false;
  const int n = 1 << bits;
  bool zero = false;
  ExtLut L{};
  L.n = n;
  for (int j = 0; j < n; ++j) {
    const float x = lut[j];
    if (!__builtin_isfinite(x) || !fp16_exact(x)) return false;
    if (j > 0 && !(x > lut[j - 1])) return false;
    if (x == 0.0f) zero = true;
    L.lvl[j] = x;
  }
  if (!zero) return false;
  for (int j = 0; j + 1 < n; ++j) {
    const double mid = ((double)lut[j] + (double)lut[j + 1]) * 0.5;
    if ((double)(float)mid != mid) return false;
    L.mid[j] = (float)mid;
  }
  L.absmax = fmaxf(fabsf(lut[0]), fabsf(lut[n - 1]));
  *out = L;
  return true;
}

bool ext_view_ok(const kvq_ext_view* v, int n_q_heads) {
  if (!v) return false;
  if (v->batch < 1 || v->kv_heads < 1) return false;
  if (v->head_dim != 32 && v->head_dim != 64 && v->head_dim != 128) return false;
  if (v->n_tok < 1 || n_q_heads < 1 || n_q_heads % v->kv_heads) return false;
  const int g = n_q_heads / v->kv_heads;
  if (g > 8) return false;
  if (v->group_tok < 1 || v->group_tok % 32 || v->group_ch < 1 || v->head_dim % v->group_ch)
    return false;
  if (!v->k_codes || !v->k_scales || !v->v_codes || !v->v_scales) return false;
  if (v->k_nuq ? (v->k_bits < 2 || v->k_bits > 4) : !bits_ok(v->k_bits)) return false;
  if (v->v_nuq ? (v->v_bits < 2 || v->v_bits > 4) : !bits_ok(v->v_bits)) return false;
  if (v->k_n_out < 0 || v->k_n_out > 16 || v->v_n_out < 0 || v->v_n_out > 16) return false;
  if ((!v->k_nuq && v->k_n_out) || (!v->v_nuq && v->v_n_out)) return false;
  if (v->k_n_out && !v->k_outliers) return false;
  if (v->v_n_out && !v->v_outliers) return false;
  if (v->v_qjl) {
    if (v->qjl_m < 32 || v->qjl_m > 256 || v->qjl_m % 32) return false;
    if (g * v->qjl_m > 8 * 256 || !v->v_sketch || !v->v_rnorm || !v->jl) return false;
  }
  if (v->v_rotated && (v->head_dim & (v->head_dim - 1))) return false;
  if (!aligned(v->k_codes, 4) || !aligned(v->v_codes, 4) || !aligned(v->k_scales, 4) ||
      !aligned(v->v_scales, 4))
    return false;
  return true;
}

}  // namespace

extern "C" {

kvq_status kvq_quantize_nuq_k(const void* k, int64_t n_mats, int64_t n_tok, int d, int bits,
                              int group_tok, const float* lut, int n_out, uint32_t* codes,
                              float* scales, uint32_t* outliers, uint32_t* err_flag,
                              void* stream) {
  ExtLut L;
  if (!make_lut(lut, bits, &L)) return KVQ_E_ARG;
  if (n_mats < 0 || n_tok < 0 || d < 1 || d > kMaxD || group_tok < 1 || n_out < 0 || n_out > 16)
    return KVQ_E_ARG;
  if ((int64_t)group_tok * d > 32768 || group_tok > 65535) return KVQ_E_ARG;
  if (n_mats == 0 || n_tok == 0) return KVQ_OK;
  if (!k || !codes || !scales || (n_out && !outliers) || !aligned(k, 2) || !aligned(codes, 4) ||
      !aligned(scales, 4) || (outliers && !aligned(outliers, 4)) ||
      (err_flag && !aligned(err_flag, 4)))
    return KVQ_E_ARG;
  if ((n_tok + group_tok - 1) / group_tok > 0x7FFFFFFF || n_mats > 65535) return KVQ_E_UNSUPPORTED;
  return hip_status(launch_quantize_nuq_k((const uint16_t*)k, n_mats, n_tok, d, bits, group_tok,
                                          L, n_out, codes, scales, outliers, err_flag,
                                          (hipStream_t)stream));
}

kvq_status kvq_quantize_nuq_v(const void* v, int64_t n_mats, int64_t n_tok, int d, int bits,
                              int group_ch, const float* lut, int n_out, uint32_t* codes,
                              float* scales, uint32_t* outliers, uint32_t* err_flag,
                              void* stream) {
  ExtLut L;
  if (!make_lut(lut, bits, &L)) return KVQ_E_ARG;
  if (n_mats < 0 || n_tok < 0 || d < 1 || d > kMaxD || group_ch < 1 || d % group_ch ||
      n_out < 0 || n_out > 16)
    return KVQ_E_ARG;
  if (n_mats == 0 || n_tok == 0) return KVQ_OK;
  if (!v || !codes || !scales || (n_out && !outliers) || !aligned(v, 2) || !aligned(codes, 4) ||
      !aligned(scales, 4) || (outliers && !aligned(outliers, 4)) ||
      (err_flag && !aligned(err_flag, 4)))
    return KVQ_E_ARG;
  if ((n_tok + 31) / 32 > 0x7FFFFFFF || n_mats > 65535) return KVQ_E_UNSUPPORTED;
  return hip_status(launch_quantize_nuq_v((const uint16_t*)v, n_mats, n_tok, d, bits, group_ch, L,
                                          n_out, codes, scales, outliers, err_flag,
                                          (hipStream_t)stream));
}

kvq_status kvq_quantize_v_qjl(const void* v, int dtype, int64_t n_mats, int64_t n_tok, int d,
                              int bits, int group_ch, const float* jl, int m, uint32_t* codes,
                              float* scales, uint32_t* sketch, float* rnorm,
                              uint32_t* err_flag, void* stream) {
  if (dtype != KVQ_F32 && dtype != KVQ_F16) return KVQ_E_ARG;
  if (n_mats < 0 || n_tok < 0 || d < 1 || d > kMaxD || !bits_ok(bits) || group_ch < 1 ||
      d % group_ch || m < 32 || m > 256 || m % 32)
    return KVQ_E_ARG;
  if (n_mats == 0 || n_tok == 0) return KVQ_OK;
  if (!v || !jl || !codes || !scales || !sketch || !rnorm ||
      !aligned(v, dtype == KVQ_F32 ? 4 : 2) || !aligned(jl, 4) || !aligned(codes, 4) ||
      !aligned(scales, 4) || !aligned(sketch, 4) || !aligned(rnorm, 4) ||
      (err_flag && !aligned(err_flag, 4)))
    return KVQ_E_ARG;
  if ((n_tok + 31) / 32 > 0x7FFFFFFF || n_mats > 65535) return KVQ_E_UNSUPPORTED;
  return hip_status(launch_quantize_v_qjl(v, dtype == KVQ_F16, n_mats, n_tok, d, bits, group_ch, jl,
                                          m, codes, scales, sketch, rnorm, err_flag,
                                          (hipStream_t)stream));
}

size_t kvq_decode_ext_workspace_bytes(const kvq_ext_view* v, int n_q_heads, int n_splits) {
  if (!ext_view_ok(v, n_q_heads) || n_splits < 0 || n_splits > 4096) return 0;
  const int parts = ext_decode_parts(*v, n_q_heads, n_splits);
  const int M = v->v_qjl ? v->qjl_m : 0;
  return (size_t)v->batch * n_q_heads * parts * (v->head_dim + 2 + M) * sizeof(float);
}

kvq_status kvq_decode_attention_ext(const kvq_ext_view* v, const void* q, int dtype,
                                    int n_q_heads, float sm_scale, float* out, int n_splits,
                                    void* workspace, size_t ws_bytes, void* stream) {
  if (!ext_view_ok(v, n_q_heads) || !q || !out || !workspace) return KVQ_E_ARG;
  if (dtype != KVQ_F16 && dtype != KVQ_F32) return KVQ_E_ARG;
  if (n_splits < 0 || n_splits > 4096) return KVQ_E_ARG;
  if (!aligned(q, dtype == KVQ_F32 ? 4 : 2) || !aligned(out, 4) || !aligned(workspace, 4))
    return KVQ_E_ARG;
  if (!(sm_scale > 0.0f) || !__builtin_isfinite(sm_scale)) return KVQ_E_ARG;
  if (ws_bytes < kvq_decode_ext_workspace_bytes(v, n_q_heads, n_splits)) return KVQ_E_ARG;
  if ((int64_t)v->batch * n_q_heads > 0x7FFFFFFF || v->batch > 65535) return KVQ_E_UNSUPPORTED;
  ExtLut lk{}, lv{};
  if (v->k_nuq && !make_lut(v->k_lut, v->k_bits, &lk)) return KVQ_E_ARG;
  if (v->v_nuq && !make_lut(v->v_lut, v->v_bits, &lv)) return KVQ_E_ARG;
  if (ext_decode_lds(*v, n_q_heads) > 160 * 1024) return KVQ_E_UNSUPPORTED;
  const int parts = ext_decode_parts(*v, n_q_heads, n_splits);
  return hip_status(launch_decode_ext(*v, lk, lv, q, dtype == KVQ_F16, n_q_heads, sm_scale,
                                      (float*)workspace, parts, out, (hipStream_t)stream));
}

kvq_status kvq_poll_error(const uint32_t* err_flag, void* stream) {
  if (!err_flag || !aligned(err_flag, 4)) return KVQ_E_ARG;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return KVQ_E_HIP;
  uint32_t h = 0;
  if (hipMemcpy(&h, err_flag, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return KVQ_E_HIP;
  return h ? KVQ_E_NONFINITE : KVQ_OK;
}

kvq_status kvq_hadamard(const void* in, int in_dtype, void* out, int out_dtype, int64_t n_rows,
                        int d, void* stream) {
  if (n_rows < 0 || d < 1 || d > kMaxD || (d & (d - 1))) return KVQ_E_ARG;
  if ((in_dtype != KVQ_F16 && in_dtype != KVQ_F32) || (out_dtype != KVQ_F16 && out_dtype != KVQ_F32))
    return KVQ_E_ARG;
  if (n_rows == 0) return KVQ_OK;
  const size_t ei = in_dtype == KVQ_F16 ? 2 : 4, eo = out_dtype == KVQ_F16 ? 2 : 4;
  if (!in || !out || !aligned(in, ei) || !aligned(out, eo)) return KVQ_E_ARG;
  if (in == out && in_dtype != out_dtype) return KVQ_E_ARG;
  return hip_status(launch_hadamard(in, in_dtype == KVQ_F16, out, out_dtype == KVQ_F16, n_rows, d,
                                    (hipStream_t)stream));
}

kvq_status kvq_fill_u32(uint32_t* dst, uint32_t value, int64_t n, void* stream) {
  if (n < 0 || (n > 0 && (!dst || !aligned(dst, 4)))) return KVQ_E_ARG;
  return hip_status(launch_fill_u32(dst, value, n, (hipStream_t)stream));
}

kvq_status kvq_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0 || bytes % 16 || (bytes > 0 && (!src || !aligned(src, 16) || !sink || !aligned(sink, 4))))
    return KVQ_E_ARG;
  return hip_status(launch_stream_read(src, bytes, sink, (hipStream_t)stream));
}

kvq_status kvq_synth_normal_f16(void* out, uint64_t seed, int tensor, int layer, int head0,
                                int n_heads, int64_t t0, int64_t n_tok, int d,
                                int64_t head_stride, void* stream) {
  if (tensor < 0 || tensor > 3 || layer < 0 || layer > 255 || head0 < 0 || n_heads < 0 ||
      head0 + n_heads > 256 || t0 < 0 || n_tok < 0 || t0 + n_tok > (1LL << 32) || d < 1 ||
      d > 256 || head_stride < n_tok * d)
    return KVQ_E_ARG;
  if (n_heads == 0 || n_tok == 0) return KVQ_OK;
  if (!out || !aligned(out, 2)) return KVQ_E_ARG;
  return hip_status(launch_synth((uint16_t*)out, seed, tensor, layer, head0, n_heads, t0,
                                 n_tok, d, head_stride, (hipStream_t)stream));
}

}  // extern "C"
