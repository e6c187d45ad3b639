/*
 * kvq.h -- C ABI of libkvq.so: quantized KV cache and decode attention for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources are the pages' titles and sections):
 *
 *  - Symmetric absmax rule ("KV quantization axes: why Key and Value need
 *    separate reasoning", section "What rows and columns mean"): for a group
 *    x, scale = max|x| / qmax, code = clip(round(x / scale), -qmax, qmax),
 *    x_hat = code * scale.  Here qmax = 2^(b-1) - 1 for b in {8, 4, 3, 2},
 *    round is round-half-to-even, and both divisions are IEEE float32
 *    divisions.  A zero group uses scale 1; NaN/Inf input is rejected (same
 *    page, closing troubleshooting paragraph).
 *  - Grouping axes ("KVQuant: Towards 10 Million Context Length LLM
 *    Inference with KV Cache Quantization", table "Measured effects"; the
 *    page above, "What rows and columns mean"): keys per channel, grouped
 *    along G tokens; values per token, grouped along Gv channels.
 *  - Residual tail and sink ("MixKVQ: Query-Aware Mixed-Precision KV Cache
 *    Quantization for Long-Context Reasoning", Figure 4; "KVQuant ...",
 *    summary): recent tokens stay in fp16 in a buffer of R tokens; the first
 *    S tokens stay fp16 as attention sinks.
 *  - Salience ("MixKVQ ...", Figure 3): A_d = I_d * S_d (query intensity
 *    times key scale); the top channels stay bf16, the next int4, the rest
 *    int2.
 *  - Decode attention ("KV quantization axes ...", section "Separate the two
 *    error paths"): out = softmax(q K_hat^T * sm_scale) V_hat per query
 *    head, over every cached token (no mask).
 *
 * Conventions for every call:
 *  - All data pointers are DEVICE pointers unless the comment says host.
 *    The caller allocates every device buffer; the library never allocates
 *    device memory (its only device memory of its own is the fixed scratch
 *    array of kvq_decode_attention_noalloc, loaded with the library).  Host
 *    handles (kvq_cache) are malloc'ed by kvq_cache_init and released by
 *    kvq_cache_free.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work and return; results are valid once the stream reaches
 *    them.  Calls on one cache or one output buffer must be ordered by the
 *    caller (same stream or explicit events).
 *  - Argument errors return at once and enqueue nothing.  Data errors
 *    (NaN/Inf input) are found on the device: the kernel sets a sticky flag
 *    and the outputs are unspecified; read the flag with kvq_poll_error or
 *    kvq_cache_check.
 *  - Outputs are deterministic: equal inputs give equal bytes.
 *  - Packed codes: offset binary u = code + 2^(b-1), b bits each,
 *    LSB-first in little-endian uint32 words, floor(32/b) fields per word,
 *    one row per token padded to whole words ("words(n, b)" below), unused
 *    bits zero.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_E_ARG = 1,        /* invalid argument; nothing was enqueued */
  KVQ_E_CAPACITY = 2,   /* append would exceed the cache's max_tokens */
  KVQ_E_NONFINITE = 3,  /* a kernel saw NaN/Inf input (sticky flag set) */
  KVQ_E_HIP = 4,        /* a HIP runtime call failed */
  KVQ_E_POISONED = 5,   /* cache saw NaN/Inf earlier; re-initialise it */
  KVQ_E_UNSUPPORTED = 6, /* valid request the library does not implement */
  KVQ_E_SCRATCH = 7      /* kvq_decode_attention_noalloc: the split partials
                            would not fit the library's fixed scratch */
} kvq_status;

typedef enum { KVQ_F32 = 0, KVQ_F16 = 1 } kvq_dtype;
typedef enum { KVQ_PER_CHANNEL = 0, KVQ_PER_TOKEN = 1 } kvq_axis;

/* Layout of value codes inside a cache (kvq_kv_view.v_layout). */
typedef enum {
  KVQ_V_ROWS = 0,   /* one packed row per token, as described above */
  KVQ_V_TILE32 = 1  /* 32-token tiles ordered for the matrix-core decode;
                       kvq_export converts to rows */
} kvq_v_layout;

/* Number of uint32 words of one packed row of n fields of b bits. */
int kvq_words(int n_fields, int bits);

/* ---------------------------------------------------------------------
 * Stateless quantizers.
 * ------------------------------------------------------------------ */

/* Per-channel key quantization ("KVQuant ...", table "Measured effects":
 * keys per channel; "KV quantization axes ...", "What rows and columns
 * mean": the rule and the (1, D) channel-scale shape).
 *   k       [n_mats][n_tok][d], dtype KVQ_F32 or KVQ_F16
 *   codes   [n_mats][n_tok][kvq_words(d, bits)] uint32 (written)
 *   scales  [n_mats][ceil(n_tok / group_tok)][d] float32 (written); the
 *           group of channel c and token t is t / group_tok; a final partial
 *           group uses its own absmax.
 *   err_flag  device uint32, nullable; bit 0 is OR-ed in on NaN/Inf.
 * Requires 1 <= d <= 256, group_tok >= 1, bits in {8,4,3,2}, 4-byte aligned
 * pointers.  n_mats or n_tok == 0 is a no-op.                           */
kvq_status kvq_quantize_k(const void* k, int dtype, int64_t n_mats,
                          int64_t n_tok, int d, int bits, int group_tok,
                          uint32_t* codes, float* scales, uint32_t* err_flag,
                          void* stream);

/* Per-token value quantization (same sources; token-scale shape (N, 1)
 * generalised to one scale per group of group_ch channels).
 *   v       [n_mats][n_tok][d]
 *   codes   [n_mats][n_tok][kvq_words(d, bits)]
 *   scales  [n_mats][n_tok][d / group_ch]
 * Requires group_ch to divide d, 1 <= d <= 256.                          */
kvq_status kvq_quantize_v(const void* v, int dtype, int64_t n_mats,
                          int64_t n_tok, int d, int bits, int group_ch,
                          uint32_t* codes, float* scales, uint32_t* err_flag,
                          void* stream);

/* Reconstruction x_hat = fl32(code * scale) ("KV quantization axes ...",
 * "What rows and columns mean").
 *   codes [n_mats][n_tok][kvq_words(d, bits)]; out [n_mats][n_tok][d] f32.
 *   axis KVQ_PER_CHANNEL: scales [n_mats][ceil(n_tok/group)][d];
 *   axis KVQ_PER_TOKEN:   scales [n_mats][n_tok][d/group].               */
kvq_status kvq_dequant(const uint32_t* codes, const float* scales,
                       int64_t n_mats, int64_t n_tok, int d, int bits,
                       int axis, int group, float* out, void* stream);

/* Key rotation ("Quantize What Counts: More for Keys, Less for Values",
 * rotation integration: rotating the keys alone; "Statistical Inference
 * and Quality Measures of KV Cache Quantisations Inspired by TurboQuant",
 * the Walsh-Hadamard step of the KQV scheme).  Row by row,
 *   out[r][:] = H in[r][:] / sqrt(d),
 * H the Sylvester Walsh-Hadamard matrix of order d (a power of two,
 * 1 <= d <= 256): orthonormal and its own inverse, so q . k = (Hq) . (Hk)
 * and rotating the keys before kvq_append and the queries before
 * kvq_decode_attention leaves the scores unchanged.  Computed in float32
 * by the fast transform (stages h = 1, 2, 4, ..., d/2: the pair
 * (x[i], x[i+h]), bit h of i clear, becomes (x[i] + x[i+h], x[i] - x[i+h]))
 * and one multiply by float32(1/sqrt(d)); a KVQ_F16 output is rounded to
 * nearest even.  The result is fixed bit for bit.
 *   in  [n_rows][d] KVQ_F16 or KVQ_F32;  out [n_rows][d] KVQ_F16 or KVQ_F32
 * out may equal in (same dtype); other overlaps are not allowed.  Pointers
 * aligned to their element size; 16-byte rows take the fast path.
 * KVQ_E_ARG for other d, dtypes or a null pointer with n_rows > 0.       */
kvq_status kvq_hadamard(const void* in, int in_dtype, void* out,
                        int out_dtype, int64_t n_rows, int d, void* stream);

/* ---------------------------------------------------------------------
 * Cache.
 * ------------------------------------------------------------------ */

typedef struct {
  int32_t batch;      /* B */
  int32_t kv_heads;   /* Hkv */
  int32_t head_dim;   /* D, 1..256 */
  int32_t k_bits;     /* uniform keys: 8|4|3|2 (ignored when k_mixed) */
  int32_t v_bits;     /* 8|4|3|2 */
  int32_t group_tok;  /* G: key group, tokens */
  int32_t group_ch;   /* Gv: value group, channels; divides D */
  int32_t residual;   /* R: fp16 tail capacity, a positive multiple of G */
  int32_t sink;       /* S: leading tokens kept in fp16 */
  int32_t k_mixed;    /* 1: MixKVQ key classes bf16 / int4 / int2 */
  int32_t n_bf16;     /* mixed: channels kept bf16 per group */
  int32_t n_int4;     /* mixed: channels at int4 per group (rest int2) */
  int64_t max_tokens; /* capacity, tokens per (batch, KV head) */
} kvq_cache_cfg;

typedef struct kvq_cache kvq_cache;

/* Device bytes the cache needs for cfg (0 if cfg is invalid). */
size_t kvq_cache_bytes(const kvq_cache_cfg* cfg);

/* Bind a cache to a caller-owned device buffer of kvq_cache_bytes(cfg)
 * bytes (256-byte aligned).  n_tokens == 0 starts empty: the error flag is
 * cleared and the salience intensity set to 1 for every channel (ranking by
 * key scale alone until kvq_salience_select).  n_tokens > 0 re-attaches a
 * buffer that already holds that many tokens (checkpoint resume: the buffer
 * is the whole state).  *out receives a host handle.                    */
kvq_status kvq_cache_init(const kvq_cache_cfg* cfg, void* dev_buf,
                          size_t bytes, int64_t n_tokens, kvq_cache** out,
                          void* stream);

/* Release the host handle (the device buffer stays the caller's). */
void kvq_cache_free(kvq_cache* c);

/* Tokens appended so far (host counter). */
int64_t kvq_cache_tokens(const kvq_cache* c);

/* Append n_new tokens of every (batch, KV head) stream ("MixKVQ ...",
 * Figure 4; "KVQuant ...", summary):
 *   k_new, v_new  [B][Hkv][n_new][D] float16
 * The first S tokens ever appended go to the fp16 sink.  Later tokens join
 * the fp16 tail; whenever the tail would exceed R tokens, its oldest G
 * tokens are quantized as one key group (per channel; MixKVQ classes when
 * k_mixed) and per token for values.  Returns KVQ_E_CAPACITY if the cache
 * would exceed max_tokens, KVQ_E_POISONED after a data error.          */
kvq_status kvq_append(kvq_cache* c, const void* k_new, const void* v_new,
                      int dtype, int64_t n_new, void* stream);

/* MixKVQ query intensity ("MixKVQ ...", Figure 3; refreshed per the
 * Figure 4 window):
 *   q_win  [B][w_rows][n_q_heads][D] float16, the last w_rows query rows.
 * I[b][kvh][d] = sum over the rows and the query heads kvh*g .. kvh*g+g-1
 * (g = n_q_heads / Hkv) of |q|, in float64 (exact).  Applies to every later
 * key-group flush.  Requires k_mixed; n_q_heads / Hkv <= 1024
 * (else KVQ_E_UNSUPPORTED).                                            */
kvq_status kvq_salience_select(kvq_cache* c, const void* q_win, int dtype,
                               int w_rows, int n_q_heads, void* stream);

/* Sync `stream`, read the cache's sticky data-error flag; on NaN/Inf the
 * cache is poisoned (every later call returns KVQ_E_POISONED) and
 * KVQ_E_NONFINITE is returned.                                          */
kvq_status kvq_cache_check(kvq_cache* c, void* stream);

/* Read-only description of a cache's device arrays.  Strides are in
 * elements of the array's type, per (batch, KV head) stream s = b*Hkv + h.
 * A view may also be filled in by hand from kvq_quantize_k/v outputs
 * (rows layout, uniform keys, no sink or tail).                          */
typedef struct {
  int32_t batch, kv_heads, head_dim;
  int32_t k_bits, v_bits, group_tok, group_ch;
  int32_t k_mixed, n_bf16, n_int4;
  int32_t v_layout;   /* kvq_v_layout */
  int32_t residual;   /* ring capacity of the tail arrays */
  int64_t n_sink;     /* fp16 sink tokens */
  int64_t n_quant;    /* quantized tokens (past-sink indices 0..n_quant-1) */
  int64_t n_tail;     /* fp16 tail tokens; past-sink index p sits in ring
                         row p % residual */
  const uint16_t* sink_k; const uint16_t* sink_v; int64_t sink_stride;
  const uint16_t* tail_k; const uint16_t* tail_v; int64_t tail_stride;
  /* uniform keys: codes [n_quant][kvq_words(D, k_bits)], scales [groups][D] */
  const uint32_t* k_codes; int64_t k_codes_stride;
  const float* k_scales; int64_t k_scales_stride;
  /* per key group: the largest channel scale (for bf16 channels of mixed
     keys, the largest |K|), a bound used to keep matrix-core operands in
     range; nullable (the matrix-core path then is not used) */
  const float* k_gmax; int64_t k_gmax_stride;
  /* mixed keys: per group, k_pos[d] = position of channel d in the order
     [bf16 channels | int4 channels | int2 channels], each ascending;
     k_scales [groups][n_int4 + n_int2] in that order;
     bf16 [n_quant][n_bf16]; int4 [n_quant][words(n_int4,4)];
     int2 [n_quant][words(n_int2,2)] */
  const uint8_t* k_pos; int64_t k_pos_stride;
  const uint16_t* k_bf16; int64_t k_bf16_stride;
  const uint32_t* k_int4; int64_t k_int4_stride;
  const uint32_t* k_int2; int64_t k_int2_stride;
  /* values: codes (v_layout), scales [n_quant][D / group_ch] */
  const uint32_t* v_codes; int64_t v_codes_stride;
  const float* v_scales; int64_t v_scales_stride;
  uint32_t* err_flag;   /* the cache's sticky data-error flag */
} kvq_kv_view;

kvq_status kvq_cache_view(const kvq_cache* c, kvq_kv_view* v);

/* Canonical dense copies of a cache (tests, audits, checkpoints).  Every
 * pointer is a device buffer; shapes with ns, nq, nt = n_sink, n_quant,
 * n_tail and ng = nq / G:
 *   sink_k, sink_v [B][Hkv][ns][D] f16;  tail_k, tail_v [B][Hkv][nt][D]
 *   f16 in token order; v_codes [B][Hkv][nq][words(D, v_bits)] rows;
 *   v_scales [B][Hkv][nq][D/Gv];
 *   uniform: k_codes [B][Hkv][nq][words(D, k_bits)], k_scales [..][ng][D];
 *   mixed: k_class [B][Hkv][ng][D] u8 (0 bf16, 1 int4, 2 int2), k_bf16,
 *   k_int4, k_int2, k_scales as in kvq_kv_view, densely per stream.
 * Pointers the layout does not use may be NULL.                         */
typedef struct {
  void* sink_k; void* sink_v; void* tail_k; void* tail_v;
  uint32_t* k_codes; float* k_scales;
  uint8_t* k_class; uint16_t* k_bf16; uint32_t* k_int4; uint32_t* k_int2;
  uint32_t* v_codes; float* v_scales;
} kvq_export_bufs;

kvq_status kvq_export(const kvq_kv_view* v, const kvq_export_bufs* out,
                      void* stream);

/* ---------------------------------------------------------------------
 * Decode attention.
 * ------------------------------------------------------------------ */

enum {
  KVQ_DECODE_AUTO = 0,     /* matrix-core kernel when the view allows it */
  KVQ_DECODE_GENERIC = 1   /* always the general vector kernel */
};

/* Bytes of the split workspace for n_splits (0 = automatic), enough for
 * kvq_decode_attention and kvq_decode_attention_rope alike. */
size_t kvq_decode_workspace_bytes(const kvq_kv_view* v, int n_q_heads,
                                  int n_splits);

/* Decode attention over every token of the view ("KV quantization axes
 * ...", section "Separate the two error paths"; "KVQuant ...", key
 * results: key and value matvecs over the quantized cache):
 *   q    [B][n_q_heads][D], KVQ_F16 or KVQ_F32
 *   out  [B][n_q_heads][D] float32 (written)
 * Query head h reads KV head h / (n_q_heads / Hkv).  The context is split
 * into n_splits ranges (0 = automatic) whose softmax partials are merged
 * with the log-sum-exp rule.  workspace >= kvq_decode_workspace_bytes.
 * The matrix-core kernel also needs q 16-byte aligned; otherwise, and for
 * views it does not cover, KVQ_DECODE_AUTO runs the general kernel.
 * An empty view (no tokens) is KVQ_E_ARG.                               */
kvq_status kvq_decode_attention(const kvq_kv_view* v, const void* q,
                                int dtype, int n_q_heads, float sm_scale,
                                float* out, int n_splits, int flags,
                                void* workspace, size_t ws_bytes,
                                void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode as kvq_decode_attention, with the split partials in a fixed array
 * of KVQ_NOALLOC_SCRATCH_BYTES of the library's own device memory (one per
 * GPU, held until the process ends) instead of a caller workspace.  The
 * caller still passes q and out.  The call allocates nothing.  It needs
 * kvq_decode_workspace_bytes(v, n_q_heads, n_splits) <= the scratch size,
 * else KVQ_E_SCRATCH and nothing is enqueued.  Every call on one GPU shares
 * its array: calls that overlap on one GPU (several streams, or threads
 * without ordering) race and must be serialized by the caller.            */
#define KVQ_NOALLOC_SCRATCH_BYTES (16u << 20)
kvq_status kvq_decode_attention_noalloc(const kvq_kv_view* v, const void* q,
                                        int dtype, int n_q_heads,
                                        float sm_scale, float* out,
                                        int n_splits, int flags, void* stream);

/* Keys cached before the rotary position embedding ("KVQuant: Towards 10
 * Million Context Length LLM Inference with KV Cache Quantization",
 * "Approach" and the table of measured effects: per-channel key
 * quantization before RoPE).  Frequency f = 0 .. D/2 - 1 turns by
 * theta_f = base^(-2f/D) radians per position; at position p the channel
 * pair (a, b) of frequency f maps (x_a, x_b) to
 * (x_a cos - x_b sin, x_a sin + x_b cos) with the angle p * theta_f.      */
enum {
  KVQ_ROPE_HALF = 0,        /* pairs channel f with channel f + D/2 */
  KVQ_ROPE_INTERLEAVED = 1  /* pairs channel 2f with channel 2f + 1 */
};

typedef struct {
  double base;       /* > 0, finite (10000 in the usual models) */
  int32_t pairing;   /* KVQ_ROPE_HALF or KVQ_ROPE_INTERLEAVED */
  int32_t reserved;  /* 0 */
  int64_t pos0;      /* position of cache-order token 0, >= 0 */
} kvq_rope;

/* Decode attention as kvq_decode_attention, over a cache whose keys (sink,
 * quantized groups and tail alike) were appended before the rotary
 * embedding: the dequantized key of cache-order token i is rotated at
 * position pos0 + i before its product with q.  q is the query already
 * rotated at its own position.  D must be even and pos0 + tokens <= 2^40
 * (else KVQ_E_ARG).  Uniform int8/int4/int2 keys with int4/int2 value
 * tiles, D = 128, G a multiple of 32, Gv >= 16 and 1 to 8 query heads
 * per KV head run a dedicated kernel (one launch per pair of query heads
 * of a KV head, the last one alone when that count is odd); every other
 * view (and
 * KVQ_DECODE_GENERIC) the general kernel.  The workspace is sized by
 * kvq_decode_workspace_bytes.  Angles are reduced in float64 and the
 * cosines and sines evaluated in float32.                                */
kvq_status kvq_decode_attention_rope(const kvq_kv_view* v, const kvq_rope* rope,
                                     const void* q, int dtype, int n_q_heads,
                                     float sm_scale, float* out, int n_splits,
                                     int flags, void* workspace, size_t ws_bytes,
                                     void* stream);

/* ---------------------------------------------------------------------
 * Extended formats: the non-uniform codebook datatype with dense-and-sparse
 * outliers, and the value-side 1-bit residual sketch.
 * ------------------------------------------------------------------ */

/* Non-uniform codebook datatype with per-vector dense-and-sparse outliers
 * ("KVQuant: Towards 10 Million Context Length LLM Inference with KV Cache
 * Quantization", summary and "Approach": nuqX datatypes and per-vector
 * dense-and-sparse outlier isolation; table "Measured effects reported in
 * the paper": 1% outliers, per-vector thresholds, keys per channel and
 * values per token).  A vector is what one scale covers: for keys one
 * channel of a group of group_tok tokens, for values one group of group_ch
 * channels of one token.  In each vector the n_out entries of largest
 * magnitude (ties to the lower position) are kept exactly; the rest (those
 * entries set to 0) get scale = max|x| / max|lut| (IEEE float32 division;
 * 1 for an all-zero rest) and per entry the index of the codebook level
 * nearest to fl32(x / scale) (ties to the lower level).  Reconstruction:
 * lut[code] * scale plus the kept entries.
 *   k, v      [n_mats][n_tok][d] float16 (device)
 *   lut       HOST float32 [2^bits], bits 2, 3 or 4: strictly ascending
 *             fp16 numbers including 0 (a synthetic or calibrated codebook)
 *   codes     [n_mats][n_tok][kvq_words(d, bits)] uint32: level indices,
 *             LSB-first (plain indices, no offset)
 *   scales    keys [n_mats][ceil(n_tok / group_tok)][d];
 *             values [n_mats][n_tok][d / group_ch] float32
 *   outliers  uint32 (position in the vector << 16 | fp16 bits of the
 *             value), positions ascending; keys
 *             [n_mats][ceil(n_tok/group_tok)][d][n_out], values
 *             [n_mats][n_tok][d / group_ch][n_out]; slots past a vector
 *             shorter than n_out hold 0
 * Requires 1 <= d <= 256, 0 <= n_out <= 16, n_out < 65536 entries per
 * vector, keys group_tok * d <= 32768; else KVQ_E_ARG.  NaN/Inf input sets
 * bit 0 of err_flag (nullable).                                          */
kvq_status kvq_quantize_nuq_k(const void* k, int64_t n_mats, int64_t n_tok, int d, int bits,
                              int group_tok, const float* lut, int n_out, uint32_t* codes,
                              float* scales, uint32_t* outliers, uint32_t* err_flag,
                              void* stream);
kvq_status kvq_quantize_nuq_v(const void* v, int64_t n_mats, int64_t n_tok, int d, int bits,
                              int group_ch, const float* lut, int n_out, uint32_t* codes,
                              float* scales, uint32_t* outliers, uint32_t* err_flag,
                              void* stream);

/* Values with the 1-bit residual sketch of the KQV scheme ("Statistical
 * Inference and Quality Measures of KV Cache Quantisations Inspired by
 * TurboQuant", "Quantization Schemes": values rotated by a Walsh-Hadamard
 * transform, scalar-quantized with n - 1 bits, plus a 1-bit QJL sketch of
 * the residual; "1. Theoretical Proof of QJL Harm on Keys": the sketch is
 * an unbiased estimator).  v is the already rotated value (kvq_hadamard);
 * per token the symmetric rule of kvq_quantize_v with `bits` bits in groups
 * of group_ch channels, then the residual r = v - fl32(code * scale) (exact
 * in float32), sketch bit i = [<S_i, r> >= 0] for the m rows of S (dot
 * products in float64), and rnorm = ||r||_2 (float64, rounded to float32).
 *   v       [n_mats][n_tok][d] KVQ_F16 or KVQ_F32
 *   jl      [m][d] float32 device: the Gaussian projection S (an input;
 *           one matrix for the whole cache)
 *   codes   [n_mats][n_tok][kvq_words(d, bits)]; scales [..][d/group_ch]
 *   sketch  [n_mats][n_tok][m / 32] uint32 (bit i of word w: row 32 w + i)
 *   rnorm   [n_mats][n_tok] float32
 * Requires m a multiple of 32, 32 <= m <= 256, 1 <= d <= 256.            */
kvq_status kvq_quantize_v_qjl(const void* v, int dtype, int64_t n_mats, int64_t n_tok, int d,
                              int bits, int group_ch, const float* jl, int m, uint32_t* codes,
                              float* scales, uint32_t* sketch, float* rnorm,
                              uint32_t* err_flag, void* stream);

/* A view over the outputs of the quantizers above (and kvq_quantize_k/v),
 * rows layout, per (batch, KV head) stream s = b * kv_heads + h (strides
 * in elements of each array's type).  Keys: codes with per-channel scales
 * per group of group_tok tokens, symmetric (k_nuq 0, k_bits 8|4|3|2) or
 * codebook (k_nuq 1, k_bits 2|3|4, k_lut, k_n_out outliers per vector).
 * Values: per-token scales per group_ch channels, symmetric or codebook
 * likewise, optionally with the residual sketch (v_qjl 1: v_sketch,
 * v_rnorm, jl [qjl_m][head_dim]); v_rotated 1 turns the output back with
 * the Walsh-Hadamard transform (values stored rotated; head_dim a power of
 * two).  Host-side codebooks are copied into the call.                   */
typedef struct {
  int32_t batch, kv_heads, head_dim, reserved0;
  int64_t n_tok;
  int32_t k_bits, group_tok, k_nuq, k_n_out;
  const uint32_t* k_codes; int64_t k_codes_stride;
  const float* k_scales; int64_t k_scales_stride;
  const uint32_t* k_outliers; int64_t k_outliers_stride;
  float k_lut[16];
  int32_t v_bits, group_ch, v_nuq, v_n_out;
  const uint32_t* v_codes; int64_t v_codes_stride;
  const float* v_scales; int64_t v_scales_stride;
  const uint32_t* v_outliers; int64_t v_outliers_stride;
  float v_lut[16];
  int32_t v_qjl, qjl_m, v_rotated, reserved1;
  const uint32_t* v_sketch; int64_t v_sketch_stride;
  const float* v_rnorm; int64_t v_rnorm_stride;
  const float* jl;
} kvq_ext_view;

/* Workspace bytes of kvq_decode_attention_ext (0 if the view is invalid). */
size_t kvq_decode_ext_workspace_bytes(const kvq_ext_view* v, int n_q_heads, int n_splits);

/* Decode attention over an extended view: out = softmax(q K_hat^T *
 * sm_scale) V_hat per query head ("KV quantization axes ...", "Separate the
 * two error paths"), K_hat and V_hat the reconstructions above (the sketch
 * contributes sqrt(pi/2)/m * rnorm * S^T b per token; rotated values are
 * turned back).  q [B][n_q_heads][D] KVQ_F16 or KVQ_F32; out float32.
 * Requires head_dim 32, 64 or 128, group_tok a multiple of 32, at most 8
 * query heads per KV head, n_splits <= 4096, n_tok >= 1 (else KVQ_E_ARG). */
kvq_status kvq_decode_attention_ext(const kvq_ext_view* v, const void* q, int dtype,
                                    int n_q_heads, float sm_scale, float* out, int n_splits,
                                    void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Errors and utilities.
 * ------------------------------------------------------------------ */

/* Sync `stream`, then read a device error flag: KVQ_E_NONFINITE if set. */
kvq_status kvq_poll_error(const uint32_t* err_flag, void* stream);

const char* kvq_strerror(kvq_status s);

/* Fill a device uint32 buffer with a value (a kernel, so the call is safe
 * inside captured graphs). */
kvq_status kvq_fill_u32(uint32_t* dst, uint32_t value, int64_t n,
                        void* stream);

/* Measured streaming-read ceiling: one launch of a plain read kernel over
 * `bytes` (a multiple of 16) of device memory at src (16-byte aligned);
 * each of the 8192 workgroups reads a contiguous share with nontemporal
 * 16-byte loads and writes the XOR of its words to sink (8192 uint32,
 * device).  Time it with events to compare the decode kernel with what a
 * bare read reaches.                                                   */
kvq_status kvq_stream_read(const void* src, int64_t bytes, uint32_t* sink,
                           void* stream);

/* Seeded synthetic fp16 data for benchmarks too large to draw on the host:
 * element (head, token, channel) of `tensor` (0 K, 1 V, 2 q) in `layer` is
 * the counter-th output of a SplitMix64 stream (Steele, Lea and Flood,
 * OOPSLA 2014) seeded with `seed`, counter = ((((tensor*256 + layer)*256 +
 * head) << 32) + token)*256 + channel; its four 16-bit lanes are summed,
 * centred at 131070, multiplied by the float32 nearest 1/sqrt((2^32-1)/3)
 * and rounded to fp16.
 *   out [n_heads][n_tok][d] with head stride head_stride halves.        */
kvq_status kvq_synth_normal_f16(void* out, uint64_t seed, int tensor,
                                int layer, int head0, int n_heads,
                                int64_t t0, int64_t n_tok, int d,
                                int64_t head_stride, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
