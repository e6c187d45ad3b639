// Internal declarations of libkvq: host cache handle, layout helpers shared
// by host and device code, and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"
#include "rope_math.h"

namespace kvq {

constexpr int kMaxD = 256;       // head_dim limit of every kernel
constexpr int kTile = 32;        // tokens per value tile / decode tile

__host__ __device__ inline int qmax_of(int bits) { return (1 << (bits - 1)) - 1; }
__host__ __device__ inline int fields_per_word(int bits) { return 32 / bits; }
__host__ __device__ inline int words_of(int n, int bits) {
  int pw = 32 / bits;
  return (n + pw - 1) / pw;
}

// ---------------------------------------------------------------------------
// Value tile layout (KVQ_V_TILE32).  A tile holds 32 consecutive quantized
// tokens x D channels at vb in {2, 4} bits, i.e. D*vb uint32 words.  It is
// ordered so that lane l = 16*q + m of a 64-wide wavefront finds, in
// contiguous 16-byte chunks, the codes of channel 16*jb + m (for every
// channel block jb) at the eight tokens
//     tau(q, s) = (s % 4) + 4*q + 16*(s / 4),   s = 0..7,
// which is the token order a 16x16 matrix-core score tile produces.  Within
// a lane's words, the two codes of slot pair i (slots 2i, 2i+1) of one block
// sit 16 bits apart, so one AND-OR turns them into two fp16 numbers.
//   vb = 2: word w holds blocks 2w and 2w+1; field p (bits 2p..2p+1):
//           even block: p = i + 8e, odd block: p = 4 + i + 8e (slot 2i+e)
//   vb = 4: word w holds block w; nibble p = i + 4e (slot 2i+e)
// Lane words are stored in chunks of C = min(4, D*vb/64) words: word w of
// lane l is at ((w / C) * 64 + l) * C + (w % C) within the tile.
// ---------------------------------------------------------------------------
__host__ __device__ inline int v_tile_lane_words(int D, int vb) { return D * vb / 64; }

__host__ __device__ inline void v_tile_pos(int64_t t, int d, int D, int vb,
                                           int64_t* word, int* bit) {
  int64_t T = t >> 5;
  int tau = (int)(t & 31);
  int q = (tau & 15) >> 2;
  int s = (tau & 3) + ((tau >> 4) << 2);
  int jb = d >> 4, m = d & 15, l = q * 16 + m;
  int Wl = v_tile_lane_words(D, vb);
  int C = Wl < 4 ? Wl : 4;
  int i = s >> 1, e = s & 1;
  int w, p;
  if (vb == 2) {
    w = jb >> 1;
    p = (jb & 1) ? (4 + i + 8 * e) : (i + 8 * e);
    *bit = 2 * p;
  } else {
    w = jb;
    p = i + 4 * e;
    *bit = 4 * p;
  }
  *word = T * (int64_t)(D * vb) + (int64_t)(((w / C) * 64 + l) * C + (w % C));
}

// Inverse: field p of lane word w of lane l -> (token within tile, channel).
__host__ __device__ inline void v_tile_field(int l, int w, int p, int vb,
                                             int* tau, int* d) {
  int q = l >> 4, m = l & 15;
  int jb, s;
  if (vb == 2) {
    int e = p >> 3, r = p & 7, odd = r >> 2, i = r & 3;
    jb = 2 * w + odd;
    s = 2 * i + e;
  } else {
    int e = p >> 2, i = p & 3;
    jb = w;
    s = 2 * i + e;
  }
  *tau = (s & 3) + 4 * q + 16 * (s >> 2);
  *d = 16 * jb + m;
}

__host__ __device__ inline bool v_tile_ok(int D, int vb, int G) {
  return (vb == 2 || vb == 4) && D % 32 == 0 && D <= kMaxD && G % kTile == 0;
}

// ---------------------------------------------------------------------------
// Device-side description of one cache, passed by value to kernels.
// ---------------------------------------------------------------------------
struct CacheDev {
  int B, H, D, k_bits, v_bits, G, Gv, R, S, mixed, n_bf16, n_int4, v_layout;
  uint32_t* err;
  double* I;                      // [B*H][D]
  uint16_t* sink_k; uint16_t* sink_v; int64_t s_sink;
  uint16_t* tail_k; uint16_t* tail_v; int64_t s_tail;
  uint32_t* k_codes; int64_t s_k_codes;
  float* k_scales; int64_t s_k_scales;
  float* k_gmax; int64_t s_k_gmax;
  uint8_t* k_pos; int64_t s_k_pos;
  uint16_t* k_bf16; int64_t s_k_bf16;
  uint32_t* k_int4; int64_t s_k_int4;
  uint32_t* k_int2; int64_t s_k_int2;
  uint32_t* v_codes; int64_t s_v_codes;
  float* v_scales; int64_t s_v_scales;
};

// ---------------------------------------------------------------------------
// Launchers (quant.hip, decode*.hip).  Each returns the launch status.
// ---------------------------------------------------------------------------
hipError_t launch_quantize_k(const void* k, int f16, int64_t n_mats,
                             int64_t n_tok, int d, int bits, int G,
                             uint32_t* codes, float* scales, uint32_t* err,
                             hipStream_t s);
hipError_t launch_quantize_v(const void* v, int f16, int64_t n_mats,
                             int64_t n_tok, int d, int bits, int Gv,
                             uint32_t* codes, float* scales, uint32_t* err,
                             hipStream_t s);
hipError_t launch_dequant(const uint32_t* codes, const float* scales,
                          int64_t n_mats, int64_t n_tok, int d, int bits,
                          int axis, int group, float* out, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* dst, uint32_t v, int64_t n, hipStream_t s);
constexpr int kStreamReadBlocks = 8192;
hipError_t launch_hadamard(const void* in, int in_f16, void* out, int out_f16, int64_t n_rows,
                           int d, hipStream_t s);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_fill_f64(double* dst, double v, int64_t n, hipStream_t s);

// Append: copy rows of the new tokens to the sink and to tail ring rows.
//   sink: input tokens [0, take) -> sink rows [ns_old, ns_old + take)
//   tail: input tokens [in_lo, in_hi) -> past-sink indices p = p_lo + (i - in_lo),
//         ring row p % R
hipError_t launch_append_rows(const CacheDev& c, const uint16_t* k_in,
                              const uint16_t* v_in, int64_t n_new,
                              int64_t ns_old, int64_t take, int64_t in_lo,
                              int64_t in_hi, int64_t p_lo, hipStream_t s);
// Flush n_groups key groups.  Group f covers past-sink indices
// p0 + f*G .. p0 + f*G + G - 1 with p0 = nq_old; index p reads the ring row
// p % R when p < nq_old + nt_old, else input token take + p - nq_old - nt_old.
hipError_t launch_flush(const CacheDev& c, const uint16_t* k_in,
                        const uint16_t* v_in, int64_t n_new, int64_t take,
                        int64_t nq_old, int64_t nt_old, int64_t n_groups,
                        hipStream_t s);
hipError_t launch_salience(const CacheDev& c, const uint16_t* q_win, int w_rows,
                           int n_q_heads, hipStream_t s);
hipError_t launch_export(const kvq_kv_view& v, const kvq_export_bufs& o,
                         hipStream_t s);
hipError_t launch_synth(uint16_t* out, uint64_t seed, int tensor, int layer,
                        int head0, int n_heads, int64_t t0, int64_t n_tok,
                        int d, int64_t head_stride, hipStream_t s);

// Decode.  partials: [B][Hq][n_parts][D + 2] float (m in log2 units, l, o).
hipError_t launch_decode_generic(const kvq_kv_view& v, const void* q, int f16,
                                 int Hq, float sm_scale, float* partials,
                                 int n_parts, hipStream_t s);
// Tokens [range_lo, range_hi) split into n_parts partials written at slots
// part_offset .. of part_stride per head.  Range index i is cache-order
// token i below gap_at and token i + gap_len from there on (so the sink and
// the tail, with the quantized tokens between them skipped, make one range).
hipError_t launch_decode_generic_range(const kvq_kv_view& v, const void* q, int f16,
                                       int Hq, float sm_scale, float* partials,
                                       int64_t range_lo, int64_t range_hi, int n_parts,
                                       int part_offset, int part_stride, const RopeDev* rope,
                                       hipStream_t s, int64_t gap_at = INT64_MAX,
                                       int64_t gap_len = 0);
bool mfma_decode_eligible(const kvq_kv_view& v, int Hq);
int mfma_decode_parts(const kvq_kv_view& v, int Hq, int n_splits);
hipError_t launch_decode_mfma(const kvq_kv_view& v, const void* q, int f16,
                              int Hq, float sm_scale, float* partials,
                              int n_splits, hipStream_t s);
// Rotary decode over keys cached before the embedding (decode_rope.hip).
// The dedicated kernel covers uniform int8/int4/int2 keys, int4/int2 value
// tiles, D = 128, G a multiple of 32, Gv >= 16 and 1 to 8 query heads per
// KV head; it writes rope_fast_parts(...) partials for the quantized
// tokens and rope_fp16_parts(v) more (sink, then tail; 32 tokens each) from
// the general kernel.
bool rope_fast_eligible(const kvq_kv_view& v, int Hq);
int rope_fast_parts(const kvq_kv_view& v, int Hq, int n_splits);
int rope_fp16_parts(const kvq_kv_view& v);
hipError_t launch_decode_rope(const kvq_kv_view& v, const void* q, int f16, int Hq,
                              float sm_scale, const RopeDev& rope, float* partials,
                              int n_parts, hipStream_t s);
hipError_t launch_merge(const float* partials, int B, int Hq, int D,
                        int n_parts, float* out, hipStream_t s);
// Codebook of the non-uniform datatype as kernel arguments: levels
// (ascending fp16 numbers including 0), the midpoints between neighbours
// (exact in float32) and the largest level magnitude.
struct ExtLut {
  float lvl[16];
  float mid[15];
  float absmax;
  int n;
};
hipError_t launch_quantize_nuq_k(const uint16_t* k, int64_t n_mats, int64_t n_tok, int d,
                                 int bits, int G, const ExtLut& L, int n_out, uint32_t* codes,
                                 float* scales, uint32_t* outl, uint32_t* err, hipStream_t s);
hipError_t launch_quantize_nuq_v(const uint16_t* v, int64_t n_mats, int64_t n_tok, int d,
                                 int bits, int Gv, const ExtLut& L, int n_out, uint32_t* codes,
                                 float* scales, uint32_t* outl, uint32_t* err, hipStream_t s);
hipError_t launch_quantize_v_qjl(const void* v, int f16, int64_t n_mats, int64_t n_tok, int d,
                                 int bits, int Gv, const float* S, int m, uint32_t* codes,
                                 float* scales, uint32_t* sketch, float* rnorm, uint32_t* err,
                                 hipStream_t s);
size_t ext_decode_lds(const kvq_ext_view& v, int Hq);
int ext_decode_parts(const kvq_ext_view& v, int Hq, int n_splits);
// Decode over an extended view: partials [B][Hq][n_parts][D + 2 + M], then
// the merge (with the sketch term and the inverse rotation) into out.
hipError_t launch_decode_ext(const kvq_ext_view& v, const ExtLut& lk, const ExtLut& lv,
                             const void* q, int f16, int Hq, float sm_scale, float* partials,
                             int n_parts, float* out, hipStream_t s);

// kvq_decode_attention with the partials in `workspace` (api.cpp); the
// scratch-backed entry point calls it too.
kvq_status decode_attention_impl(const kvq_kv_view* v, const void* q, int dtype, int n_q_heads,
                                 float sm_scale, float* out, int n_splits, int flags,
                                 void* workspace, size_t ws_bytes, void* stream);

}  // namespace kvq
