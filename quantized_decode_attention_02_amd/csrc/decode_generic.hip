// General decode attention of libkvq (any bit width, layout, D <= 256,
// mixed keys) and the cross-split merge.
//
// Computes, per query head h reading KV head h / g, the stable softmax of
// q . k_hat_t * sm_scale over every cached token and the weighted sum of
// v_hat_t ("KV quantization axes ...", section "Separate the two error
// paths").  Scores are kept in log2 units (q pre-multiplied by
// sm_scale * log2(e)), so exp2 replaces exp.  Each split writes a partial
// (m, l, o): m the largest score, l = sum 2^(s - m), o = sum 2^(s - m) v_hat;
// the merge combines partials with the log-sum-exp rule.
//
// With a rotary embedding (keys cached before it), the key of cache-order
// token i is turned at position pos0 + i before the product with q (see
// rope_math.h); that path computes every cosine and sine it uses and is
// meant for the views the dedicated kernel does not cover, and for the
// few fp16 sink and tail tokens.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"
#include "rope_math.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kChunkTok = 128;
// The rotary form stages a chunk's keys and values in LDS: smaller chunks
// keep its footprint near 26 KB so that several workgroups share a CU.
constexpr int kRopeChunkTok = 32;
template <bool ROPE>
constexpr int chunk_tok() { return ROPE ? kRopeChunkTok : kChunkTok; }
constexpr float kLog2e = 1.4426950408889634f;
typedef float float4v __attribute__((ext_vector_type(4)));

__device__ inline float h2f(uint16_t u) {
  return (float)__builtin_bit_cast(_Float16, u);
}
__device__ inline float bf2f(uint16_t u) {
  return __builtin_bit_cast(float, (uint32_t)u << 16);
}

__device__ inline uint32_t field(uint32_t w, int j, int bits) {
  return (w >> (j * bits)) & ((1u << bits) - 1u);
}

// Ring row of past-sink index p in the tail (32-bit remainder when p fits).
__device__ inline int64_t ring_row(int64_t p, int R) {
  return p <= 0x7FFFFFFF ? (int64_t)((uint32_t)p % (uint32_t)R) : p % R;
}

// Dequantized key of token t (cache order: sink, quantized, tail) channel d.
__device__ float kdeq(const kvq_kv_view& v, int64_t s, int64_t t, int d) {
  const int D = v.head_dim;
  if (t < v.n_sink) return h2f(v.sink_k[s * v.sink_stride + t * D + d]);
  t -= v.n_sink;
  if (t < v.n_quant) {
    const int64_t g = t / v.group_tok;
    if (!v.k_mixed) {
      const int kb = v.k_bits, pw = fields_per_word(kb), wk = words_of(D, kb);
      uint32_t w = v.k_codes[s * v.k_codes_stride + t * wk + d / pw];
      int u = (int)field(w, d % pw, kb);
      return (float)(u - qmax_of(kb) - 1) *
             v.k_scales[s * v.k_scales_stride + g * D + d];
    }
    const int nb = v.n_bf16, n4 = v.n_int4, n2 = D - nb - n4;
    const int pos = v.k_pos[s * v.k_pos_stride + g * D + d];
    if (pos < nb) return bf2f(v.k_bf16[s * v.k_bf16_stride + t * nb + pos]);
    const float sc = v.k_scales[s * v.k_scales_stride + g * (n4 + n2) + (pos - nb)];
    if (pos < nb + n4) {
      const int k = pos - nb, w4 = words_of(n4, 4);
      uint32_t w = v.k_int4[s * v.k_int4_stride + t * w4 + k / 8];
      return (float)((int)field(w, k % 8, 4) - 8) * sc;
    }
    const int k = pos - nb - n4, w2 = words_of(n2, 2);
    uint32_t w = v.k_int2[s * v.k_int2_stride + t * w2 + k / 16];
    return (float)((int)field(w, k % 16, 2) - 2) * sc;
  }
  t -= v.n_quant;
  return h2f(v.tail_k[s * v.tail_stride + ring_row(v.n_quant + t, v.residual) * D + d]);
}

__device__ float vdeq(const kvq_kv_view& v, int64_t s, int64_t t, int d) {
  const int D = v.head_dim;
  if (t < v.n_sink) return h2f(v.sink_v[s * v.sink_stride + t * D + d]);
  t -= v.n_sink;
  if (t < v.n_quant) {
    const int vb = v.v_bits;
    uint32_t u;
    if (v.v_layout == KVQ_V_ROWS) {
      const int pw = fields_per_word(vb), wv = words_of(D, vb);
      u = field(v.v_codes[s * v.v_codes_stride + t * wv + d / pw], d % pw, vb);
    } else {
      int64_t widx;
      int bit;
      v_tile_pos(t, d, D, vb, &widx, &bit);
      u = (v.v_codes[s * v.v_codes_stride + widx] >> bit) & ((1u << vb) - 1u);
    }
    const int ng = D / v.group_ch;
    return (float)((int)u - qmax_of(vb) - 1) *
           v.v_scales[s * v.v_scales_stride + t * ng + d / v.group_ch];
  }
  t -= v.n_quant;
  return h2f(v.tail_v[s * v.tail_stride + ring_row(v.n_quant + t, v.residual) * D + d]);
}

// Dequantized keys (or values) of range tokens c0 .. c0 + n - 1 into
// dst[t][D], eight channels per item: an fp16 sink or tail row moves with
// one 16-byte load (every item's load is independent of the others), a
// quantized row goes through kdeq / vdeq.
__device__ inline void stage_rows(const kvq_kv_view& v, int64_t s, int64_t c0, int n,
                                  int64_t gap_at, int64_t gap_len, bool keys, float* dst) {
  const int D = v.head_dim;
  const int nb = (D + 7) / 8;
  for (int i = threadIdx.x; i < n * nb; i += blockDim.x) {
    const int t = i / nb, d0 = 8 * (i % nb);
    const int64_t ci = c0 + t < gap_at ? c0 + t : c0 + t + gap_len;
    const uint16_t* row = nullptr;
    if (ci < v.n_sink) {
      row = (keys ? v.sink_k : v.sink_v) + s * v.sink_stride + ci * D;
    } else if (ci >= v.n_sink + v.n_quant) {
      row = (keys ? v.tail_k : v.tail_v) + s * v.tail_stride +
            ring_row(ci - v.n_sink, v.residual) * D;
    }
    if (!row && keys && v.k_mixed && d0 + 8 <= D) {
      // a quantized mixed-key row: the eight channels' class positions
      // first, then every channel's code (or bf16 value) and scale, each
      // round issued as independent loads
      const int64_t q = ci - v.n_sink;
      const int64_t g = q / v.group_tok;
      const int nb = v.n_bf16, n4 = v.n_int4, n2 = D - nb - n4;
      const int w4 = words_of(n4, 4), w2 = words_of(n2, 2);
      const uint8_t* kp = v.k_pos + s * v.k_pos_stride + g * D + d0;
      int pos[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) pos[k] = kp[k];
      uint32_t raw[8];
      float sc[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int ps = pos[k];
        if (ps < nb) {
          raw[k] = v.k_bf16[s * v.k_bf16_stride + q * nb + ps];
          sc[k] = 1.0f;
        } else if (ps < nb + n4) {
          raw[k] = v.k_int4[s * v.k_int4_stride + q * w4 + (ps - nb) / 8];
          sc[k] = v.k_scales[s * v.k_scales_stride + g * (n4 + n2) + (ps - nb)];
        } else {
          raw[k] = v.k_int2[s * v.k_int2_stride + q * w2 + (ps - nb - n4) / 16];
          sc[k] = v.k_scales[s * v.k_scales_stride + g * (n4 + n2) + (ps - nb)];
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int ps = pos[k];
        float x;
        if (ps < nb) {
          x = bf2f((uint16_t)raw[k]);
        } else if (ps < nb + n4) {
          x = (float)((int)field(raw[k], (ps - nb) % 8, 4) - 8) * sc[k];
        } else {
          x = (float)((int)field(raw[k], (ps - nb - n4) % 16, 2) - 2) * sc[k];
        }
        dst[t * D + d0 + k] = x;
      }
    } else if (!row && !keys && d0 + 8 <= D) {
      // a quantized value row: the eight channels' code words (either
      // layout) and scales as independent loads, then the codes
      const int64_t q = ci - v.n_sink;
      const int vb = v.v_bits, ng = D / v.group_ch;
      uint32_t wv[8];
      int bit[8];
      float sc[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int d = d0 + k;
        int64_t widx;
        if (v.v_layout == KVQ_V_ROWS) {
          const int pw = fields_per_word(vb);
          widx = q * words_of(D, vb) + d / pw;
          bit[k] = (d % pw) * vb;
        } else {
          v_tile_pos(q, d, D, vb, &widx, &bit[k]);
        }
        wv[k] = v.v_codes[s * v.v_codes_stride + widx];
        sc[k] = v.v_scales[s * v.v_scales_stride + q * ng + d / v.group_ch];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k)
        dst[t * D + d0 + k] =
            (float)((int)((wv[k] >> bit[k]) & ((1u << vb) - 1u)) - qmax_of(vb) - 1) * sc[k];
    } else if (row && d0 + 8 <= D && ((uintptr_t)(row + d0) & 15) == 0) {
      const uint4 w = *(const uint4*)(row + d0);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        dst[t * D + d0 + 2 * k] = h2f((uint16_t)(u[k] & 0xFFFFu));
        dst[t * D + d0 + 2 * k + 1] = h2f((uint16_t)(u[k] >> 16));
      }
    } else {
      for (int d = d0; d < D && d < d0 + 8; ++d)
        dst[t * D + d] = keys ? kdeq(v, s, ci, d) : vdeq(v, s, ci, d);
    }
  }
}

template <typename T> __device__ inline float ldq(const T* p, int64_t i);
template <> __device__ inline float ldq<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ inline float ldq<uint16_t>(const uint16_t* p, int64_t i) {
  return h2f(p[i]);
}

template <typename QT, bool ROPE>
__global__ void __launch_bounds__(kThreads)
decode_generic_kernel(kvq_kv_view v, const QT* __restrict__ q, int Hq,
                      float qscale, float* __restrict__ partials,
                      int64_t range_lo, int64_t range_hi, int n_parts,
                      int part_offset, int part_stride, int64_t gap_at, int64_t gap_len,
                      RopeDev rope) {
  constexpr int CT = chunk_tok<ROPE>();
  extern __shared__ float smem[];
  const int D = v.head_dim;
  const int g = Hq / v.kv_heads;
  double* phis = (double*)smem;      // [D/2] turns per position (rotary only)
  float* qs = smem + (ROPE ? D : 0); // [g][D]
  float* ps = qs + g * D;            // [g][CT]
  float* os = ps + g * CT;           // [g][D]
  float* ms = os + g * D;            // [g]
  float* ls = ms + g;                // [g]
  float* as = ls + g;                // [g]
  float* kr = as + g;                // [CT][D] turned keys (rotary only)
  const int tid = threadIdx.x;
  const int part = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int64_t s = (int64_t)b * v.kv_heads + kvh;
  const int64_t N = range_hi - range_lo;
  const int64_t per = (N + n_parts - 1) / n_parts;
  const int64_t t_lo = range_lo + min(N, (int64_t)part * per);
  const int64_t t_hi = min(range_hi, t_lo + per);

  for (int i = tid; i < g * D; i += kThreads) {
    const int h = i / D, d = i % D;
    qs[i] = ldq(q, ((int64_t)b * Hq + kvh * g + h) * D + d) * qscale;
    os[i] = 0.0f;
  }
  if (tid < g) {
    ms[tid] = -INFINITY;
    ls[tid] = 0.0f;
  }
  if (ROPE)
    for (int f = tid; f < D / 2; f += kThreads) phis[f] = rope.phi[f];
  __syncthreads();

  for (int64_t c0 = t_lo; c0 < t_hi; c0 += CT) {
    const int n = (int)min((int64_t)CT, t_hi - c0);
    if (ROPE) {
      // the chunk's dequantized keys into LDS, eight channels per item
      // (fp16 rows with one 16-byte load), then turned in place, one
      // (token, frequency) pair per item: pair (a, b) of frequency f by the
      // angle (pos0 + i) * theta_f
      stage_rows(v, s, c0, n, gap_at, gap_len, true, kr);
      __syncthreads();
      const int hd = D / 2;
      for (int i = tid; i < n * hd; i += kThreads) {
        const int t = i / hd, f = i % hd;
        const int a = rope.interleaved ? 2 * f : f;
        const int bb = rope.interleaved ? 2 * f + 1 : f + hd;
        const int64_t ci = c0 + t < gap_at ? c0 + t : c0 + t + gap_len;
        const float2 cs = rope_cos_sin(rope_turns((double)(rope.pos0 + ci), phis[f]));
        const float ka = kr[t * D + a], kb = kr[t * D + bb];
        kr[t * D + a] = ka * cs.x - kb * cs.y;
        kr[t * D + bb] = ka * cs.y + kb * cs.x;
      }
      __syncthreads();
    }
    if (ROPE) {
      // scores from the turned keys: four lanes per (token, head), each
      // summing every fourth channel, then a 4-lane sum
      for (int i0 = 0; i0 < n * g * 4; i0 += kThreads) {
        const int i = i0 + tid;
        const int it = i >> 2, qd = i & 3;
        const int t = it % n, h = it / n;
        float acc = 0.0f;
        if (i < n * g * 4)
          for (int d = qd; d < D; d += 4) acc += qs[h * D + d] * kr[t * D + d];
        acc += __shfl_xor(acc, 1);
        acc += __shfl_xor(acc, 2);
        if (i < n * g * 4 && qd == 0) ps[h * CT + t] = acc;
      }
    }
    for (int i = tid; i < (ROPE ? 0 : n * g); i += kThreads) {
      const int t = i % n, h = i / n;
      float acc = 0.0f;
      {
        const int64_t ci = c0 + t < gap_at ? c0 + t : c0 + t + gap_len;
        for (int d = 0; d < D; ++d) acc += qs[h * D + d] * kdeq(v, s, ci, d);
      }
      ps[h * CT + t] = acc;
    }
    __syncthreads();
    if (tid < g) {
      float mx = -INFINITY;
      for (int t = 0; t < n; ++t) mx = fmaxf(mx, ps[tid * CT + t]);
      const float mnew = fmaxf(ms[tid], mx);
      as[tid] = exp2f(ms[tid] - mnew);
      ms[tid] = mnew;
    }
    __syncthreads();
    for (int i = tid; i < n * g; i += kThreads) {
      const int t = i % n, h = i / n;
      ps[h * CT + t] = exp2f(ps[h * CT + t] - ms[h]);
    }
    __syncthreads();
    if (tid < g) {
      float l = ls[tid] * as[tid];
      for (int t = 0; t < n; ++t) l += ps[tid * CT + t];
      ls[tid] = l;
    }
    if (ROPE) {
      // the chunk's values into the (now free) LDS rows of the turned keys
      stage_rows(v, s, c0, n, gap_at, gap_len, false, kr);
      __syncthreads();
    }
    for (int i = tid; i < g * D; i += kThreads) {
      const int h = i / D, d = i % D;
      float acc = os[i] * as[h];
      for (int t = 0; t < n; ++t) {
        float vv;
        if (ROPE) {
          vv = kr[t * D + d];
        } else {
          const int64_t ci = c0 + t < gap_at ? c0 + t : c0 + t + gap_len;
          vv = vdeq(v, s, ci, d);
        }
        acc += ps[h * CT + t] * vv;
      }
      os[i] = acc;
    }
    __syncthreads();
  }
  for (int i = tid; i < g * (D + 2); i += kThreads) {
    const int h = i / (D + 2), j = i % (D + 2);
    float val = j == 0 ? ms[h] : (j == 1 ? ls[h] : os[h * D + j - 2]);
    partials[(((int64_t)b * Hq + kvh * g + h) * part_stride + part_offset + part) * (D + 2) + j] =
        val;
  }
}

// out[b][h][:] = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, one
// workgroup per (batch, query head).  The merge is latency-bound (a few
// hundred partials of D + 2 floats per head), so every load of a pass is
// issued before anything waits: thread (row r, column c) loads channels
// 4c .. 4c + 3 of partials r, r + R, ... (kMergeK of them, R = 256 / C rows
// for C = the power of two >= D / 4 columns) while the (m, l) pairs go to
// LDS and M and the weights are formed; the R row sums are then added in
// LDS.  More than R * kMergeK partials take further passes.
constexpr int kMergeThreads = 256;
constexpr int kMergeK = 16;
// Wave reductions for the merge: four DPP row rotations (8, 4, 2, 1) give
// every lane its 16-lane row's result, and the four rows are combined from
// scalar reads (a chain of VALU steps instead of six cross-lane LDS
// permutes); the result is the same in every lane.
template <int CTRL>
__device__ inline float row_rot(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ inline float lane_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ inline float wave_max(float x) {
  x = fmaxf(x, row_rot<0x128>(x));
  x = fmaxf(x, row_rot<0x124>(x));
  x = fmaxf(x, row_rot<0x122>(x));
  x = fmaxf(x, row_rot<0x121>(x));
  return fmaxf(fmaxf(lane_f(x, 0), lane_f(x, 16)), fmaxf(lane_f(x, 32), lane_f(x, 48)));
}
__device__ inline float wave_sum(float x) {
  x += row_rot<0x128>(x);
  x += row_rot<0x124>(x);
  x += row_rot<0x122>(x);
  x += row_rot<0x121>(x);
  return (lane_f(x, 0) + lane_f(x, 16)) + (lane_f(x, 32) + lane_f(x, 48));
}
template <bool EVEN>  // D even: every channel pair is 8-byte aligned
__global__ void __launch_bounds__(kMergeThreads)
merge_kernel(const float* __restrict__ partials, int D, int n_parts, int cols_log2,
             float* __restrict__ out) {
  __shared__ float red[kMergeThreads / 64];
  __shared__ float4v osum[kMergeThreads];
  extern __shared__ float ml[];  // [2][n_parts]: m, then l, then the weight
  float* mm = ml;
  float* ww = ml + n_parts;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = tid & ((1 << cols_log2) - 1), row = tid >> cols_log2;
  const int rows = kMergeThreads >> cols_log2;
  const int64_t bh = blockIdx.x;
  const int64_t stride = D + 2;
  const float* p = partials + bh * n_parts * stride;
  const int c0 = 4 * col;
  // this thread's channels c0 .. c0 + 3 of partial i (indexes clamped into
  // the array: columns past D and partials past n_parts are never used)
  auto load4 = [&](int i) {
    const float* src = p + (int64_t)min(i, n_parts - 1) * stride + 2;
    float4v x;
    if (EVEN) {
      const int cc = c0 < D ? c0 : 0;
      const float2 a = *(const float2*)(src + cc), b = *(const float2*)(src + min(cc + 2, D - 2));
      x = (float4v){a.x, a.y, b.x, b.y};
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = src[min(c0 + j, D - 1)];
    }
    return x;
  };
  const int per_pass = rows * kMergeK;
  float4v x[kMergeK];
#pragma unroll
  for (int k = 0; k < kMergeK; ++k) x[k] = load4(row + rows * k);
  float M = -INFINITY;
  for (int i = tid; i < n_parts; i += kMergeThreads) {
    const float m = p[i * stride], l = p[i * stride + 1];
    mm[i] = m;
    ww[i] = l;
    if (l > 0.0f) M = fmaxf(M, m);
  }
  M = wave_max(M);
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float L = 0.0f;
  for (int i = tid; i < n_parts; i += kMergeThreads) {
    const float l = ww[i];
    const float w = l > 0.0f ? exp2f(mm[i] - M) : 0.0f;
    ww[i] = w;
    L += l * w;
  }
  L = wave_sum(L);
  __syncthreads();
  if (lane == 0) red[wave] = L;
  __syncthreads();
  L = red[0] + red[1] + red[2] + red[3];
  float4v acc = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
  for (int base = 0;;) {
#pragma unroll
    for (int k = 0; k < kMergeK; ++k) {
      const int i = base + row + rows * k;
      if (i < n_parts) acc += x[k] * ww[i];
    }
    base += per_pass;
    if (base >= n_parts) break;
#pragma unroll
    for (int k = 0; k < kMergeK; ++k) x[k] = load4(base + row + rows * k);
  }
  osum[tid] = acc;
  __syncthreads();
  for (int d = tid; d < D; d += kMergeThreads) {
    const int cc = d >> 2, e = d & 3;
    float sum = 0.0f;
    for (int r = 0; r < rows; ++r) sum += osum[(r << cols_log2) + cc][e];
    out[bh * D + d] = sum / L;
  }
}

template <bool ROPE>
hipError_t launch_generic_t(const kvq_kv_view& v, const void* q, int f16, int Hq,
                            float qscale, float* partials, int64_t range_lo, int64_t range_hi,
                            int n_parts, int part_offset, int part_stride, int64_t gap_at,
                            int64_t gap_len, const RopeDev& rope, hipStream_t s) {
  const int g = Hq / v.kv_heads;
  const size_t lds =
      sizeof(float) * ((size_t)g * v.head_dim * 2 + (size_t)g * chunk_tok<ROPE>() + 3 * (size_t)g +
                       (ROPE ? (size_t)v.head_dim * (1 + chunk_tok<ROPE>()) : 0));
  dim3 grid((unsigned)n_parts, (unsigned)v.kv_heads, (unsigned)v.batch);
  const void* fn = f16 ? (const void*)decode_generic_kernel<uint16_t, ROPE>
                       : (const void*)decode_generic_kernel<float, ROPE>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (f16)
    decode_generic_kernel<uint16_t, ROPE><<<grid, kThreads, lds, s>>>(
        v, (const uint16_t*)q, Hq, qscale, partials, range_lo, range_hi, n_parts, part_offset,
        part_stride, gap_at, gap_len, rope);
  else
    decode_generic_kernel<float, ROPE><<<grid, kThreads, lds, s>>>(
        v, (const float*)q, Hq, qscale, partials, range_lo, range_hi, n_parts, part_offset,
        part_stride, gap_at, gap_len, rope);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_generic_range(const kvq_kv_view& v, const void* q, int f16,
                                       int Hq, float sm_scale, float* partials,
                                       int64_t range_lo, int64_t range_hi, int n_parts,
                                       int part_offset, int part_stride, const RopeDev* rope,
                                       hipStream_t s, int64_t gap_at, int64_t gap_len) {
  const float qscale = sm_scale * kLog2e;
  if (rope)
    return launch_generic_t<true>(v, q, f16, Hq, qscale, partials, range_lo, range_hi, n_parts,
                                  part_offset, part_stride, gap_at, gap_len, *rope, s);
  return launch_generic_t<false>(v, q, f16, Hq, qscale, partials, range_lo, range_hi, n_parts,
                                 part_offset, part_stride, gap_at, gap_len, RopeDev{}, s);
}

hipError_t launch_decode_generic(const kvq_kv_view& v, const void* q, int f16,
                                 int Hq, float sm_scale, float* partials,
                                 int n_parts, hipStream_t s) {
  const int64_t N = v.n_sink + v.n_quant + v.n_tail;
  return launch_decode_generic_range(v, q, f16, Hq, sm_scale, partials, 0, N, n_parts, 0,
                                     n_parts, nullptr, s);
}

hipError_t launch_merge(const float* partials, int B, int Hq, int D,
                        int n_parts, float* out, hipStream_t s) {
  const size_t lds = 2 * sizeof(float) * (size_t)n_parts;
  if (lds + 5 * 1024 > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)merge_kernel<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)merge_kernel<false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  int cols_log2 = 0;
  while ((4 << cols_log2) < D) ++cols_log2;  // D <= 256: at most 64 columns
  const dim3 grid((unsigned)(B * Hq));
  if (D % 2 == 0)
    merge_kernel<true><<<grid, kMergeThreads, lds, s>>>(partials, D, n_parts, cols_log2, out);
  else
    merge_kernel<false><<<grid, kMergeThreads, lds, s>>>(partials, D, n_parts, cols_log2, out);
  return hipGetLastError();
}

}  // namespace kvq
