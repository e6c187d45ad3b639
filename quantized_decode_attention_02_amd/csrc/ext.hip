// Extended formats of libkvq for gfx950: the non-uniform codebook datatype
// with per-vector dense-and-sparse outliers, the value-side 1-bit residual
// sketch, and the decode attention that reads them.
//
// Non-uniform datatype ("KVQuant: Towards 10 Million Context Length LLM
// Inference with KV Cache Quantization", summary, "Approach" and the table
// "Measured effects reported in the paper"): per vector (keys: one channel
// of a group of G tokens; values: one group of Gv channels of one token)
// the n_out entries of largest magnitude are kept exactly (position and
// fp16 value, ties to the lower position); the rest, with those entries set
// to zero, get scale = max|dense| / max|level| (IEEE float32 division, 1
// for a zero dense part) and per entry the index of the codebook level
// nearest to fl32(x / scale), ties to the lower level.  Reconstruction:
// level[code] * scale plus the outliers (the codebook holds an exact 0,
// which every outlier position's dense entry becomes).
//
// Residual sketch ("Statistical Inference and Quality Measures of KV Cache
// Quantisations Inspired by TurboQuant", "Quantization Schemes" (KQV) and
// "1. Theoretical Proof of QJL Harm on Keys"): a value row (rotated by the
// caller) is quantized per token with the symmetric rule; its residual
// r = x - fl32(code * scale) (exact in float32) is kept as the signs of
// S r for the m rows of a Gaussian matrix S (dot products in float64, +1 at
// zero) and gamma = ||r|| (float64 sum, rounded to float32).  The decode
// uses x_hat + sqrt(pi/2)/m * gamma * S^T b, an unbiased estimate of the
// value: the sign sums are accumulated per query head like one more value
// channel of 1-bit codes, and S^T is applied once per output row in the
// merge, followed by the inverse rotation.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsV = 32;    // token rows per workgroup of the value quantizers
constexpr int kCT = 64;       // tokens per decode chunk
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float h2f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
__device__ inline bool f16_finite(uint16_t u) { return (u & 0x7C00u) != 0x7C00u; }

// Level index of q: the number of midpoints strictly below q (a midpoint
// of two fp16 levels is exact in float32), i.e. the nearest level with
// ties to the lower one.
__device__ inline uint32_t nearest_code(float q, const ExtLut& L) {
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < 15; ++j)
    if (j < L.n - 1) c += q > L.mid[j] ? 1u : 0u;
  return c;
}

// One step of the per-vector top-n_out selection: the candidate (magnitude
// key, position) moves through the list, sorted strongest first, swapping
// with every entry it beats (larger magnitude, or equal magnitude at a
// lower position); empty slots hold key -1.  Positions arrive ascending,
// so an equal magnitude never displaces an earlier entry.
__device__ inline void topk_insert(int (&key)[16], int (&pos)[16], int n_out, int k, int p) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < n_out) {
      const bool beats = k > key[j] || (k == key[j] && p < pos[j]);
      if (beats) {
        const int tk = key[j], tp = pos[j];
        key[j] = k;
        pos[j] = p;
        k = tk;
        p = tp;
      }
    }
  }
}

// Sort the selected positions ascending (at most 16, insertion sort).
__device__ inline void sort_positions(int (&pos)[16], int n) {
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    if (i < n) {
      const int x = pos[i];
      int j = i - 1;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        if (j >= 0 && pos[j] > x) {
          pos[j + 1] = pos[j];
          --j;
        }
      }
      pos[j + 1] = x;
    }
  }
}

// Pack the u8 level indices of `rows` rows of d channels into words.
__device__ inline void pack_rows(const uint8_t* u8, int rows, int d, int bits,
                                 uint32_t* __restrict__ codes, int64_t row0) {
  const int wk = words_of(d, bits), pw = fields_per_word(bits);
  for (int i = threadIdx.x; i < rows * wk; i += kThreads) {
    const int r = i / wk, w = i % wk;
    uint32_t word = 0;
    for (int j = 0; j < pw; ++j) {
      const int c = w * pw + j;
      if (c < d) word |= (uint32_t)u8[r * d + c] << (j * bits);
    }
    codes[(row0 + r) * wk + w] = word;
  }
}

// ---------------------------------------------------------------------------
// Keys: one workgroup per (matrix, group of G tokens); the group's fp16 rows
// in LDS, one thread per channel for the selection and the scale, then
// every element's code.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
quantize_nuq_k_kernel(const uint16_t* __restrict__ k, int64_t n_tok, int d, int bits, int G,
                      ExtLut L, int n_out, uint32_t* __restrict__ codes,
                      float* __restrict__ scales, uint32_t* __restrict__ outl, uint32_t* err) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int rows_max = G;
  uint16_t* xs = (uint16_t*)smem;                                   // [G][d]
  float* sc = (float*)(smem + ((size_t)rows_max * d * 2 + 15) / 16 * 16);  // [d]
  uint8_t* u8 = (uint8_t*)(sc + d);                                 // [G][d]
  const int tid = threadIdx.x;
  const int64_t mat = blockIdx.y, g = blockIdx.x;
  const int64_t ng = (n_tok + G - 1) / G;
  const int64_t t0 = g * G;
  const int rows = (int)min((int64_t)G, n_tok - t0);
  const uint16_t* x = k + (mat * n_tok + t0) * d;
  bool bad = false;
  for (int i = tid; i < rows * d; i += kThreads) {
    const uint16_t u = x[i];
    bad |= !f16_finite(u);
    xs[i] = u;
  }
  if (bad && err) atomicOr(err, 1u);
  __syncthreads();
  for (int c = tid; c < d; c += kThreads) {
    int key[16], pos[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) { key[j] = -1; pos[j] = 0; }
    for (int r = 0; r < rows; ++r) topk_insert(key, pos, n_out, xs[r * d + c] & 0x7FFF, r);
    const int nk = n_out < rows ? n_out : rows;
    sort_positions(pos, nk);
    uint32_t* o = outl + ((mat * ng + g) * d + c) * n_out;
    for (int j = 0; j < n_out; ++j) {
      uint32_t e = 0;
      if (j < nk) {
        e = ((uint32_t)pos[j] << 16) | xs[pos[j] * d + c];
        xs[pos[j] * d + c] = 0;     // the dense part is zero there
      }
      o[j] = e;
    }
    float m = 0.0f;
    for (int r = 0; r < rows; ++r) m = fmaxf(m, fabsf(h2f(xs[r * d + c])));
    float s = __fdiv_rn(m, L.absmax);
    if (m == 0.0f || s == 0.0f) s = 1.0f;
    sc[c] = s;
    scales[(mat * ng + g) * d + c] = s;
  }
  __syncthreads();
  for (int i = tid; i < rows * d; i += kThreads)
    u8[i] = (uint8_t)nearest_code(__fdiv_rn(h2f(xs[i]), sc[i % d]), L);
  __syncthreads();
  pack_rows(u8, rows, d, bits, codes, mat * n_tok + t0);
}

// ---------------------------------------------------------------------------
// Values: one workgroup per (matrix, kRowsV tokens); one thread per
// (token, channel group) for the selection and the scale.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
quantize_nuq_v_kernel(const uint16_t* __restrict__ v, int64_t n_tok, int d, int bits, int Gv,
                      ExtLut L, int n_out, uint32_t* __restrict__ codes,
                      float* __restrict__ scales, uint32_t* __restrict__ outl, uint32_t* err) {
  __shared__ uint16_t xs[kRowsV * kMaxD];
  __shared__ float sc[kRowsV * kMaxD];
  __shared__ uint8_t u8[kRowsV * kMaxD];
  const int tid = threadIdx.x;
  const int64_t mat = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.x * kRowsV;
  const int rows = (int)min((int64_t)kRowsV, n_tok - r0);
  const uint16_t* x = v + (mat * n_tok + r0) * d;
  const int ng = d / Gv;
  bool bad = false;
  for (int i = tid; i < rows * d; i += kThreads) {
    const uint16_t u = x[i];
    bad |= !f16_finite(u);
    xs[i] = u;
  }
  if (bad && err) atomicOr(err, 1u);
  __syncthreads();
  for (int i = tid; i < rows * ng; i += kThreads) {
    const int r = i / ng, j = i % ng;
    uint16_t* row = xs + r * d + j * Gv;
    int key[16], pos[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) { key[s] = -1; pos[s] = 0; }
    for (int c = 0; c < Gv; ++c) topk_insert(key, pos, n_out, row[c] & 0x7FFF, c);
    const int nk = n_out < Gv ? n_out : Gv;
    sort_positions(pos, nk);
    uint32_t* o = outl + ((mat * n_tok + r0 + r) * ng + j) * n_out;
    for (int s = 0; s < n_out; ++s) {
      uint32_t e = 0;
      if (s < nk) {
        e = ((uint32_t)pos[s] << 16) | row[pos[s]];
        row[pos[s]] = 0;
      }
      o[s] = e;
    }
    float m = 0.0f;
    for (int c = 0; c < Gv; ++c) m = fmaxf(m, fabsf(h2f(row[c])));
    float s = __fdiv_rn(m, L.absmax);
    if (m == 0.0f || s == 0.0f) s = 1.0f;
    sc[i] = s;
    scales[(mat * n_tok + r0 + r) * ng + j] = s;
  }
  __syncthreads();
  for (int i = tid; i < rows * d; i += kThreads) {
    const int r = i / d, c = i % d;
    u8[i] = (uint8_t)nearest_code(__fdiv_rn(h2f(xs[i]), sc[r * ng + c / Gv]), L);
  }
  __syncthreads();
  pack_rows(u8, rows, d, bits, codes, mat * n_tok + r0);
}

// ---------------------------------------------------------------------------
// Values with the 1-bit residual sketch: one workgroup per (matrix,
// kRowsV tokens).  Symmetric scalar codes per (token, Gv channels), the
// exact float32 residual, its float64 norm, and the float64 signs of S r
// packed with a ballot (wave lane i = sketch row i0 + i).
// ---------------------------------------------------------------------------
template <typename T> __device__ inline float ldx(const T* p, int64_t i);
template <> __device__ inline float ldx<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ inline float ldx<uint16_t>(const uint16_t* p, int64_t i) { return h2f(p[i]); }

template <typename T>
__global__ void __launch_bounds__(kThreads)
quantize_v_qjl_kernel(const T* __restrict__ v, int64_t n_tok, int d, int bits, int Gv,
                      const float* __restrict__ S, int m, uint32_t* __restrict__ codes,
                      float* __restrict__ scales, uint32_t* __restrict__ sketch,
                      float* __restrict__ rnorm, uint32_t* err) {
  __shared__ float rs[kRowsV * kMaxD];   // the values, then the residuals
  __shared__ float sc[kRowsV * kMaxD];
  __shared__ uint8_t u8[kRowsV * kMaxD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t mat = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.x * kRowsV;
  const int rows = (int)min((int64_t)kRowsV, n_tok - r0);
  const T* x = v + (mat * n_tok + r0) * d;
  const int ng = d / Gv, qmax = qmax_of(bits);
  bool bad = false;
  for (int i = tid; i < rows * d; i += kThreads) {
    const float val = ldx(x, i);
    bad |= !__builtin_isfinite(val);
    rs[i] = val;
  }
  if (bad && err) atomicOr(err, 1u);
  __syncthreads();
  for (int i = tid; i < rows * ng; i += kThreads) {
    const int r = i / ng, j = i % ng;
    float mx = 0.0f;
    for (int c = 0; c < Gv; ++c) mx = fmaxf(mx, fabsf(rs[r * d + j * Gv + c]));
    float s = __fdiv_rn(mx, (float)qmax);
    if (mx == 0.0f || s == 0.0f) s = 1.0f;
    sc[i] = s;
    scales[(mat * n_tok + r0 + r) * ng + j] = s;
  }
  __syncthreads();
  for (int i = tid; i < rows * d; i += kThreads) {
    const int r = i / d, c = i % d;
    const float s = sc[r * ng + c / Gv];
    float q = rintf(__fdiv_rn(rs[i], s));
    q = fminf(fmaxf(q, (float)-qmax), (float)qmax);
    u8[i] = (uint8_t)((int)q + qmax + 1);
    rs[i] = rs[i] - q * s;        // x - fl32(code * scale), exact
  }
  __syncthreads();
  pack_rows(u8, rows, d, bits, codes, mat * n_tok + r0);
  if (tid < rows) {
    double acc = 0.0;
    for (int c = 0; c < d; ++c) {
      const double t = rs[tid * d + c];
      acc += t * t;
    }
    rnorm[mat * n_tok + r0 + tid] = (float)sqrt(acc);
  }
  const int mw = m / 32;
  for (int r = wave; r < rows; r += kThreads / 64) {
    for (int i0 = 0; i0 < m; i0 += 64) {
      const int i = i0 + lane;
      double dot = 0.0;
      if (i < m) {
        const float* srow = S + (int64_t)i * d;
        for (int c = 0; c < d; ++c) dot += (double)srow[c] * (double)rs[r * d + c];
      }
      const uint64_t bal = __ballot(i < m && dot >= 0.0);
      uint32_t* out = sketch + (mat * n_tok + r0 + r) * mw + i0 / 32;
      if (lane == 0) out[0] = (uint32_t)bal;
      if (lane == 32 && i0 + 32 < m) out[1] = (uint32_t)(bal >> 32);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode over an extended view: one workgroup per (split, KV head, batch);
// splits are whole 64-token chunks.  Thread tid owns channel c = tid % D of
// the tokens tid / D, tid / D + 256 / D, ... of a chunk for the dequant
// (the field's word and shift, the channel's scale and the codebook in LDS
// are fixed per thread or per chunk, so no division runs per element);
// the chunk's keys go to LDS, the group's outliers are added, four lanes
// per token score it against every query head (a lane sums every fourth
// channel: rows padded to D + 4 floats, so the 16 tokens x 4 lanes of a
// wave hit distinct banks), the online softmax runs a wave per head, then
// the values the same way, and thread (channel, head set) accumulates the
// weighted sums; the sketch words and norms of the chunk go to LDS for the
// per-head sign sums.  Partial record per (batch, head, split): m (log2
// units), l, o[D], z[M] (M = m of the sketch, 0 without one).
// ---------------------------------------------------------------------------
struct ExtArgs {
  kvq_ext_view v;
  ExtLut lk, lv;
  int Hq;
  float qscale;       // sm_scale * log2(e)
  float* partials;
  int n_parts;
  int rec;            // D + 2 + M
  int64_t per;        // tokens per split, a multiple of kCT
};

// LDS words of the per-chunk staging areas (codes, scales, sketch words).
struct ExtStage {
  int kw, vw, ngv, mw;   // words per key / value row, value groups, sketch words
};

template <typename QT, int D>
__global__ void __launch_bounds__(kThreads)
decode_ext_kernel(ExtArgs a, const QT* __restrict__ q) {
  constexpr int Dp = D + 4;               // padded LDS row
  constexpr int TPT = kThreads / D;       // token lanes of the dequant
  extern __shared__ __align__(16) float sm[];
  const kvq_ext_view& v = a.v;
  const int g = a.Hq / v.kv_heads;
  const int M = v.v_qjl ? v.qjl_m : 0, MW = M / 32;
  const int kb = v.k_bits, vb = v.v_bits;
  const int kw_row = words_of(D, kb), vw_row = words_of(D, vb);
  const int ngv = D / v.group_ch;
  float* lut = sm;                        // [32]: key levels, value levels
  float* qs = lut + 32;                   // [g][D]
  float* buf = qs + g * D;                // [kCT][Dp]
  float* ps = buf + kCT * Dp;             // [g][kCT]
  float* st = ps + g * kCT;               // [3][g]: m, l, alpha
  float* gam = st + 3 * g;                // [kCT]
  float* ksl = gam + kCT;                 // [2][D]: scales of the chunk's key groups
  float* vsl = ksl + 2 * D;               // [kCT][ngv]
  uint32_t* skw = (uint32_t*)(vsl + kCT * ngv);  // [kCT][MW]
  uint32_t* kcw = skw + kCT * MW;         // [kCT][kw_row]
  uint32_t* vcw = kcw + kCT * kw_row;     // [kCT][vw_row]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int64_t s = (int64_t)b * v.kv_heads + kvh;
  const int64_t N = v.n_tok;
  const int64_t t_lo = min(N, (int64_t)part * a.per), t_hi = min(N, t_lo + a.per);
  const int G = v.group_tok;

  // per-thread constants of the dequant: channel c of tokens t0 + TPT j
  const int c = tid % D, t0 = tid / D;
  const int kword = c / fields_per_word(kb), kshift = (c % fields_per_word(kb)) * kb;
  const int vword = c / fields_per_word(vb), vshift = (c % fields_per_word(vb)) * vb;
  const uint32_t kmask = (1u << kb) - 1u, vmask = (1u << vb) - 1u;
  const int vgrp = c / v.group_ch;
  const float koff = v.k_nuq ? 0.0f : (float)(qmax_of(kb) + 1);
  const float voff = v.v_nuq ? 0.0f : (float)(qmax_of(vb) + 1);

  if (tid < 16) {
    lut[tid] = v.k_nuq ? a.lk.lvl[tid] : 0.0f;
    lut[16 + tid] = v.v_nuq ? a.lv.lvl[tid] : 0.0f;
  }
  for (int i = tid; i < g * D; i += kThreads)
    qs[i] = ldx(q, ((int64_t)b * a.Hq + kvh * g) * D + i) * a.qscale;
  if (tid < g) {
    st[tid] = -INFINITY;
    st[g + tid] = 0.0f;
  }
  float o[8], z[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) { o[k] = 0.0f; z[k] = 0.0f; }
  __syncthreads();

  const uint32_t* kc = v.k_codes + s * v.k_codes_stride;
  const float* ks = v.k_scales + s * v.k_scales_stride;
  const uint32_t* ko = v.k_n_out ? v.k_outliers + s * v.k_outliers_stride : nullptr;
  const uint32_t* vc = v.v_codes + s * v.v_codes_stride;
  const float* vs = v.v_scales + s * v.v_scales_stride;
  const uint32_t* vo = v.v_n_out ? v.v_outliers + s * v.v_outliers_stride : nullptr;

  for (int64_t c0 = t_lo; c0 < t_hi; c0 += kCT) {
    const int n = (int)min((int64_t)kCT, t_hi - c0);
    // ---- every load of the chunk at once, into LDS: the code rows (one
    //      contiguous range each), the key scales of its (at most two)
    //      groups, the value scales, the sketch words and norms
    const int64_t g0 = c0 / G;
    const int r0 = (int)(c0 - g0 * G);            // chunk start within its group
    const int ng_chunk = (r0 + n > G) ? 2 : 1;
    for (int i = tid; i < n * kw_row; i += kThreads) kcw[i] = kc[c0 * kw_row + i];
    for (int i = tid; i < n * vw_row; i += kThreads) vcw[i] = vc[c0 * vw_row + i];
    for (int i = tid; i < ng_chunk * D; i += kThreads) ksl[i] = ks[g0 * D + i];
    for (int i = tid; i < n * ngv; i += kThreads) vsl[i] = vs[c0 * ngv + i];
    if (M) {
      for (int i = tid; i < n * MW; i += kThreads)
        skw[i] = v.v_sketch[s * v.v_sketch_stride + c0 * MW + i];
      for (int t = tid; t < n; t += kThreads) gam[t] = v.v_rnorm[s * v.v_rnorm_stride + c0 + t];
    }
    __syncthreads();
    // ---- keys of the chunk: level (or centred code) times the channel's
    //      scale of the token's group
    for (int t = t0; t < n; t += TPT) {
      const uint32_t code = (kcw[t * kw_row + kword] >> kshift) & kmask;
      const float lvl = v.k_nuq ? lut[code] : (float)code - koff;
      buf[t * Dp + c] = lvl * ksl[(r0 + t >= G ? D : 0) + c];
    }
    if (ko) {
      const int per_g = D * v.k_n_out;
      __syncthreads();
      for (int gi = 0; gi < ng_chunk; ++gi) {
        for (int i = tid; i < per_g; i += kThreads) {
          const uint32_t e = ko[(g0 + gi) * per_g + i];
          if ((e & 0x7FFFu) == 0) continue;               // +-0: nothing to add
          const int64_t tok = (g0 + gi) * G + (e >> 16);
          if (tok < c0 || tok >= c0 + n) continue;
          buf[(tok - c0) * Dp + i / v.k_n_out] += h2f((uint16_t)(e & 0xFFFFu));
        }
      }
    }
    __syncthreads();
    // ---- scores: lane (token tid / 4, quarter tid % 4) sums channels
    //      quarter, quarter + 4, ... for every head
    {
      const int t = tid >> 2, qd = tid & 3;
      float acc[8];
#pragma unroll
      for (int h = 0; h < 8; ++h) acc[h] = 0.0f;
      if (t < n) {
#pragma unroll 4
        for (int j = qd; j < D; j += 4) {
          const float kv = buf[t * Dp + j];
#pragma unroll
          for (int h = 0; h < 8; ++h)
            if (h < g) acc[h] = __builtin_fmaf(qs[h * D + j], kv, acc[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        if (h < g) {
          float x = acc[h];
          x += __shfl_xor(x, 1);
          x += __shfl_xor(x, 2);
          if (qd == 0 && t < n) ps[h * kCT + t] = x;
        }
      }
    }
    __syncthreads();
    // ---- online softmax: a wave per head (lane = token)
    for (int h = wave; h < g; h += kThreads / 64) {
      const float x = lane < n ? ps[h * kCT + lane] : -INFINITY;
      float mx = x;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_old = st[h];
      const float m_new = fmaxf(m_old, mx);
      const float p = lane < n ? exp2f(x - m_new) : 0.0f;
      float ls = p;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) ls += __shfl_xor(ls, off);
      const float alpha = exp2f(m_old - m_new);
      if (lane < n) ps[h * kCT + lane] = p;
      if (lane == 0) {
        st[h] = m_new;
        st[g + h] = st[g + h] * alpha + ls;
        st[2 * g + h] = alpha;
      }
    }
    // ---- values of the chunk (into the key rows: the scores are done)
    for (int t = t0; t < n; t += TPT) {
      const uint32_t code = (vcw[t * vw_row + vword] >> vshift) & vmask;
      const float lvl = v.v_nuq ? lut[16 + code] : (float)code - voff;
      buf[t * Dp + c] = lvl * vsl[t * ngv + vgrp];
    }
    if (vo) {
      const int per_t = ngv * v.v_n_out;
      __syncthreads();
      for (int i = tid; i < n * per_t; i += kThreads) {
        const int t = i / per_t, r = i - t * per_t;
        const uint32_t e = vo[(c0 + t) * per_t + r];
        if ((e & 0x7FFFu) == 0) continue;
        const int cc = (r / v.v_n_out) * v.group_ch + (int)(e >> 16);
        buf[t * Dp + cc] += h2f((uint16_t)(e & 0xFFFFu));
      }
    }
    __syncthreads();
    // ---- weighted sums: channel c of heads t0, t0 + TPT, ...
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int h = t0 + k * TPT;
      if (h < g) {
        float acc = o[k] * st[2 * g + h];
#pragma unroll 8
        for (int t = 0; t < n; ++t) acc = __builtin_fmaf(ps[h * kCT + t], buf[t * Dp + c], acc);
        o[k] = acc;
      }
    }
    if (M) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = tid + k * kThreads;
        if (i < g * M) {
          const int h = i / M, j = i - h * M;
          float acc = z[k] * st[2 * g + h];
          for (int t = 0; t < n; ++t) {
            const float w = ps[h * kCT + t] * gam[t];
            acc += ((skw[t * MW + (j >> 5)] >> (j & 31)) & 1u) ? w : -w;
          }
          z[k] = acc;
        }
      }
    }
    __syncthreads();
  }
  float* out = a.partials + (((int64_t)b * a.Hq + kvh * g) * a.n_parts + part) * a.rec;
  const int64_t hstride = (int64_t)a.n_parts * a.rec;
  if (tid < g) {
    out[tid * hstride] = st[tid];
    out[tid * hstride + 1] = st[g + tid];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int h = t0 + k * TPT;
    if (h < g) out[h * hstride + 2 + c] = o[k];
    const int i = tid + k * kThreads;
    if (M && i < g * M) out[(i / M) * hstride + 2 + D + i % M] = z[k];
  }
}

// out = turn(O + sqrt(pi/2)/m S^T Z) / L over the partials of one (batch,
// query head): O, Z and L summed with the log-sum-exp weights; turn is the
// normalized Walsh-Hadamard transform when the values were stored rotated.
__global__ void __launch_bounds__(kThreads)
merge_ext_kernel(const float* __restrict__ partials, int D, int M, int n_parts, int rec,
                 const float* __restrict__ S, int rotated, float* __restrict__ out) {
  __shared__ float red[kThreads / 64];
  __shared__ float acc[kMaxD + 256];
  extern __shared__ float wts[];   // [n_parts]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bh = blockIdx.x;
  const float* p = partials + bh * n_parts * rec;
  float mx = -INFINITY;
  for (int i = tid; i < n_parts; i += kThreads)
    if (p[(int64_t)i * rec + 1] > 0.0f) mx = fmaxf(mx, p[(int64_t)i * rec]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float Mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float L = 0.0f;
  for (int i = tid; i < n_parts; i += kThreads) {
    const float l = p[(int64_t)i * rec + 1];
    const float w = l > 0.0f ? exp2f(p[(int64_t)i * rec] - Mx) : 0.0f;
    wts[i] = w;
    L += w * l;
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) L += __shfl_xor(L, off);
  if (lane == 0) red[wave] = L;
  __syncthreads();
  L = red[0] + red[1] + red[2] + red[3];
  // wave w sums partials w, w + 4, ... (lane l on entries l, l + 64, ...,
  // eight partials in flight), then the four waves are added in LDS
  __shared__ float part_sum[kThreads / 64][kMaxD + 256];
  {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = 0.0f;
    const int nj = D + M;
    for (int i = wave; i < n_parts; i += 4 * 2) {
      const bool two = i + 4 < n_parts;
      const float w0 = wts[i], w1 = two ? wts[i + 4] : 0.0f;
      const float* p0 = p + (int64_t)i * rec + 2;
      const float* p1 = p + (int64_t)(two ? i + 4 : i) * rec + 2;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = lane + 64 * k;
        if (j < nj) x[k] = __builtin_fmaf(w0, p0[j], __builtin_fmaf(w1, p1[j], x[k]));
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = lane + 64 * k;
      if (j < nj) part_sum[wave][j] = x[k];
    }
  }
  __syncthreads();
  for (int j = tid; j < D + M; j += kThreads)
    acc[j] = part_sum[0][j] + part_sum[1][j] + part_sum[2][j] + part_sum[3][j];
  __syncthreads();
  if (M) {
    const float c = 1.2533141373155003f / (float)M;   // sqrt(pi/2) / m
    for (int d = tid; d < D; d += kThreads) {
      float r = 0.0f;
      for (int i = 0; i < M; ++i) r = __builtin_fmaf(S[(int64_t)i * D + d], acc[D + i], r);
      acc[d] = __builtin_fmaf(c, r, acc[d]);
    }
    __syncthreads();
  }
  for (int d = tid; d < D; d += kThreads) acc[d] = acc[d] / L;
  __syncthreads();
  if (rotated) {
    for (int h = 1; h < D; h <<= 1) {
      for (int i = tid; i < D / 2; i += kThreads) {
        const int lo = (i / h) * 2 * h + (i % h), hi = lo + h;
        const float x = acc[lo], y = acc[hi];
        acc[lo] = x + y;
        acc[hi] = x - y;
      }
      __syncthreads();
    }
    const float f = 1.0f / sqrtf((float)D);
    for (int d = tid; d < D; d += kThreads) acc[d] *= f;
    __syncthreads();
  }
  for (int d = tid; d < D; d += kThreads) out[bh * D + d] = acc[d];
}

}  // namespace

hipError_t launch_quantize_nuq_k(const uint16_t* k, int64_t n_mats, int64_t n_tok, int d,
                                 int bits, int G, const ExtLut& L, int n_out, uint32_t* codes,
                                 float* scales, uint32_t* outl, uint32_t* err, hipStream_t s) {
  const size_t lds = ((size_t)G * d * 2 + 15) / 16 * 16 + (size_t)d * 4 + (size_t)G * d;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)quantize_nuq_k_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)((n_tok + G - 1) / G), (unsigned)n_mats);
  quantize_nuq_k_kernel<<<grid, kThreads, lds, s>>>(k, n_tok, d, bits, G, L, n_out, codes, scales,
                                                    outl, err);
  return hipGetLastError();
}

hipError_t launch_quantize_nuq_v(const uint16_t* v, int64_t n_mats, int64_t n_tok, int d,
                                 int bits, int Gv, const ExtLut& L, int n_out, uint32_t* codes,
                                 float* scales, uint32_t* outl, uint32_t* err, hipStream_t s) {
  dim3 grid((unsigned)((n_tok + kRowsV - 1) / kRowsV), (unsigned)n_mats);
  quantize_nuq_v_kernel<<<grid, kThreads, 0, s>>>(v, n_tok, d, bits, Gv, L, n_out, codes, scales,
                                                  outl, err);
  return hipGetLastError();
}

hipError_t launch_quantize_v_qjl(const void* v, int f16, int64_t n_mats, int64_t n_tok, int d,
                                 int bits, int Gv, const float* S, int m, uint32_t* codes,
                                 float* scales, uint32_t* sketch, float* rnorm, uint32_t* err,
                                 hipStream_t s) {
  dim3 grid((unsigned)((n_tok + kRowsV - 1) / kRowsV), (unsigned)n_mats);
  if (f16)
    quantize_v_qjl_kernel<uint16_t><<<grid, kThreads, 0, s>>>(
        (const uint16_t*)v, n_tok, d, bits, Gv, S, m, codes, scales, sketch, rnorm, err);
  else
    quantize_v_qjl_kernel<float><<<grid, kThreads, 0, s>>>(
        (const float*)v, n_tok, d, bits, Gv, S, m, codes, scales, sketch, rnorm, err);
  return hipGetLastError();
}

size_t ext_decode_lds(const kvq_ext_view& v, int Hq) {
  const int g = Hq / v.kv_heads, D = v.head_dim, M = v.v_qjl ? v.qjl_m : 0;
  const size_t words = 32 + (size_t)g * D + (size_t)kCT * (D + 4) + (size_t)g * kCT + 3 * (size_t)g +
                       kCT + 2 * (size_t)D + (size_t)kCT * (D / v.group_ch) + (size_t)kCT * (M / 32) +
                       (size_t)kCT * words_of(D, v.k_bits) + (size_t)kCT * words_of(D, v.v_bits);
  return sizeof(float) * words;
}

// Splits are whole chunks: about 1024 workgroups, at least one chunk each.
int ext_decode_parts(const kvq_ext_view& v, int n_splits) {
  const int64_t chunks = (v.n_tok + kCT - 1) / kCT;
  int64_t p = n_splits;
  if (p <= 0) {
    const int64_t streams = (int64_t)v.batch * v.kv_heads;
    p = (1024 + streams - 1) / streams;
  }
  if (p > chunks) p = chunks;
  if (p < 1) p = 1;
  if (p > 4096) p = 4096;
  return (int)p;
}

template <int D>
hipError_t launch_decode_ext_d(const ExtArgs& a, const void* q, int f16, dim3 grid, size_t lds,
                               hipStream_t s) {
  const void* fn = f16 ? (const void*)decode_ext_kernel<uint16_t, D>
                       : (const void*)decode_ext_kernel<float, D>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (f16)
    decode_ext_kernel<uint16_t, D><<<grid, kThreads, lds, s>>>(a, (const uint16_t*)q);
  else
    decode_ext_kernel<float, D><<<grid, kThreads, lds, s>>>(a, (const float*)q);
  return hipGetLastError();
}

hipError_t launch_decode_ext(const kvq_ext_view& v, const ExtLut& lk, const ExtLut& lv,
                             const void* q, int f16, int Hq, float sm_scale, float* partials,
                             int n_parts, float* out, hipStream_t s) {
  const int M = v.v_qjl ? v.qjl_m : 0;
  const int64_t chunks = (v.n_tok + kCT - 1) / kCT;
  const int64_t per = (chunks + n_parts - 1) / n_parts * kCT;
  ExtArgs a{v, lk, lv, Hq, sm_scale * kLog2e, partials, n_parts, v.head_dim + 2 + M, per};
  const size_t lds = ext_decode_lds(v, Hq);
  dim3 grid((unsigned)n_parts, (unsigned)v.kv_heads, (unsigned)v.batch);
  hipError_t e;
  switch (v.head_dim) {
    case 32: e = launch_decode_ext_d<32>(a, q, f16, grid, lds, s); break;
    case 64: e = launch_decode_ext_d<64>(a, q, f16, grid, lds, s); break;
    case 128: e = launch_decode_ext_d<128>(a, q, f16, grid, lds, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  merge_ext_kernel<<<dim3((unsigned)(v.batch * Hq)), kThreads, sizeof(float) * (size_t)n_parts, s>>>(
      partials, v.head_dim, M, n_parts, a.rec, v.jl, v.v_rotated, out);
  return hipGetLastError();
}

}  // namespace kvq
