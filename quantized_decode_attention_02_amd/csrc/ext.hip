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
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ inline float h2f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }

// Wave-wide max and sum: four DPP row rotations (8, 4, 2, 1 lanes) leave
// every lane of a 16-lane row with its row's result; the four rows are
// combined through readlane (a few cycles each, against the LDS round trip
// of a shuffle per step).
template <int CTRL>
__device__ inline float dppf(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ inline float rdl(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ inline float wave_max64(float x) {
  x = fmaxf(x, dppf<0x128>(x));
  x = fmaxf(x, dppf<0x124>(x));
  x = fmaxf(x, dppf<0x122>(x));
  x = fmaxf(x, dppf<0x121>(x));
  return fmaxf(fmaxf(rdl(x, 0), rdl(x, 16)), fmaxf(rdl(x, 32), rdl(x, 48)));
}
__device__ inline float wave_sum64(float x) {
  x += dppf<0x128>(x);
  x += dppf<0x124>(x);
  x += dppf<0x122>(x);
  x += dppf<0x121>(x);
  return (rdl(x, 0) + rdl(x, 16)) + (rdl(x, 32) + rdl(x, 48));
}
// Sum over the four lanes of a quad (DPP quad permutations).
__device__ inline float quad_sum(float x) {
  x += dppf<0xB1>(x);  // quad_perm [1, 0, 3, 2]
  x += dppf<0x4E>(x);  // quad_perm [2, 3, 0, 1]
  return x;
}
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
  // sign of <S_i, r> for every row r and sketch row i, in float64: thread
  // (row tid / 8, lane group ig = tid % 8) accumulates sketch rows
  // ih + 32 k + 4 ig + j (j < 4, k < 4) of a half of at most 128 sketch
  // rows, over blocks of 32 channels of S staged transposed in LDS (rows
  // of 132 floats); the 4-bit groups of a word are OR-ed over the row's
  // eight lanes.
  const int mw = m / 32;
  float* St = sc;  // [32][132], free after the codes
  const int rr = tid >> 3, ig = tid & 7;
  for (int ih = 0; ih < m; ih += 128) {
    const int mi = min(128, m - ih);
    double dot[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) dot[k][j] = 0.0;
    for (int cb = 0; cb < d; cb += 32) {
      const int nc = min(32, d - cb);
      __syncthreads();
      for (int e = tid; e < 32 * mi; e += kThreads) {
        const int i = e >> 5, cc = e & 31;
        St[cc * 132 + i] = cc < nc ? S[(int64_t)(ih + i) * d + cb + cc] : 0.0f;
      }
      __syncthreads();
      if (rr < rows) {
        for (int cc = 0; cc < nc; ++cc) {
          const double xr = rs[rr * d + cb + cc];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if (32 * k < mi) {
              const float4v s4 = *(const float4v*)&St[cc * 132 + 32 * k + 4 * ig];
#pragma unroll
              for (int j = 0; j < 4; ++j) dot[k][j] = __builtin_fma((double)s4[j], xr, dot[k][j]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (32 * k < mi) {
        uint32_t nib = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) nib |= (dot[k][j] >= 0.0 ? 1u : 0u) << (4 * ig + j);
        nib |= __shfl_xor(nib, 1);
        nib |= __shfl_xor(nib, 2);
        nib |= __shfl_xor(nib, 4);
        if (ig == 0 && rr < rows) sketch[(mat * n_tok + r0 + rr) * mw + ih / 32 + k] = nib;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode over an extended view: one workgroup per (split, KV head, batch);
// splits are whole 64-token chunks.  Per chunk, every load goes to LDS in one
// pass (code rows, the key scales of its at most two groups, value scales,
// sketch words transposed to word-major, norms).  Thread tid dequantizes
// channel c = tid % D of the tokens tid / D, tid / D + 256 / D, ... (the
// field's word and shift, the channel's key scales and the codebook are
// fixed per thread or per chunk) into fp32 rows padded to D + 16 floats, and
// the group's outliers are added.  Four lanes per token score it against
// every query head with 16-byte reads of key rows and queries (lane
// quarter qd takes channels 16 i + 4 qd .. + 3).  A wave per head runs the
// online softmax over the chunk's tokens (one token per lane).  The values
// are dequantized into the same rows, then thread (channel c, slice tid / D)
// accumulates every head's weighted sum over its slice of the chunk's
// tokens, reading four weights per 16-byte load; the slices are added at
// the end.  The sketch's per-head sign sums z[h][j] = sum_t p gamma b are a
// product of the weights (hi and lo fp16 limbs of p * gamma times a power of
// two per chunk) with the +-1 sketch signs, on matrix cores: rows 2 h + limb,
// 32 tokens per step, 16 sketch rows j per block, fp32 accumulation.
// Partial record per (batch, head, split): m (log2 units), l, o[D], z[M]
// (M = m of the sketch, 0 without one).
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

constexpr int kExtPad = 16;  // floats of padding per fp32 row (16-byte rows, b128 reads)

// The next chunk's words of one contiguous source range, held in registers
// while the current chunk is computed: thread tid takes words tid + 256 k,
// k < CAP; words past CAP * 256 are copied directly when stored.
template <int CAP>
struct Staged {
  uint32_t r[CAP];
  __device__ void load(const uint32_t* src, int cnt) {
#pragma unroll
    for (int k = 0; k < CAP; ++k) {
      const int i = threadIdx.x + kThreads * k;
      r[k] = i < cnt ? src[i] : 0u;
    }
  }
  // dst[map(i)] = word i
  template <typename F>
  __device__ void store(const uint32_t* src, int cnt, uint32_t* dst, F map) const {
#pragma unroll
    for (int k = 0; k < CAP; ++k) {
      const int i = threadIdx.x + kThreads * k;
      if (i < cnt) dst[map(i)] = r[k];
    }
    for (int i = threadIdx.x + kThreads * CAP; i < cnt; i += kThreads) dst[map(i)] = src[i];
  }
};

// Dequantize a chunk's code rows into fp32 rows of LDS: thread tid takes
// the (token, word) items tid, tid + 256, ... of n rows of words_of(D, BITS)
// words and writes every field of its word: level (codebook entry lut[code],
// or code - off) times the scale sc(t, channel).
template <int BITS, bool NUQ, int D, int DP, typename SC>
__device__ inline void dequant_rows(const uint32_t* cw, int n, float* buf, const float* lut,
                                    float off, SC sc) {
  constexpr int FPW = 32 / BITS, WR = (D + FPW - 1) / FPW;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  for (int i = threadIdx.x; i < n * WR; i += kThreads) {
    const int t = i / WR, w = i - t * WR;
    const uint32_t word = cw[i];
    float* row = buf + t * DP + w * FPW;
#pragma unroll
    for (int f = 0; f < FPW; ++f) {
      if (w * FPW + f < D) {
        const uint32_t code = (word >> (f * BITS)) & MASK;
        const float lvl = NUQ ? lut[code] : (float)code - off;
        row[f] = lvl * sc(t, w * FPW + f);
      }
    }
  }
}
template <int D, int DP, typename SC>
__device__ inline void dequant_rows_any(int bits, bool nuq, const uint32_t* cw, int n, float* buf,
                                        const float* lut, float off, SC sc) {
  if (nuq) {
    if (bits == 2) dequant_rows<2, true, D, DP>(cw, n, buf, lut, off, sc);
    else if (bits == 3) dequant_rows<3, true, D, DP>(cw, n, buf, lut, off, sc);
    else dequant_rows<4, true, D, DP>(cw, n, buf, lut, off, sc);
  } else {
    if (bits == 2) dequant_rows<2, false, D, DP>(cw, n, buf, lut, off, sc);
    else if (bits == 3) dequant_rows<3, false, D, DP>(cw, n, buf, lut, off, sc);
    else if (bits == 4) dequant_rows<4, false, D, DP>(cw, n, buf, lut, off, sc);
    else dequant_rows<8, false, D, DP>(cw, n, buf, lut, off, sc);
  }
}

template <typename QT, int D>
__global__ void __launch_bounds__(kThreads, 3)  // three waves per SIMD, as the LDS allows
decode_ext_kernel(ExtArgs a, const QT* __restrict__ q) {
  constexpr int Dp = D + kExtPad;
  constexpr int TPT = kThreads / D;       // dequant token lanes; weighted-sum slices
  constexpr int TS = kCT / TPT;           // tokens per slice
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
  float* ps = buf + kCT * Dp;             // [g][kCT] weights
  float* pg = ps + g * kCT;               // [g][kCT] weight * gamma * 2^-e (sketch)
  float* st = pg + g * kCT;               // [4][8]: m, l, alpha; st[24] = 2^e
  float* gam = st + 32;                   // [kCT]
  float* ksl = gam + kCT;                 // [2][D]: scales of the chunk's key groups
  float* vsl = ksl + 2 * D;               // [kCT][ngv]
  uint32_t* skT = (uint32_t*)(vsl + ((kCT * ngv + 3) & ~3));  // [MW][kCT]
  uint32_t* kcw = skT + kCT * MW;         // [kCT][kw_row]
  uint32_t* vcw = kcw + kCT * kw_row;     // [kCT][vw_row]
  uint32_t* kol = vcw + kCT * vw_row;     // [2][D * k_n_out]: the groups' key outliers
  uint32_t* vol = kol + 2 * D * v.k_n_out;  // [kCT][ngv * v_n_out]: value outliers
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lq = lane >> 4, ln = lane & 15;
  const int part = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int64_t s = (int64_t)b * v.kv_heads + kvh;
  const int64_t N = v.n_tok;
  const int64_t t_lo = min(N, (int64_t)part * a.per), t_hi = min(N, t_lo + a.per);
  const int G = v.group_tok;

  // per-thread constants of the dequant: channel c of tokens t0 + TPT j;
  // the weighted sums: channel c of tokens t0 * TS .. t0 * TS + TS - 1
  const int c = tid % D, t0 = tid / D;
  int gv_shift = 0;  // group_ch divides D, a power of two
  while ((1 << gv_shift) < v.group_ch) ++gv_shift;
  const float koff = v.k_nuq ? 0.0f : (float)(qmax_of(kb) + 1);
  const float voff = v.v_nuq ? 0.0f : (float)(qmax_of(vb) + 1);

  if (tid < 16) {
    lut[tid] = v.k_nuq ? a.lk.lvl[tid] : 0.0f;
    lut[16 + tid] = v.v_nuq ? a.lv.lvl[tid] : 0.0f;
  }
  for (int i = tid; i < g * D; i += kThreads)
    qs[i] = ldx(q, ((int64_t)b * a.Hq + kvh * g) * D + i) * a.qscale;
  if (tid < 8) {
    st[tid] = -INFINITY;
    st[8 + tid] = 0.0f;
  }
  float o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = 0.0f;
  // sketch sums: this wave's blocks of 16 sketch rows, nb = wave + 4 i
  float4v zacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) zacc[i] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
  __syncthreads();

  const uint32_t* kc = v.k_codes + s * v.k_codes_stride;
  const float* ks = v.k_scales + s * v.k_scales_stride;
  const uint32_t* ko = v.k_n_out ? v.k_outliers + s * v.k_outliers_stride : nullptr;
  const uint32_t* vc = v.v_codes + s * v.v_codes_stride;
  const float* vs = v.v_scales + s * v.v_scales_stride;
  const uint32_t* vo = v.v_n_out ? v.v_outliers + s * v.v_outliers_stride : nullptr;

  // Chunk loads: issued one chunk ahead into registers (so they overlap the
  // current chunk's work), stored to LDS when the chunk starts.
  const int per_g = D * v.k_n_out, per_t = ngv * v.v_n_out;
  // (capacities for up to 4-bit codes, four value groups, four sketch
  // words and one outlier per vector; larger views copy the rest directly)
  Staged<(D >= 64 ? D / 32 : 1)> st_k, st_v;
  Staged<1> st_ks, st_gam, st_vs, st_sk, st_ko, st_vo;
  struct ChunkSrc {
    const uint32_t *k, *v, *ks, *vs, *sk, *gam, *ko, *vo;
    int nk, nv, nks, nvs, nsk, ngam, nko, nvo;
  };
  // chunk c0 starts at token r0 of key group g0 (chunks start at multiples
  // of 64 and G is a multiple of 32, so a chunk spans at most two groups;
  // g0 and r0 are carried from chunk to chunk instead of divided out)
  auto chunk_src = [&](int64_t c0, int64_t g0, int r0) {
    const int n = (int)min((int64_t)kCT, t_hi - c0);
    const int ng = (r0 + n > G) ? 2 : 1;
    ChunkSrc cs;
    cs.k = kc + c0 * kw_row;                       cs.nk = n * kw_row;
    cs.v = vc + c0 * vw_row;                       cs.nv = n * vw_row;
    cs.ks = (const uint32_t*)(ks + g0 * D);        cs.nks = ng * D;
    cs.vs = (const uint32_t*)(vs + c0 * ngv);      cs.nvs = n * ngv;
    cs.sk = M ? v.v_sketch + s * v.v_sketch_stride + c0 * MW : nullptr;
    cs.nsk = M ? n * MW : 0;
    cs.gam = M ? (const uint32_t*)(v.v_rnorm + s * v.v_rnorm_stride + c0) : nullptr;
    cs.ngam = M ? n : 0;
    cs.ko = ko ? ko + g0 * per_g : nullptr;        cs.nko = ko ? ng * per_g : 0;
    cs.vo = vo ? vo + c0 * per_t : nullptr;        cs.nvo = vo ? n * per_t : 0;
    return cs;
  };
  auto stage_load = [&](const ChunkSrc& cs) {
    st_k.load(cs.k, cs.nk);
    st_v.load(cs.v, cs.nv);
    st_ks.load(cs.ks, cs.nks);
    st_vs.load(cs.vs, cs.nvs);
    st_sk.load(cs.sk, cs.nsk);
    st_gam.load(cs.gam, cs.ngam);
    st_ko.load(cs.ko, cs.nko);
    st_vo.load(cs.vo, cs.nvo);
  };
  auto ident = [](int i) { return i; };
  int64_t g_cur = t_lo / G;
  int r_cur = (int)(t_lo - g_cur * G);
  ChunkSrc cur = chunk_src(t_lo, g_cur, r_cur);
  if (t_lo < t_hi) stage_load(cur);

  for (int64_t c0 = t_lo; c0 < t_hi; c0 += kCT) {
    const int n = (int)min((int64_t)kCT, t_hi - c0);
    const int64_t g0 = g_cur;
    const int r0 = r_cur;                          // chunk start within its group
    r_cur += kCT;
    while (r_cur >= G) {
      r_cur -= G;
      ++g_cur;
    }
    const int ng_chunk = (r0 + n > G) ? 2 : 1;
    // ---- this chunk's words into LDS (sketch words transposed to
    //      word-major), then the next chunk's loads
    st_k.store(cur.k, cur.nk, kcw, ident);
    st_v.store(cur.v, cur.nv, vcw, ident);
    st_ks.store(cur.ks, cur.nks, (uint32_t*)ksl, ident);
    st_vs.store(cur.vs, cur.nvs, (uint32_t*)vsl, ident);
    st_sk.store(cur.sk, cur.nsk, skT, [&](int i) { return (i % MW) * kCT + i / MW; });
    st_gam.store(cur.gam, cur.ngam, (uint32_t*)gam, ident);
    st_ko.store(cur.ko, cur.nko, kol, ident);
    st_vo.store(cur.vo, cur.nvo, vol, ident);
    if (c0 + kCT < t_hi) {
      cur = chunk_src(c0 + kCT, g_cur, r_cur);
      stage_load(cur);
    }
    __syncthreads();
    // ---- keys of the chunk: level (or centred code) times the channel's
    //      scale of the token's group
    {
      const int t_split = G - r0;  // first token of the second group
      dequant_rows_any<D, Dp>(kb, v.k_nuq, kcw, n, buf, lut, koff, [&](int t, int ch) {
        return ksl[(t >= t_split ? D : 0) + ch];
      });
    }
    if (ko) {
      __syncthreads();
      for (int gi = 0; gi < ng_chunk; ++gi) {
        for (int i = tid; i < per_g; i += kThreads) {
          const uint32_t e = kol[gi * per_g + i];
          if ((e & 0x7FFFu) == 0) continue;               // +-0: nothing to add
          const int64_t tok = (g0 + gi) * G + (e >> 16);
          if (tok < c0 || tok >= c0 + n) continue;
          buf[(tok - c0) * Dp + i / v.k_n_out] += h2f((uint16_t)(e & 0xFFFFu));
        }
      }
    }
    __syncthreads();
    // ---- scores: lane (token tid / 4, quarter qd = tid % 4) sums channels
    //      16 i + 4 qd .. + 3 for every head
    {
      const int t = tid >> 2, qd = tid & 3;
      float acc[8];
#pragma unroll
      for (int h = 0; h < 8; ++h) acc[h] = 0.0f;
      if (t < n) {
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
          const int cc = 16 * i + 4 * qd;
          const float4v kv = *(const float4v*)&buf[t * Dp + cc];
#pragma unroll
          for (int h = 0; h < 8; ++h) {
            if (h < g) {
              const float4v qv = *(const float4v*)&qs[h * D + cc];
              acc[h] = __builtin_fmaf(qv[0], kv[0], acc[h]);
              acc[h] = __builtin_fmaf(qv[1], kv[1], acc[h]);
              acc[h] = __builtin_fmaf(qv[2], kv[2], acc[h]);
              acc[h] = __builtin_fmaf(qv[3], kv[3], acc[h]);
            }
          }
        }
      }
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        if (h < g) {
          float x = acc[h];
          x = quad_sum(x);
          if (qd == 0 && t < n) ps[h * kCT + t] = x;
        }
      }
    }
    __syncthreads();
    // ---- online softmax: a wave per head (lane = token); with the sketch,
    //      the weights times gamma times 2^-e, e the exponent of the chunk's
    //      largest gamma
    float gsig = 1.0f;
    if (M) {
      float gm = lane < n ? gam[lane] : 0.0f;
      gm = wave_max64(gm);
      int e = gm > 0.0f ? (int)((__builtin_bit_cast(uint32_t, gm) >> 23) & 0xFF) - 127 : 0;
      e = e < -100 ? -100 : (e > 100 ? 100 : e);
      gsig = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);
      if (tid == 0) st[24] = __builtin_bit_cast(float, (uint32_t)(127 + e) << 23);
    }
    for (int h = wave; h < g; h += kThreads / 64) {
      const float x = lane < n ? ps[h * kCT + lane] : -INFINITY;
      float mx = x;
      mx = wave_max64(mx);
      const float m_old = st[h];
      const float m_new = fmaxf(m_old, mx);
      const float p = lane < n ? exp2f(x - m_new) : 0.0f;
      float ls = p;
      ls = wave_sum64(ls);
      const float alpha = exp2f(m_old - m_new);
      ps[h * kCT + lane] = p;
      if (M) pg[h * kCT + lane] = lane < n ? p * gam[lane] * gsig : 0.0f;
      if (lane == 0) {
        st[h] = m_new;
        st[8 + h] = st[8 + h] * alpha + ls;
        st[16 + h] = alpha;
      }
    }
    // ---- values of the chunk (into the key rows: the scores are done);
    //      rows past n are cleared (their weights are 0)
    dequant_rows_any<D, Dp>(vb, v.v_nuq, vcw, n, buf, lut + 16, voff, [&](int t, int ch) {
      return vsl[t * ngv + (ch >> gv_shift)];
    });
    for (int i = tid; i < (kCT - n) * D; i += kThreads) buf[(n + i / D) * Dp + i % D] = 0.0f;
    if (vo) {
      __syncthreads();
      for (int i = tid; i < n * per_t; i += kThreads) {
        const int t = i / per_t, r = i - t * per_t;
        const uint32_t e = vol[i];
        if ((e & 0x7FFFu) == 0) continue;
        const int cc = (r / v.v_n_out) * v.group_ch + (int)(e >> 16);
        buf[t * Dp + cc] += h2f((uint16_t)(e & 0xFFFFu));
      }
    }
    __syncthreads();
    // ---- weighted sums: channel c over this thread's token slice, every
    //      head (four weights per 16-byte load)
    {
      const int tb = t0 * TS;
#pragma unroll
      for (int h = 0; h < 8; ++h)
        if (h < g) o[h] *= st[16 + h];
      if (tb < n) {
#pragma unroll
        for (int t = tb; t < tb + TS; t += 4) {
          const float v0 = buf[t * Dp + c], v1 = buf[(t + 1) * Dp + c];
          const float v2 = buf[(t + 2) * Dp + c], v3 = buf[(t + 3) * Dp + c];
#pragma unroll
          for (int h = 0; h < 8; ++h) {
            if (h < g) {
              const float4v w4 = *(const float4v*)&ps[h * kCT + t];
              o[h] = __builtin_fmaf(w4[0], v0, o[h]);
              o[h] = __builtin_fmaf(w4[1], v1, o[h]);
              o[h] = __builtin_fmaf(w4[2], v2, o[h]);
              o[h] = __builtin_fmaf(w4[3], v3, o[h]);
            }
          }
        }
      }
    }
    // ---- sketch sums on matrix cores: A = weight limbs (row 2 h + limb,
    //      8 tokens per lane group), B = +-1 signs of sketch row j = 16 nb +
    //      column; two 32-token steps per chunk
    if (M) {
      half8 A[2];
      const int ah = ln >> 1, limb = ln & 1;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        float x[8];
        if (ah < g) {
          const float4v x0 = *(const float4v*)&pg[ah * kCT + 32 * k2 + 8 * lq];
          const float4v x1 = *(const float4v*)&pg[ah * kCT + 32 * k2 + 8 * lq + 4];
          x[0] = x0[0]; x[1] = x0[1]; x[2] = x0[2]; x[3] = x0[3];
          x[4] = x1[0]; x[5] = x1[1]; x[6] = x1[2]; x[7] = x1[3];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const _Float16 hi = (_Float16)x[e];
          A[k2][e] = limb ? (_Float16)(x[e] - (float)hi) : hi;
        }
      }
      const float ginv = st[24];
      float al[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = (4 * lq + r) >> 1;
        al[r] = h < g ? st[16 + h] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nb = wave + 4 * i;
        if (nb < M / 16) {
          const int j = 16 * nb + ln;
          const uint32_t* wrow = skT + (j >> 5) * kCT;
          const int bit = j & 31;
          float4v zc = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const u32x4 w0 = *(const u32x4*)&wrow[32 * k2 + 8 * lq];
            const u32x4 w1 = *(const u32x4*)&wrow[32 * k2 + 8 * lq + 4];
            u32x4 bw;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t wa = e < 2 ? w0[2 * e] : w1[2 * e - 4];
              const uint32_t wb = e < 2 ? w0[2 * e + 1] : w1[2 * e - 3];
              // +1 (0x3C00) where the bit is set, -1 (0xBC00) where clear
              bw[e] = 0xBC00BC00u ^ (((wa >> bit) & 1u) << 15) ^ (((wb >> bit) & 1u) << 31);
            }
            zc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[k2], __builtin_bit_cast(half8, bw), zc,
                                                         0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) zacc[i][r] = __builtin_fmaf(zacc[i][r], al[r], zc[r] * ginv);
        }
      }
    }
    __syncthreads();
  }
  // ---- partial record: m, l; o summed over the slices; z from the limb rows
  float* out = a.partials + (((int64_t)b * a.Hq + kvh * g) * a.n_parts + part) * a.rec;
  const int64_t hstride = (int64_t)a.n_parts * a.rec;
  if (tid < g) {
    out[tid * hstride] = st[tid];
    out[tid * hstride + 1] = st[8 + tid];
  }
  float* red = buf;  // [TPT][8][D]
#pragma unroll
  for (int h = 0; h < 8; ++h)
    if (h < g) red[(t0 * 8 + h) * D + c] = o[h];
  __syncthreads();
  for (int h = t0; h < g; h += TPT) {
    float sum = 0.0f;
#pragma unroll
    for (int sl = 0; sl < TPT; ++sl) sum += red[(sl * 8 + h) * D + c];
    out[h * hstride + 2 + c] = sum;
  }
  if (M) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int nb = wave + 4 * i;
      if (nb < M / 16) {
        const int j = 16 * nb + ln;
        const int h0 = 2 * lq, h1 = 2 * lq + 1;
        if (h0 < g) out[h0 * hstride + 2 + D + j] = zacc[i][0] + zacc[i][1];
        if (h1 < g) out[h1 * hstride + 2 + D + j] = zacc[i][2] + zacc[i][3];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core form of the extended decode (g * D / Gv <= 16 query-head and
// value-group columns, g <= 8).  Same workgroup, split and chunk structure
// as decode_ext_kernel; per 64-token chunk:
//  - dequant: thread tid decodes its staged code words (key and value rows,
//    loaded one chunk ahead) field by field into fp16 levels through a
//    per-kind table of the 2^bits levels (codebook entries, or code - off;
//    both exact in fp16): keys into rows Lk[t][c], values transposed into
//    LvT[c][t];
//  - scores on v_mfma_f32_16x16x32_f16: wave w takes tokens 16 w .. + 15;
//    A = Q' = q * sm_scale * log2(e) * (key scale of the token's group) *
//    2^(13 - e_q - e_k) as hi and lo fp16 limbs (rows 2 h + limb, rebuilt
//    when the wave's group changes), B = the key levels; the key outliers
//    are added to the scores with LDS atomics (q times the exact value);
//  - softmax: a wave per head; the value operand P'[h * ngv + grp][t] =
//    p * v_scale * 2^(14 - e_v) in fp16 (e_v the chunk's largest value-scale
//    exponent), so P' < 2^15;
//  - values on v_mfma_f32_16x16x32_f16: wave w takes channel blocks w,
//    w + 4 (A = LvT rows, B = P'), a fresh accumulator per chunk folded into
//    the running one as o = o * alpha + o_chunk * 2^(e_v - 14); column
//    (h, grp) is kept only on the channels of group grp; value outliers go
//    to an fp32 LDS accumulator (scaled by alpha per chunk) with atomics;
//  - sketch sums as in decode_ext_kernel.
// ---------------------------------------------------------------------------
constexpr int kLkPad = 8;    // halves of padding per fp16 key row
constexpr int kQbPad = 8;    // halves of padding per Q' row
constexpr int kLvStride = kCT + 8;  // halves per transposed value row and P' row
constexpr int kLvSpare = 8;  // spare channel rows past D of the transposed values

// Key code words of a chunk to fp16 level rows (D + kLkPad halves per
// token) through the tables: word i is token i / WR, word i % WR; the first
// CK words of each thread come from registers, the rest from memory.  Codes
// of up to 4 bits go two neighbouring fields at a time through the pair
// table.  A row's last word may hold unused fields past D (3-bit codes):
// their levels land in the row's padding, which no operand reads, so no
// field needs a bounds test.
template <int BITS, int D, int CK>
__device__ inline void deq_keys(const uint32_t (&r)[CK], const uint32_t* src, int cnt,
                                const uint16_t* lut, const uint32_t* lut2, uint16_t* dst) {
  constexpr int FPW = 32 / BITS, WR = (D + FPW - 1) / FPW;
  constexpr uint32_t MASK = (1u << BITS) - 1u, PMASK = (1u << (2 * BITS)) - 1u;
  static_assert(WR * FPW - D <= kLkPad, "fields past D must fit the row padding");
  auto one = [&](int i, uint32_t word) {
    const int t = i / WR, w = i - t * WR;
    uint16_t* o = dst + t * (D + kLkPad) + w * FPW;
    if (BITS <= 4) {
#pragma unroll
      for (int f = 0; f < FPW; f += 2) *(uint32_t*)(o + f) = lut2[(word >> (f * BITS)) & PMASK];
    } else {
#pragma unroll
      for (int f = 0; f < FPW; ++f) o[f] = lut[(word >> (f * BITS)) & MASK];
    }
  };
  // one word at a time (unrolled, every field's table read would be in
  // flight at once)
#pragma unroll 1
  for (int k = 0; k < CK; ++k) {
    uint32_t wk = 0;
#pragma unroll
    for (int k2 = 0; k2 < CK; ++k2)
      if (k2 == k) wk = r[k2];
    const int i = threadIdx.x + kThreads * k;
    if (i < cnt) one(i, wk);
  }
  for (int i = threadIdx.x + kThreads * CK; i < cnt; i += kThreads) one(i, src[i]);
}
template <int D, int CK>
__device__ inline void deq_keys_any(int bits, const uint32_t (&r)[CK], const uint32_t* src,
                                    int cnt, const uint16_t* lut, const uint32_t* lut2,
                                    uint16_t* dst) {
  switch (bits) {
    case 2: deq_keys<2, D, CK>(r, src, cnt, lut, lut2, dst); break;
    case 3: deq_keys<3, D, CK>(r, src, cnt, lut, lut2, dst); break;
    case 4: deq_keys<4, D, CK>(r, src, cnt, lut, lut2, dst); break;
    default: deq_keys<8, D, CK>(r, src, cnt, lut, lut2, dst); break;
  }
}

// Value code words by token pairs: pair item j is word w = j % WP of tokens
// 2p and 2p + 1 (p = j / WP, WP the power of two at or above the words per
// row, items with w past the row idle), so that the transposed level rows
// (kLvStride halves per channel) take both tokens of a channel in one
// 4-byte store.  The second word of a pair past the chunk's n tokens reads
// as 0 and its level is stored as 0.  Unused fields past D land in the
// spare channel rows.
__host__ __device__ constexpr int ceil_log2(int x) { return x <= 1 ? 0 : 1 + ceil_log2((x + 1) / 2); }
template <int CP>
__device__ inline void load_vpairs(uint32_t (&r)[CP][2], const uint32_t* src, int n, int wr,
                                   int lg) {
#pragma unroll
  for (int k = 0; k < CP; ++k) {
    const int j = threadIdx.x + kThreads * k;
    const int p = j >> lg, w = j & ((1 << lg) - 1);
    const int at = 2 * p * wr + w;
    const bool ok = w < wr && 2 * p < n;
    r[k][0] = ok ? src[at] : 0u;
    r[k][1] = (ok && 2 * p + 1 < n) ? src[at + wr] : 0u;
  }
}
template <int BITS, int D, int CP>
__device__ inline void deq_vpairs(const uint32_t (&r)[CP][2], const uint32_t* src, int n,
                                  const uint16_t* lut, const uint32_t* lut2, uint16_t* LvT) {
  constexpr int FPW = 32 / BITS, WR = (D + FPW - 1) / FPW, LG = ceil_log2(WR), WP = 1 << LG;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  static_assert(WR * FPW - D <= kLvSpare, "fields past D must fit the spare rows");
  const int cnt = ((n + 1) >> 1) * WP;
  auto one = [&](int j, uint32_t wa, uint32_t wb) {
    const int p = j >> LG, w = j & (WP - 1);
    const uint32_t keep = 2 * p + 1 < n ? 0xFFFFFFFFu : 0xFFFFu;
    uint16_t* o = LvT + w * FPW * kLvStride + 2 * p;
#pragma unroll
    for (int f = 0; f < FPW; ++f) {
      const uint32_t ca = (wa >> (f * BITS)) & MASK, cb = (wb >> (f * BITS)) & MASK;
      const uint32_t lv = BITS <= 4 ? lut2[ca | cb << BITS] : lut[ca] | (uint32_t)lut[cb] << 16;
      *(uint32_t*)(o + f * kLvStride) = lv & keep;
    }
  };
#pragma unroll 1
  for (int k = 0; k < CP; ++k) {
    uint32_t wa = 0, wb = 0;
#pragma unroll
    for (int k2 = 0; k2 < CP; ++k2)
      if (k2 == k) {
        wa = r[k2][0];
        wb = r[k2][1];
      }
    const int j = threadIdx.x + kThreads * k;
    if (j < cnt && (WP == WR || (j & (WP - 1)) < WR)) one(j, wa, wb);
  }
  for (int j = threadIdx.x + kThreads * CP; j < cnt; j += kThreads) {
    const int p = j >> LG, w = j & (WP - 1);
    if (WP != WR && w >= WR) continue;
    const int at = 2 * p * WR + w;
    one(j, src[at], 2 * p + 1 < n ? src[at + WR] : 0u);
  }
}
template <int D, int CP>
__device__ inline void deq_vpairs_any(int bits, const uint32_t (&r)[CP][2], const uint32_t* src,
                                      int n, const uint16_t* lut, const uint32_t* lut2,
                                      uint16_t* LvT) {
  switch (bits) {
    case 2: deq_vpairs<2, D, CP>(r, src, n, lut, lut2, LvT); break;
    case 3: deq_vpairs<3, D, CP>(r, src, n, lut, lut2, LvT); break;
    case 4: deq_vpairs<4, D, CP>(r, src, n, lut, lut2, LvT); break;
    default: deq_vpairs<8, D, CP>(r, src, n, lut, lut2, LvT); break;
  }
}

template <int D>
struct ExtMLayout {
  // byte offsets of the LDS arrays (every one 16-byte aligned)
  int lut, lut2, qs, qb, lk, lv, ps, pg, pv, oc, corr, st, gam, ksl, vsl, skT, vol, total;
  // pair-table entries of a code width (none for 8 bits)
  __host__ __device__ static int pairs(int bits) { return bits <= 4 ? 1 << (2 * bits) : 0; }
  __host__ __device__ ExtMLayout(int g, int ngv, int MW, int per_g, int per_t, int kb, int vb) {
    int o = 0;
    auto take = [&](int bytes) { const int at = o; o += (bytes + 15) & ~15; return at; };
    lut = take(2 * 256 * 2);
    lut2 = take((pairs(kb) + pairs(vb)) * 4);
    qs = take(g * D * 4);
    qb = take(2 * g * (D + kQbPad) * 2);
    lk = take(kCT * (D + kLkPad) * 2);
    lv = take((D + kLvSpare) * kLvStride * 2);
    ps = take(g * kCT * 4);
    pg = take(g * kCT * 4);
    pv = take(16 * kLvStride * 2);
    oc = take(g * D * 4);
    corr = take(per_g > 0 ? g * kCT * 4 : 0);  // only with key outliers
    st = take(32 * 4);
    gam = take(kCT * 4);
    ksl = take(2 * D * 4);
    vsl = take(kCT * ngv * 4);
    skT = take(MW * kCT * 4);
    vol = take(kCT * per_t * 4);
    total = o;
  }
};

// x / d for x >= 0, d >= 1 and x * d < 2^32: the high word of x times
// ceil(2^32 / d) (a 33-bit multiplier: its low word and its top bit).  With
// ceil(2^32 / d) = (2^32 + r) / d, 0 <= r < d, the product is x / d plus
// x r / (d 2^32) < 1 / d, so its integer part is the quotient.
struct FastDiv {
  uint32_t m, top;
  __device__ explicit FastDiv(uint32_t d) {
    const uint64_t mm = ((1ull << 32) + d - 1) / d;
    m = (uint32_t)mm;
    top = (uint32_t)(mm >> 32);
  }
  __device__ int operator()(int x) const {
    return (int)(__umulhi((uint32_t)x, m) + (top ? (uint32_t)x : 0u));
  }
};

__device__ inline int fexp(float x) {  // exponent of a positive normal float
  int e = (int)((__builtin_bit_cast(uint32_t, x) >> 23) & 0xFF) - 127;
  return e < -100 ? -100 : (e > 100 ? 100 : e);
}
__device__ inline float p2(int k) { return __builtin_bit_cast(float, (uint32_t)(127 + k) << 23); }

template <typename QT, int D>
__global__ void __launch_bounds__(kThreads, 3)
decode_ext_mfma_kernel(ExtArgs a, const QT* __restrict__ q) {
  constexpr int KB = D / 32;              // 32-channel blocks of the score contraction
  constexpr int LkS = D + kLkPad;         // halves per key row
  constexpr int kQbS = D + kQbPad;        // halves per Q' row
  extern __shared__ __align__(16) unsigned char smem[];
  const kvq_ext_view& v = a.v;
  const int g = a.Hq / v.kv_heads;
  const int M = v.v_qjl ? v.qjl_m : 0, MW = M / 32;
  const int kb = v.k_bits, vb = v.v_bits;
  const int kw_row = words_of(D, kb), vw_row = words_of(D, vb);
  const int vlg = ceil_log2(vw_row);  // value pair items per token pair: 2^vlg
  // divisions by runtime sizes in the chunk loop
  const FastDiv div_mw(MW > 0 ? MW : 1), div_kno(v.k_n_out > 0 ? v.k_n_out : 1);
  const int ngv = D / v.group_ch;
  const int per_g = D * v.k_n_out, per_t = ngv * v.v_n_out;
  const ExtMLayout<D> L(g, ngv, MW, per_g, per_t, kb, vb);
  const FastDiv div_pt(per_t > 0 ? per_t : 1), div_vno(v.v_n_out > 0 ? v.v_n_out : 1);
  uint16_t* lutK = (uint16_t*)(smem + L.lut);
  uint16_t* lutV = lutK + 256;
  uint32_t* lut2K = (uint32_t*)(smem + L.lut2);  // level pairs: code a | code b << bits
  uint32_t* lut2V = lut2K + ExtMLayout<D>::pairs(kb);
  float* qs = (float*)(smem + L.qs);
  _Float16* qb = (_Float16*)(smem + L.qb);
  uint16_t* Lk = (uint16_t*)(smem + L.lk);
  uint16_t* LvT = (uint16_t*)(smem + L.lv);
  float* ps = (float*)(smem + L.ps);
  float* pg = (float*)(smem + L.pg);
  uint16_t* Pv = (uint16_t*)(smem + L.pv);
  float* OC = (float*)(smem + L.oc);
  float* st = (float*)(smem + L.st);      // m[8], l[8], alpha[8]; [24] 2^e_gamma; [25] 2^(e_v-14)
  float* gam = (float*)(smem + L.gam);
  float* ksl = (float*)(smem + L.ksl);
  float* vsl = (float*)(smem + L.vsl);
  uint32_t* skT = (uint32_t*)(smem + L.skT);
  uint32_t* vol = (uint32_t*)(smem + L.vol);
  float* corr = (float*)(smem + L.corr);  // [g][kCT] key-outlier score terms
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lq = lane >> 4, ln = lane & 15;
  const int part = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int64_t s = (int64_t)b * v.kv_heads + kvh;
  const int64_t N = v.n_tok;
  const int64_t t_lo = min(N, (int64_t)part * a.per), t_hi = min(N, t_lo + a.per);
  const int G = v.group_tok;

  // level tables (fp16 bit patterns), queries, state, cleared P' columns and
  // value-outlier accumulators
  auto level = [&](bool isk, int code) {
    const int bits = isk ? kb : vb;
    float lv = 0.0f;
    if (code < (1 << bits)) {
      const bool nuq = isk ? v.k_nuq : v.v_nuq;
      lv = nuq ? (isk ? a.lk.lvl[code] : a.lv.lvl[code]) : (float)(code - qmax_of(bits) - 1);
    }
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lv);
  };
  for (int u = tid; u < 512; u += kThreads) lutK[u] = (uint16_t)level(u < 256, u & 255);
  {
    const int pk = ExtMLayout<D>::pairs(kb), pv = ExtMLayout<D>::pairs(vb);
    for (int u = tid; u < pk + pv; u += kThreads) {
      const bool isk = u < pk;
      const int uu = isk ? u : u - pk, bits = isk ? kb : vb;
      lut2K[u] = level(isk, uu & ((1 << bits) - 1)) | level(isk, uu >> bits) << 16;
    }
  }
  for (int i = tid; i < g * D; i += kThreads) {
    qs[i] = ldx(q, ((int64_t)b * a.Hq + kvh * g) * D + i) * a.qscale;
    OC[i] = 0.0f;
  }
  for (int i = tid; i < 16 * kLvStride; i += kThreads) Pv[i] = 0;
  if (v.k_n_out)
    for (int i = tid; i < g * kCT; i += kThreads) corr[i] = 0.0f;
  if (tid < 8) {
    st[tid] = -INFINITY;
    st[8 + tid] = 0.0f;
  }
  __syncthreads();
  // largest |q * sm_scale * log2 e| of the workgroup's heads (power of two)
  int eq;
  {
    float mx = 0.0f;
    for (int i = lane; i < g * D; i += 64) mx = fmaxf(mx, fabsf(qs[i]));
    mx = wave_max64(mx);
    eq = mx > 0.0f ? fexp(mx) : 0;
  }

  // per-wave state: Q' limbs of the wave's current key group, value and
  // sketch accumulators
  half8 qa[KB];
  int64_t qgrp = -1;                       // key group of the wave's qa
  int64_t qb_grp = -1;                     // key group of the Q' rows in LDS
  float qsc = 0.0f;                        // 2^(e_q + e_k - 13): score units
  const int nblk = D / 16;                 // 16-channel value blocks
  const int col_head = ln / ngv;           // head of value-operand column ln
  float4v ot[2];                           // blocks wave, wave + 4
#pragma unroll
  for (int i = 0; i < 2; ++i) ot[i] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
  float4v zacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) zacc[i] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  const uint32_t* kc = v.k_codes + s * v.k_codes_stride;
  const float* ks = v.k_scales + s * v.k_scales_stride;
  const uint32_t* ko = v.k_n_out ? v.k_outliers + s * v.k_outliers_stride : nullptr;
  const uint32_t* vc = v.v_codes + s * v.v_codes_stride;
  const float* vs = v.v_scales + s * v.v_scales_stride;
  const uint32_t* vo = v.v_n_out ? v.v_outliers + s * v.v_outliers_stride : nullptr;

  Staged<(D >= 64 ? D / 32 : 1)> st_k;
  constexpr int CP = D >= 128 ? D / 64 : 1;  // value word pairs per thread in registers
  uint32_t rv[CP][2];
  Staged<1> st_ks, st_gam, st_vs, st_sk, st_ko, st_vo;
  struct ChunkSrc {
    const uint32_t *k, *v, *ks, *vs, *sk, *gam, *ko, *vo;
    int n, nk, nv, nks, nvs, nsk, ngam, nko, nvo;
  };
  // chunk c0 starts at token r0 of key group g0 (chunks start at multiples
  // of 64 and G is a multiple of 32, so a chunk spans at most two groups;
  // g0 and r0 are carried from chunk to chunk instead of divided out)
  auto chunk_src = [&](int64_t c0, int64_t g0, int r0) {
    const int n = (int)min((int64_t)kCT, t_hi - c0);
    const int ng = (r0 + n > G) ? 2 : 1;
    ChunkSrc cs;
    cs.n = n;
    cs.k = kc + c0 * kw_row;                       cs.nk = n * kw_row;
    cs.v = vc + c0 * vw_row;                       cs.nv = n * vw_row;
    cs.ks = (const uint32_t*)(ks + g0 * D);        cs.nks = ng * D;
    cs.vs = (const uint32_t*)(vs + c0 * ngv);      cs.nvs = n * ngv;
    cs.sk = M ? v.v_sketch + s * v.v_sketch_stride + c0 * MW : nullptr;
    cs.nsk = M ? n * MW : 0;
    cs.gam = M ? (const uint32_t*)(v.v_rnorm + s * v.v_rnorm_stride + c0) : nullptr;
    cs.ngam = M ? n : 0;
    cs.ko = ko ? ko + g0 * per_g : nullptr;        cs.nko = ko ? ng * per_g : 0;
    cs.vo = vo ? vo + c0 * per_t : nullptr;        cs.nvo = vo ? n * per_t : 0;
    return cs;
  };
  auto stage_load = [&](const ChunkSrc& cs) {
    st_k.load(cs.k, cs.nk);
    load_vpairs<CP>(rv, cs.v, cs.n, vw_row, vlg);
    st_ks.load(cs.ks, cs.nks);
    st_vs.load(cs.vs, cs.nvs);
    st_sk.load(cs.sk, cs.nsk);
    st_gam.load(cs.gam, cs.ngam);
    st_ko.load(cs.ko, cs.nko);
    st_vo.load(cs.vo, cs.nvo);
  };
  auto ident = [](int i) { return i; };
  int64_t g_cur = t_lo / G;
  int r_cur = (int)(t_lo - g_cur * G);
  ChunkSrc cur = chunk_src(t_lo, g_cur, r_cur);
  if (t_lo < t_hi) stage_load(cur);

  for (int64_t c0 = t_lo; c0 < t_hi; c0 += kCT) {
    const int n = (int)min((int64_t)kCT, t_hi - c0);
    const int64_t g0 = g_cur;
    const int r0 = r_cur;                          // chunk start within its group
    r_cur += kCT;
    while (r_cur >= G) {
      r_cur -= G;
      ++g_cur;
    }
    const int ng_chunk = (r0 + n > G) ? 2 : 1;
    // ---- dequant this chunk's code words (staged registers, the rest from
    //      memory) into fp16 levels; the other staged words into LDS; then
    //      the next chunk's loads
    {
      constexpr int CK = D >= 64 ? D / 32 : 1;
      deq_keys_any<D, CK>(kb, st_k.r, cur.k, cur.nk, lutK, lut2K, Lk);
      deq_vpairs_any<D, CP>(vb, rv, cur.v, n, lutV, lut2V, LvT);
      // value columns past the last token pair: zero (their weights are 0;
      // LDS may hold NaN)
      const int ne = (n + 1) & ~1;
      for (int i = tid; i < (kCT - ne) * D; i += kThreads)
        LvT[(i % D) * kLvStride + ne + i / D] = 0;
    }
    st_ks.store(cur.ks, cur.nks, (uint32_t*)ksl, ident);
    st_vs.store(cur.vs, cur.nvs, (uint32_t*)vsl, ident);
    st_sk.store(cur.sk, cur.nsk, skT, [&](int i) {
      const int w = div_mw(i);
      return (i - w * MW) * kCT + w;
    });
    st_gam.store(cur.gam, cur.ngam, (uint32_t*)gam, ident);
    st_vo.store(cur.vo, cur.nvo, vol, ident);
    // key outliers: q . (exact value) into the score terms of their tokens
    for (int i = tid; i < cur.nko; i += kThreads) {
      const uint32_t e = i < kThreads ? st_ko.r[0] : cur.ko[i];
      if ((e & 0x7FFFu) == 0) continue;
      const int gi = i >= per_g ? 1 : 0;  // (at most two groups per chunk)
      const int c = div_kno(i - gi * per_g);
      const int64_t tok = (g0 + gi) * G + (e >> 16) - c0;
      if (tok < 0 || tok >= n) continue;
      const float val = h2f((uint16_t)(e & 0xFFFFu));
      for (int h = 0; h < g; ++h) atomicAdd(&corr[h * kCT + (int)tok], qs[h * D + c] * val);
    }
    if (c0 + kCT < t_hi) {
      cur = chunk_src(c0 + kCT, g_cur, r_cur);
      stage_load(cur);
    }
    __syncthreads();
    // ---- Q' of the chunk's key groups: q times the channel's scale times
    //      2^(13 - e_q - e_k) in hi and lo fp16 limbs, built once per group
    //      by the workgroup into LDS (row 2 h + limb); each wave loads the
    //      rows of its tokens' group as its A operand (rows past 2 g are 0)
    const int tw = 16 * wave;
    const int gw = (r0 + tw >= G) ? 1 : 0;  // the wave's key group: one per 16 tokens
    for (int gi = 0; gi < ng_chunk; ++gi) {
      if (g0 + gi != qb_grp) {
        if (gi > 0) __syncthreads();  // the first group's rows are loaded
        const float* kss = ksl + gi * D;
        float km = 0.0f;
        for (int c = lane; c < D; c += 64) km = fmaxf(km, kss[c]);
        km = wave_max64(km);
        const int ek = km > 0.0f ? fexp(km) : 0;
        const float sg = p2(13 - eq - ek);
        if (tid == 0) st[26] = p2(eq + ek - 13);
        for (int i = tid; i < g * (D / 2); i += kThreads) {
          const int h = i / (D / 2), c = 2 * (i - h * (D / 2));
          const float x0 = qs[h * D + c] * kss[c] * sg, x1 = qs[h * D + c + 1] * kss[c + 1] * sg;
          const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
          *(half2v*)&qb[2 * h * kQbS + c] = (half2v){h0, h1};
          *(half2v*)&qb[(2 * h + 1) * kQbS + c] =
              (half2v){(_Float16)(x0 - (float)h0), (_Float16)(x1 - (float)h1)};
        }
        __syncthreads();
        qb_grp = g0 + gi;
      }
      if (gw == gi && g0 + gi != qgrp) {
        qgrp = g0 + gi;
        qsc = st[26];
#pragma unroll
        for (int k = 0; k < KB; ++k)
          qa[k] = ln < 2 * g ? *(const half8*)&qb[ln * kQbS + 32 * k + 8 * lq] : (half8){};
      }
    }
    // ---- scores: wave w, tokens 16 w .. 16 w + 15
    if (16 * wave < n) {  // (a partial chunk may leave a wave without tokens)
      float4v acc = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const half8 kbv = *(const half8*)&Lk[(tw + ln) * LkS + 32 * k + 8 * lq];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[k], kbv, acc, 0, 0, 0);
      }
      // lane (token tw + ln, lq): rows 4 lq .. 4 lq + 3 = heads 2 lq, 2 lq + 1
      int t = tw + ln, h0 = 2 * lq;
      // (recomputed here: hoisted out of the loop, the LDS addresses below
      // get spilled, and their reload waits for the next chunk's loads)
      asm volatile("" : "+v"(t), "+v"(h0));
      if (t < n) {
        // the outlier terms of this chunk are consumed and cleared here
        float c0v = 0.0f, c1v = 0.0f;
        if (ko) {
          if (h0 < g) {
            c0v = corr[h0 * kCT + t];
            corr[h0 * kCT + t] = 0.0f;
          }
          if (h0 + 1 < g) {
            c1v = corr[(h0 + 1) * kCT + t];
            corr[(h0 + 1) * kCT + t] = 0.0f;
          }
        }
        if (h0 < g) ps[h0 * kCT + t] = (acc[0] + acc[1]) * qsc + c0v;
        if (h0 + 1 < g) ps[(h0 + 1) * kCT + t] = (acc[2] + acc[3]) * qsc + c1v;
      }
    }
    __syncthreads();
    // ---- online softmax: a wave per head (lane = token); P' for the value
    //      operand, gamma-weighted weights for the sketch
    float gsig = 1.0f;
    if (M) {
      float gm = lane < n ? gam[lane] : 0.0f;
      gm = wave_max64(gm);
      const int e = gm > 0.0f ? fexp(gm) : 0;
      gsig = p2(-e);
      if (tid == 0) st[24] = p2(e);
    }
    int ev;
    {
      float vm = 0.0f;
      for (int j = 0; j < ngv; ++j) vm = fmaxf(vm, lane < n ? vsl[lane * ngv + j] : 0.0f);
      vm = wave_max64(vm);
      ev = vm > 0.0f ? fexp(vm) : 0;
    }
    const float vsig = p2(14 - ev);
    if (tid == 0) st[25] = p2(ev - 14);
    for (int h = wave; h < g; h += kThreads / 64) {
      const float x = lane < n ? ps[h * kCT + lane] : -INFINITY;
      float mx = x;
      mx = wave_max64(mx);
      const float m_old = st[h];
      const float m_new = fmaxf(m_old, mx);
      const float p = lane < n ? exp2f(x - m_new) : 0.0f;
      float ls = p;
      ls = wave_sum64(ls);
      const float alpha = exp2f(m_old - m_new);
      if (M) pg[h * kCT + lane] = lane < n ? p * gam[lane] * gsig : 0.0f;
      for (int j = 0; j < ngv; ++j) {
        const float pv = lane < n ? p * vsl[lane * ngv + j] * vsig : 0.0f;
        Pv[(h * ngv + j) * kLvStride + lane] = __builtin_bit_cast(uint16_t, (_Float16)pv);
      }
      if (vo) {
        // the value-outlier side accumulator of head h follows the softmax,
        // then takes this chunk's outliers, p_t * value (this wave only
        // touches row h; lanes that meet on a channel add atomically)
        for (int c = lane; c < D; c += 64) OC[h * D + c] *= alpha;
        for (int i0 = 0; i0 < n * per_t; i0 += 64) {
          const int i = i0 + lane;
          const bool in = i < n * per_t;
          const uint32_t e = in ? vol[i] : 0u;
          const int t = in ? div_pt(i) : 0;
          const float pt = __shfl(p, t);
          if (in && (e & 0x7FFFu) != 0) {
            const int cc = div_vno(i - t * per_t) * v.group_ch + (int)(e >> 16);
            atomicAdd(&OC[h * D + cc], pt * h2f((uint16_t)(e & 0xFFFFu)));
          }
        }
      }
      if (lane == 0) {
        st[h] = m_new;
        st[8 + h] = st[8 + h] * alpha + ls;
        st[16 + h] = alpha;
      }
    }
    __syncthreads();
    // ---- values: channel blocks wave, wave + 4 of 16 channels; columns
    //      (head, value group); two 32-token steps
    {
      const float vun = st[25];
      const int col = ln;
      const float al = (col_head < g) ? st[16 + col_head] : 0.0f;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int jb = wave + 4 * i;
        if (jb < nblk) {
          float4v oc = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const half8 av = *(const half8*)&LvT[(16 * jb + ln) * kLvStride + 32 * k2 + 8 * lq];
            const half8 bv = *(const half8*)&Pv[col * kLvStride + 32 * k2 + 8 * lq];
            oc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, oc, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) ot[i][r] = __builtin_fmaf(ot[i][r], al, oc[r] * vun);
        }
      }
    }
    // ---- sketch sums (as in decode_ext_kernel)
    if (M) {
      half8 A[2];
      const int ah = ln >> 1, limb = ln & 1;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        float x[8];
        if (ah < g) {
          const float4v x0 = *(const float4v*)&pg[ah * kCT + 32 * k2 + 8 * lq];
          const float4v x1 = *(const float4v*)&pg[ah * kCT + 32 * k2 + 8 * lq + 4];
          x[0] = x0[0]; x[1] = x0[1]; x[2] = x0[2]; x[3] = x0[3];
          x[4] = x1[0]; x[5] = x1[1]; x[6] = x1[2]; x[7] = x1[3];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const _Float16 hi = (_Float16)x[e];
          A[k2][e] = limb ? (_Float16)(x[e] - (float)hi) : hi;
        }
      }
      const float ginv = st[24];
      float alr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = (4 * lq + r) >> 1;
        alr[r] = h < g ? st[16 + h] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nb = wave + 4 * i;
        if (nb < M / 16) {
          const int j = 16 * nb + ln;
          const uint32_t* wrow = skT + (j >> 5) * kCT;
          const int bit = j & 31;
          float4v zc = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const u32x4 w0 = *(const u32x4*)&wrow[32 * k2 + 8 * lq];
            const u32x4 w1 = *(const u32x4*)&wrow[32 * k2 + 8 * lq + 4];
            u32x4 bw;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t wa = e < 2 ? w0[2 * e] : w1[2 * e - 4];
              const uint32_t wb = e < 2 ? w0[2 * e + 1] : w1[2 * e - 3];
              bw[e] = 0xBC00BC00u ^ (((wa >> bit) & 1u) << 15) ^ (((wb >> bit) & 1u) << 31);
            }
            zc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[k2], __builtin_bit_cast(half8, bw), zc,
                                                         0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) zacc[i][r] = __builtin_fmaf(zacc[i][r], alr[r], zc[r] * ginv);
        }
      }
    }
    __syncthreads();
  }
  // ---- partial record: m, l; o (column of the channel's value group) plus
  //      the outlier accumulator; z from the limb rows
  float* out = a.partials + (((int64_t)b * a.Hq + kvh * g) * a.n_parts + part) * a.rec;
  const int64_t hstride = (int64_t)a.n_parts * a.rec;
  if (tid < g) {
    out[tid * hstride] = st[tid];
    out[tid * hstride + 1] = st[8 + tid];
  }
  {
    const int col = ln, hc = col / ngv, gc = col % ngv;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int jb = wave + 4 * i;
      if (jb < nblk && hc < g) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = 16 * jb + 4 * lq + r;
          if (c / v.group_ch == gc) out[hc * hstride + 2 + c] = ot[i][r] + OC[hc * D + c];
        }
      }
    }
  }
  if (M) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int nb = wave + 4 * i;
      if (nb < M / 16) {
        const int j = 16 * nb + ln;
        const int h0 = 2 * lq, h1 = 2 * lq + 1;
        if (h0 < g) out[h0 * hstride + 2 + D + j] = zacc[i][0] + zacc[i][1];
        if (h1 < g) out[h1 * hstride + 2 + D + j] = zacc[i][2] + zacc[i][3];
      }
    }
  }
}

// out = turn(O + sqrt(pi/2)/m S^T Z) / L over the partials of one (batch,
// query head): O, Z and L summed with the log-sum-exp weights; turn is the
// normalized Walsh-Hadamard transform when the values were stored rotated.
// Latency-bound (one workgroup per query head), so every pass keeps many
// loads in flight: thread (row group rg, float2 column c) sums partials rg,
// rg + R, ... of its column, and its first kMergeK loads are issued before
// the (m, l) pass that yields their weights.
constexpr int kMergeExtK = 16;
__global__ void __launch_bounds__(kThreads)
merge_ext_kernel(const float* __restrict__ partials, int D, int M, int n_parts, int rec,
                 const float* __restrict__ S, int rotated, float* __restrict__ out) {
  typedef float float2v __attribute__((ext_vector_type(2)));
  __shared__ float red[kThreads / 64];
  __shared__ float acc[kMaxD + 256];
  __shared__ float2v psum[kThreads];
  extern __shared__ float wts[];   // [n_parts]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bh = blockIdx.x;
  const float* p = partials + bh * n_parts * rec;
  const int C = (D + M) / 2;             // float2 columns of (o, z) (D + M is even)
  const int R = kThreads / C;            // row groups (C <= 192)
  const int col = tid % C, rg = tid / C;
  const bool act = rg < R;
  // a part's (o, z) at float offset 2 of its record (rec is even, so the
  // float2 loads are aligned); parts past the end are clamped, their weight
  // is taken as 0
  auto ld = [&](int i) {
    const int ic = i < n_parts ? i : n_parts - 1;
    return *(const float2v*)(p + (int64_t)ic * rec + 2 + 2 * col);
  };
  float2v pre[kMergeExtK];
#pragma unroll
  for (int k = 0; k < kMergeExtK; ++k) pre[k] = act ? ld(rg + R * k) : (float2v){0.0f, 0.0f};
  float mx = -INFINITY;
  for (int i = tid; i < n_parts; i += kThreads)
    if (p[(int64_t)i * rec + 1] > 0.0f) mx = fmaxf(mx, p[(int64_t)i * rec]);
  mx = wave_max64(mx);
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
  L = wave_sum64(L);
  if (lane == 0) red[wave] = L;
  __syncthreads();
  L = red[0] + red[1] + red[2] + red[3];
  if (act) {
    float2v sum = (float2v){0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < kMergeExtK; ++k) {
      const int i = rg + R * k;
      const float w = i < n_parts ? wts[i] : 0.0f;
      sum[0] = __builtin_fmaf(w, pre[k][0], sum[0]);
      sum[1] = __builtin_fmaf(w, pre[k][1], sum[1]);
    }
    for (int i0 = rg + R * kMergeExtK; i0 < n_parts; i0 += R * kMergeExtK) {
      float2v x[kMergeExtK];
#pragma unroll
      for (int k = 0; k < kMergeExtK; ++k) x[k] = ld(i0 + R * k);
#pragma unroll
      for (int k = 0; k < kMergeExtK; ++k) {
        const int i = i0 + R * k;
        const float w = i < n_parts ? wts[i] : 0.0f;
        sum[0] = __builtin_fmaf(w, x[k][0], sum[0]);
        sum[1] = __builtin_fmaf(w, x[k][1], sum[1]);
      }
    }
    psum[tid] = sum;
  }
  __syncthreads();
  for (int j = tid; j < C; j += kThreads) {
    float2v t = (float2v){0.0f, 0.0f};
    for (int r = 0; r < R; ++r) t += psum[r * C + j];
    acc[2 * j] = t[0];
    acc[2 * j + 1] = t[1];
  }
  __syncthreads();
  if (M) {
    // S^T z: thread (d, slice) sums the sketch rows of its slice (every
    // P-th row), kMergeExtK loads in flight; the slices are added in LDS
    const float c = 1.2533141373155003f / (float)M;   // sqrt(pi/2) / m
    float* tq = (float*)psum;                          // [P][D], free again
    const int P = kThreads / D, d = tid % D, sl = tid / D;
    float r0 = 0.0f, r1 = 0.0f;
    for (int i0 = sl; i0 < M; i0 += P * kMergeExtK) {
      float sv[kMergeExtK];
#pragma unroll
      for (int k = 0; k < kMergeExtK; ++k) {
        const int i = i0 + P * k;
        sv[k] = i < M ? S[(int64_t)i * D + d] : 0.0f;
      }
#pragma unroll
      for (int k = 0; k < kMergeExtK; k += 2) {
        const int i = i0 + P * k, i1 = i + P;
        r0 = __builtin_fmaf(sv[k], i < M ? acc[D + i] : 0.0f, r0);
        r1 = __builtin_fmaf(sv[k + 1], i1 < M ? acc[D + i1] : 0.0f, r1);
      }
    }
    tq[sl * D + d] = r0 + r1;
    __syncthreads();
    for (int dd = tid; dd < D; dd += kThreads) {
      float t = 0.0f;
      for (int q = 0; q < P; ++q) t += tq[q * D + dd];
      acc[dd] = __builtin_fmaf(c, t, acc[dd]);
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

// Whether the matrix-core form runs: at most 16 (query head, value group)
// columns of the value product.
bool ext_mfma(const kvq_ext_view& v, int Hq) {
  const int g = Hq / v.kv_heads;
  return g <= 8 && g * (v.head_dim / v.group_ch) <= 16;
}

size_t ext_decode_lds(const kvq_ext_view& v, int Hq) {
  const int g = Hq / v.kv_heads, D = v.head_dim, M = v.v_qjl ? v.qjl_m : 0;
  if (ext_mfma(v, Hq)) {
    const int ngv = D / v.group_ch, per_g = D * v.k_n_out, per_t = ngv * v.v_n_out;
    switch (D) {
      case 32: return (size_t)ExtMLayout<32>(g, ngv, M / 32, per_g, per_t, v.k_bits, v.v_bits).total;
      case 64: return (size_t)ExtMLayout<64>(g, ngv, M / 32, per_g, per_t, v.k_bits, v.v_bits).total;
      default:
        return (size_t)ExtMLayout<128>(g, ngv, M / 32, per_g, per_t, v.k_bits, v.v_bits).total;
    }
  }
  const size_t ngv4 = ((size_t)kCT * (D / v.group_ch) + 3) & ~(size_t)3;
  const size_t words = 32 + (size_t)g * D + (size_t)kCT * (D + kExtPad) + 2 * (size_t)g * kCT +
                       32 + kCT + 2 * (size_t)D + ngv4 + (size_t)kCT * (M / 32) +
                       (size_t)kCT * words_of(D, v.k_bits) + (size_t)kCT * words_of(D, v.v_bits) +
                       2 * (size_t)D * v.k_n_out + (size_t)kCT * (D / v.group_ch) * v.v_n_out;
  return sizeof(float) * words;
}

const void* ext_kernel_fn(const kvq_ext_view& v, int Hq, bool f16) {
  const bool m = ext_mfma(v, Hq);
  switch (v.head_dim) {
    case 32:
      return m ? (f16 ? (const void*)decode_ext_mfma_kernel<uint16_t, 32>
                      : (const void*)decode_ext_mfma_kernel<float, 32>)
               : (f16 ? (const void*)decode_ext_kernel<uint16_t, 32>
                      : (const void*)decode_ext_kernel<float, 32>);
    case 64:
      return m ? (f16 ? (const void*)decode_ext_mfma_kernel<uint16_t, 64>
                      : (const void*)decode_ext_mfma_kernel<float, 64>)
               : (f16 ? (const void*)decode_ext_kernel<uint16_t, 64>
                      : (const void*)decode_ext_kernel<float, 64>);
    default:
      return m ? (f16 ? (const void*)decode_ext_mfma_kernel<uint16_t, 128>
                      : (const void*)decode_ext_mfma_kernel<float, 128>)
               : (f16 ? (const void*)decode_ext_kernel<uint16_t, 128>
                      : (const void*)decode_ext_kernel<float, 128>);
  }
}

// Splits are whole chunks: about 1024 workgroups, at least one chunk each.
// Splits per (batch, KV head): one round of the workgroups the compute
// units hold at once (LDS and registers of the kernel for this view), at
// most one per 64-token chunk.
int ext_decode_parts(const kvq_ext_view& v, int Hq, int n_splits) {
  const int64_t chunks = (v.n_tok + kCT - 1) / kCT;
  int64_t p = n_splits;
  if (p <= 0) {
    static int cus = 0;
    if (cus == 0) {
      int dev = 0, n = 0;
      cus = (hipGetDevice(&dev) == hipSuccess &&
             hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
             n > 0)
                ? n
                : 256;
    }
    const size_t lds = ext_decode_lds(v, Hq);
    const void* fn = ext_kernel_fn(v, Hq, true);
    int wgs = 0;
    if ((lds > 64 * 1024 &&
         hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) !=
             hipSuccess) ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&wgs, fn, kThreads, lds) != hipSuccess ||
        wgs < 1)
      wgs = 1;
    const int64_t streams = (int64_t)v.batch * v.kv_heads;
    p = ((int64_t)cus * wgs) / streams;
  }
  if (p > chunks) p = chunks;
  if (p < 1) p = 1;
  if (p > 4096) p = 4096;
  return (int)p;
}

hipError_t launch_decode_ext_k(const ExtArgs& a, const void* q, int f16, dim3 grid, size_t lds,
                               hipStream_t s) {
  const void* fn = ext_kernel_fn(a.v, a.Hq, f16 != 0);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  void* args[] = {(void*)&a, (void*)&q};
  return hipLaunchKernel(fn, grid, dim3(kThreads), args, lds, s);
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
  if (v.head_dim != 32 && v.head_dim != 64 && v.head_dim != 128) return hipErrorInvalidValue;
  e = launch_decode_ext_k(a, q, f16, grid, lds, s);
  if (e != hipSuccess) return e;
  merge_ext_kernel<<<dim3((unsigned)(v.batch * Hq)), kThreads, sizeof(float) * (size_t)n_parts, s>>>(
      partials, v.head_dim, M, n_parts, a.rec, v.jl, v.v_rotated, out);
  return hipGetLastError();
}

}  // namespace kvq
