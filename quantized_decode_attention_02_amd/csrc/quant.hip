// Quantize, append (sink / tail / flush), salience, export and synthetic-data
// kernels of libkvq for gfx950.
//
// The rule ("KV quantization axes: why Key and Value need separate
// reasoning", section "What rows and columns mean"): scale = max|x| / qmax,
// code = clip(round_half_even(x / scale), -qmax, qmax), with both divisions
// IEEE float32 (__fdiv_rn) so codes are bit-exact; a zero group (or a scale
// that underflows to 0) uses scale 1; NaN/Inf input sets the sticky error
// flag (closing troubleshooting paragraph of the same page).
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 32;   // token rows staged in LDS per step

__device__ inline float h2f(uint16_t u) {
  return (float)__builtin_bit_cast(_Float16, u);
}
__device__ inline bool finite(float x) { return __builtin_isfinite(x); }

template <typename T> __device__ inline float ld(const T* p, int64_t i);
template <> __device__ inline float ld<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ inline float ld<uint16_t>(const uint16_t* p, int64_t i) {
  return h2f(p[i]);
}

// scale of a group from its absmax m: one IEEE float32 division.
__device__ inline float group_scale(float m, int qmax) {
  float s = __fdiv_rn(m, (float)qmax);
  return (m == 0.0f || s == 0.0f) ? 1.0f : s;
}
// offset-binary code of x under scale s.
__device__ inline uint32_t encode(float x, float s, int qmax) {
  float q = rintf(__fdiv_rn(x, s));
  q = fminf(fmaxf(q, (float)-qmax), (float)qmax);
  return (uint32_t)((int)q + qmax + 1);
}

__device__ inline uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Stateless per-channel quantizer: one workgroup per (matrix, key group).
// Pass 1 reduces the per-channel absmax over the group's tokens; pass 2
// encodes kChunk-row chunks into LDS bytes and packs them into rows.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(kThreads)
quantize_k_kernel(const T* __restrict__ k, int64_t n_tok, int d, int bits,
                  int G, uint32_t* __restrict__ codes,
                  float* __restrict__ scales, uint32_t* err) {
  __shared__ float red[kThreads];
  __shared__ float sc[kMaxD];
  __shared__ uint8_t u8[kChunk * kMaxD];
  const int tid = threadIdx.x;
  const int64_t mat = blockIdx.y;
  const int64_t g = blockIdx.x;
  const int64_t n_groups = (n_tok + G - 1) / G;
  const int64_t t0 = g * G, t1 = min(n_tok, t0 + G);
  const T* x = k + mat * n_tok * d;
  const int qmax = qmax_of(bits);
  const int slices = kThreads / d;
  bool bad = false;
  if (tid < slices * d) {
    int c = tid % d, sl = tid / d;
    float m = 0.0f;
    for (int64_t t = t0 + sl; t < t1; t += slices) {
      float v = ld(x, t * d + c);
      bad |= !finite(v);
      m = fmaxf(m, fabsf(v));
    }
    red[tid] = m;
  }
  __syncthreads();
  if (tid < d) {
    float m = red[tid];
    for (int sl = 1; sl < slices; ++sl) m = fmaxf(m, red[sl * d + tid]);
    float s = group_scale(m, qmax);
    sc[tid] = s;
    scales[(mat * n_groups + g) * d + tid] = s;
  }
  if (bad && err) atomicOr(err, 1u);
  __syncthreads();
  const int wk = words_of(d, bits), pw = fields_per_word(bits);
  for (int64_t r0 = t0; r0 < t1; r0 += kChunk) {
    const int rows = (int)min((int64_t)kChunk, t1 - r0);
    for (int i = tid; i < rows * d; i += kThreads) {
      int r = i / d, c = i % d;
      u8[i] = (uint8_t)encode(ld(x, (r0 + r) * d + c), sc[c], qmax);
    }
    __syncthreads();
    for (int i = tid; i < rows * wk; i += kThreads) {
      int r = i / wk, w = i % wk;
      uint32_t word = 0;
      for (int j = 0; j < pw; ++j) {
        int c = w * pw + j;
        if (c < d) word |= (uint32_t)u8[r * d + c] << (j * bits);
      }
      codes[(mat * n_tok + r0 + r) * wk + w] = word;
    }
    __syncthreads();
  }
}

// Stateless per-token quantizer: one workgroup per (matrix, kChunk tokens).
template <typename T>
__global__ void __launch_bounds__(kThreads)
quantize_v_kernel(const T* __restrict__ v, int64_t n_tok, int d, int bits,
                  int Gv, uint32_t* __restrict__ codes,
                  float* __restrict__ scales, uint32_t* err) {
  __shared__ float xs[kChunk * kMaxD];
  __shared__ float sc[kChunk * kMaxD];  // worst case Gv = 1
  __shared__ uint8_t u8[kChunk * kMaxD];
  const int tid = threadIdx.x;
  const int64_t mat = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.x * kChunk;
  const int rows = (int)min((int64_t)kChunk, n_tok - r0);
  const T* x = v + (mat * n_tok + r0) * d;
  const int qmax = qmax_of(bits);
  const int ng = d / Gv;
  bool bad = false;
  for (int i = tid; i < rows * d; i += kThreads) {
    float val = ld(x, i);
    bad |= !finite(val);
    xs[i] = val;
  }
  if (bad && err) atomicOr(err, 1u);
  __syncthreads();
  for (int i = tid; i < rows * ng; i += kThreads) {
    int r = i / ng, j = i % ng;
    float m = 0.0f;
    for (int c = 0; c < Gv; ++c) m = fmaxf(m, fabsf(xs[r * d + j * Gv + c]));
    float s = group_scale(m, qmax);
    sc[i] = s;
    scales[(mat * n_tok + r0 + r) * ng + j] = s;
  }
  __syncthreads();
  for (int i = tid; i < rows * d; i += kThreads) {
    int r = i / d, c = i % d;
    u8[i] = (uint8_t)encode(xs[i], sc[r * ng + c / Gv], qmax);
  }
  __syncthreads();
  const int wk = words_of(d, bits), pw = fields_per_word(bits);
  for (int i = tid; i < rows * wk; i += kThreads) {
    int r = i / wk, w = i % wk;
    uint32_t word = 0;
    for (int j = 0; j < pw; ++j) {
      int c = w * pw + j;
      if (c < d) word |= (uint32_t)u8[r * d + c] << (j * bits);
    }
    codes[(mat * n_tok + r0 + r) * wk + w] = word;
  }
}

__global__ void dequant_kernel(const uint32_t* __restrict__ codes,
                               const float* __restrict__ scales,
                               int64_t n_mats, int64_t n_tok, int d, int bits,
                               int axis, int group, float* __restrict__ out) {
  const int64_t total = n_mats * n_tok * d;
  const int wk = words_of(d, bits), pw = fields_per_word(bits);
  const int off = qmax_of(bits) + 1;
  const int64_t n_groups = (n_tok + group - 1) / group;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t row = i / d;
    int c = (int)(i % d);
    int64_t mat = row / n_tok, t = row % n_tok;
    uint32_t w = codes[row * wk + c / pw];
    int u = (int)((w >> ((c % pw) * bits)) & ((1u << bits) - 1u));
    float s = axis == KVQ_PER_CHANNEL
                  ? scales[(mat * n_groups + t / group) * d + c]
                  : scales[row * (d / group) + c / group];
    out[i] = (float)(u - off) * s;
  }
}

__global__ void fill_u32_kernel(uint32_t* dst, uint32_t v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = v;
}
// Streaming read: block b reads its contiguous share of src with 16-byte
// loads, four in flight per thread, and stores the XOR of what it read to
// sink[b] (so the loads cannot be dropped).
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
// Plain streaming read: workgroup b XORs the words of its contiguous share
// into sink[b], eight nontemporal 16-byte loads in flight per thread.
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4v* __restrict__ src, int64_t n16,
                                                          uint32_t* sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  u32x4v acc = {0u, 0u, 0u, 0u};
  for (int64_t i = lo + threadIdx.x; i < hi; i += 8 * 256) {
    u32x4v v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = i + 256 * u < hi ? __builtin_nontemporal_load(src + i + 256 * u) : (u32x4v){0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 1; o < 64; o <<= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}
__global__ void fill_f64_kernel(double* dst, double v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = v;
}

// ---------------------------------------------------------------------------
// Append: fp16 rows to the sink and to ring rows of the tail.
// grid.y = stream; grid.x covers the rows.
// ---------------------------------------------------------------------------
__global__ void append_rows_kernel(CacheDev c, const uint16_t* __restrict__ k_in,
                                   const uint16_t* __restrict__ v_in,
                                   int64_t n_new, int64_t ns_old, int64_t take,
                                   int64_t in_lo, int64_t in_hi, int64_t p_lo) {
  const int64_t st = blockIdx.y;
  const int D = c.D;
  const int64_t n_rows = take + (in_hi - in_lo);
  const int64_t total = n_rows * D;
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = i / D;
    int d = (int)(i % D);
    int64_t src, dst;
    uint16_t *dk, *dv;
    if (r < take) {
      src = r;
      dst = st * c.s_sink + (ns_old + r) * D + d;
      dk = c.sink_k; dv = c.sink_v;
    } else {
      int64_t in = in_lo + (r - take);
      src = in;
      int64_t p = p_lo + (in - in_lo);
      dst = st * c.s_tail + (p % c.R) * D + d;
      dk = c.tail_k; dv = c.tail_v;
    }
    uint16_t kk = k_in[(st * n_new + src) * D + d];
    uint16_t vv = v_in[(st * n_new + src) * D + d];
    bad |= !finite(h2f(kk)) || !finite(h2f(vv));
    dk[dst] = kk;
    dv[dst] = vv;
  }
  if (bad) atomicOr(c.err, 1u);
}

// ---------------------------------------------------------------------------
// Flush: one workgroup per (key group, KV head, batch).
// ---------------------------------------------------------------------------
struct FlushSrc {
  const uint16_t* k_in;
  const uint16_t* v_in;
  int64_t n_new, take, nq_old, nt_old;
};

__device__ inline int64_t src_index(const CacheDev& c, const FlushSrc& f,
                                    int64_t st, int64_t p, bool* from_ring) {
  if (p < f.nq_old + f.nt_old) {
    *from_ring = true;
    return st * c.s_tail + (p % c.R) * c.D;
  }
  *from_ring = false;
  return (st * f.n_new + f.take + (p - f.nq_old - f.nt_old)) * c.D;
}

// MAXD: largest head dimension the LDS rows hold (128 or 256; the smaller
// one fits four workgroups per compute unit).
template <int MAXD>
__global__ void __launch_bounds__(kThreads)
flush_kernel(CacheDev c, FlushSrc f) {
  // pass 1 reduction scratch shares storage with the staged fp16 rows
  __shared__ __align__(16) union {
    float red[kThreads * 8];
    struct {
      uint16_t xk[kChunk * MAXD];
      uint16_t xv[kChunk * MAXD];
    } rows;
  } U;
  float* red = U.red;
  uint16_t* xk = U.rows.xk;
  uint16_t* xv = U.rows.xv;
  __shared__ float kmax[MAXD];     // S_d (absmax per channel)
  __shared__ float ksc[MAXD];      // scale per channel (uniform or class)
  __shared__ int kpos[MAXD];       // position in class order (mixed)
  __shared__ int kcls[MAXD];
  __shared__ double A[MAXD];
  __shared__ float vsc[kChunk * (MAXD / 2)];  // value scales (D / Gv <= MAXD / 2)
  __shared__ uint8_t u8[kChunk * MAXD];
  __shared__ uint16_t b16[kChunk * MAXD];
  const int tid = threadIdx.x;
  const int D = c.D, G = c.G;
  const int64_t st = (int64_t)blockIdx.z * c.H + blockIdx.y;
  const int64_t grp = f.nq_old / G + blockIdx.x;
  const int64_t p0 = grp * G;
  bool bad = false;
  // 16-byte row chunks when rows allow it (else element by element)
  const bool vec = (D % 8 == 0) && (((uintptr_t)f.k_in | (uintptr_t)f.v_in) % 16 == 0);
  const int cpr = D / 8;  // 16-byte chunks per row

  // ---- keys, pass 1: per-channel absmax over the G tokens.
  if (vec) {
    // thread = (row slice, 8-channel chunk); rows stride by the slice count
    const int slices = kThreads / cpr;
    const int c8 = tid % cpr, sl = tid / cpr;
    float m[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (sl < slices) {
#pragma unroll 4
      for (int r = sl; r < G; r += slices) {
        bool ring;
        const int64_t base = src_index(c, f, st, p0 + r, &ring) + 8 * c8;
        const uint4 w = *(const uint4*)((ring ? c.tail_k : f.k_in) + base);
        const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = h2f((uint16_t)(wv[j >> 1] >> (16 * (j & 1))));
          bad |= !finite(x);
          m[j] = fmaxf(m[j], fabsf(x));
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) red[sl * D + 8 * c8 + j] = m[j];
    }
    __syncthreads();
    if (tid < D) {
      float mm = red[tid];
      for (int q = 1; q < slices; ++q) mm = fmaxf(mm, red[q * D + tid]);
      kmax[tid] = mm;
    }
  } else {
    const int slices = kThreads / D;
    if (tid < slices * D) {
      int ch = tid % D, sl = tid / D;
      float m = 0.0f;
      for (int r = sl; r < G; r += slices) {
        bool ring;
        int64_t base = src_index(c, f, st, p0 + r, &ring);
        float v = h2f(ring ? c.tail_k[base + ch] : f.k_in[base + ch]);
        bad |= !finite(v);
        m = fmaxf(m, fabsf(v));
      }
      red[tid] = m;
    }
    __syncthreads();
    if (tid < D) {
      float m = red[tid];
      for (int sl = 1; sl < slices; ++sl) m = fmaxf(m, red[sl * D + tid]);
      kmax[tid] = m;
    }
  }
  __syncthreads();

  if (!c.mixed) {
    if (tid < D) {
      float s = group_scale(kmax[tid], qmax_of(c.k_bits));
      ksc[tid] = s;
      c.k_scales[st * c.s_k_scales + grp * D + tid] = s;
    }
  } else {
    // MixKVQ classes: A_d = I_d * S_d (float64), rank by (-A, d).
    if (tid < D) A[tid] = c.I[st * D + tid] * (double)kmax[tid];
    __syncthreads();
    if (tid < D) {
      double a = A[tid];
      int rank = 0;
      for (int e = 0; e < D; ++e) {
        double b = A[e];
        rank += (b > a) || (b == a && e < tid);
      }
      kcls[tid] = rank < c.n_bf16 ? 0 : (rank < c.n_bf16 + c.n_int4 ? 1 : 2);
    }
    __syncthreads();
    if (tid < D) {
      int cl = kcls[tid], before = 0;
      for (int e = 0; e < tid; ++e) before += (kcls[e] == cl);
      int start = cl == 0 ? 0 : (cl == 1 ? c.n_bf16 : c.n_bf16 + c.n_int4);
      int pos = start + before;
      kpos[tid] = pos;
      c.k_pos[st * c.s_k_pos + grp * D + tid] = (uint8_t)pos;
      if (cl != 0) {
        float s = group_scale(kmax[tid], qmax_of(cl == 1 ? 4 : 2));
        ksc[tid] = s;
        c.k_scales[st * c.s_k_scales + grp * (D - c.n_bf16) + (pos - c.n_bf16)] = s;
      } else {
        ksc[tid] = 1.0f;
      }
    }
  }
  // bound on |k_hat| / code of the group: the largest channel scale (the
  // absmax itself for bf16 channels)
  if (tid == 0) {
    float gm = 0.0f;
    for (int e = 0; e < D; ++e) gm = fmaxf(gm, (c.mixed && kcls[e] == 0) ? kmax[e] : ksc[e]);
    c.k_gmax[st * c.s_k_gmax + grp] = gm;
  }
  __syncthreads();

  // ---- keys, pass 2 and values, chunk by chunk of kChunk tokens.
  const int ngv = D / c.Gv;
  const int qv = qmax_of(c.v_bits);
  for (int r0 = 0; r0 < G; r0 += kChunk) {
    const int rows = min(kChunk, G - r0);
    // stage the chunk's K and V rows (fp16) in LDS
    if (vec) {
      for (int i = tid; i < rows * cpr; i += kThreads) {
        const int r = i / cpr, c8 = i % cpr;
        bool ring;
        const int64_t base = src_index(c, f, st, p0 + r0 + r, &ring) + 8 * c8;
        *(uint4*)&xk[r * D + 8 * c8] = *(const uint4*)((ring ? c.tail_k : f.k_in) + base);
        *(uint4*)&xv[r * D + 8 * c8] = *(const uint4*)((ring ? c.tail_v : f.v_in) + base);
      }
    } else {
      for (int i = tid; i < rows * D; i += kThreads) {
        const int r = i / D, ch = i % D;
        bool ring;
        const int64_t base = src_index(c, f, st, p0 + r0 + r, &ring);
        xk[i] = ring ? c.tail_k[base + ch] : f.k_in[base + ch];
        xv[i] = ring ? c.tail_v[base + ch] : f.v_in[base + ch];
      }
    }
    __syncthreads();
    // encode K
    for (int i = tid; i < rows * D; i += kThreads) {
      int r = i / D, ch = i % D;
      float v = h2f(xk[i]);
      if (!c.mixed) {
        u8[i] = (uint8_t)encode(v, ksc[ch], qmax_of(c.k_bits));
      } else {
        int cl = kcls[ch];
        if (cl == 0) {
          b16[r * D + kpos[ch]] = f32_to_bf16_rne(v);
        } else {
          u8[r * D + kpos[ch]] = (uint8_t)encode(v, ksc[ch], qmax_of(cl == 1 ? 4 : 2));
        }
      }
    }
    __syncthreads();
    const int64_t prow = p0 + r0;  // quantized index of the chunk's first row
    if (!c.mixed) {
      const int wk = words_of(D, c.k_bits), pw = fields_per_word(c.k_bits);
      for (int i = tid; i < rows * wk; i += kThreads) {
        int r = i / wk, w = i % wk;
        uint32_t word = 0;
        for (int j = 0; j < pw; ++j) {
          int ch = w * pw + j;
          if (ch < D) word |= (uint32_t)u8[r * D + ch] << (j * c.k_bits);
        }
        c.k_codes[st * c.s_k_codes + (prow + r) * wk + w] = word;
      }
    } else {
      const int nb = c.n_bf16, n4 = c.n_int4, n2 = D - nb - n4;
      for (int i = tid; i < rows * nb; i += kThreads) {
        int r = i / nb, j = i % nb;
        c.k_bf16[st * c.s_k_bf16 + (prow + r) * nb + j] = b16[r * D + j];
      }
      const int w4 = words_of(n4, 4), w2 = words_of(n2, 2);
      for (int i = tid; i < rows * (w4 + w2); i += kThreads) {
        int r = i / (w4 + w2), w = i % (w4 + w2);
        uint32_t word = 0;
        if (w < w4) {
          for (int j = 0; j < 8; ++j) {
            int k = w * 8 + j;
            if (k < n4) word |= (uint32_t)u8[r * D + nb + k] << (4 * j);
          }
          c.k_int4[st * c.s_k_int4 + (prow + r) * w4 + w] = word;
        } else {
          w -= w4;
          for (int j = 0; j < 16; ++j) {
            int k = w * 16 + j;
            if (k < n2) word |= (uint32_t)u8[r * D + nb + n4 + k] << (2 * j);
          }
          c.k_int2[st * c.s_k_int2 + (prow + r) * w2 + w] = word;
        }
      }
    }
    __syncthreads();
    // values: per-token group scales, encode, pack
    for (int i = tid; i < rows * ngv; i += kThreads) {
      int r = i / ngv, j = i % ngv;
      float m = 0.0f;
      for (int e = 0; e < c.Gv; ++e) {
        const float x = h2f(xv[r * D + j * c.Gv + e]);
        bad |= !finite(x);
        m = fmaxf(m, fabsf(x));
      }
      float s = group_scale(m, qv);
      if (ngv <= MAXD / 2) vsc[i] = s;
      c.v_scales[st * c.s_v_scales + (prow + r) * ngv + j] = s;
    }
    __syncthreads();
    for (int i = tid; i < rows * D; i += kThreads) {
      int r = i / D, ch = i % D;
      const float x = h2f(xv[i]);
      // more groups than the LDS row holds only with Gv = 1: the scale of a
      // one-element group is |x| / qmax
      const float sv = ngv <= MAXD / 2 ? vsc[r * ngv + ch / c.Gv] : group_scale(fabsf(x), qv);
      u8[i] = (uint8_t)encode(x, sv, qv);
    }
    __syncthreads();
    if (c.v_layout == KVQ_V_ROWS) {
      const int wv = words_of(D, c.v_bits), pw = fields_per_word(c.v_bits);
      for (int i = tid; i < rows * wv; i += kThreads) {
        int r = i / wv, w = i % wv;
        uint32_t word = 0;
        for (int j = 0; j < pw; ++j) {
          int ch = w * pw + j;
          if (ch < D) word |= (uint32_t)u8[r * D + ch] << (j * c.v_bits);
        }
        c.v_codes[st * c.s_v_codes + (prow + r) * wv + w] = word;
      }
    } else {
      // whole 32-token tile (G and the group start are multiples of 32)
      const int vb = c.v_bits;
      const int Wl = v_tile_lane_words(D, vb);
      const int C = Wl < 4 ? Wl : 4;
      const int n_words = D * vb;
      const int nf = 32 / vb;
      uint32_t* tile = c.v_codes + st * c.s_v_codes + (prow >> 5) * (int64_t)n_words;
      for (int i = tid; i < n_words; i += kThreads) {
        int chunk = i / (64 * C), rem = i % (64 * C);
        int l = rem / C, w = chunk * C + rem % C;
        uint32_t word = 0;
        for (int p = 0; p < nf; ++p) {
          int tau, ch;
          v_tile_field(l, w, p, vb, &tau, &ch);
          word |= (uint32_t)u8[tau * D + ch] << (p * vb);
        }
        tile[i] = word;
      }
    }
    __syncthreads();
  }
  if (bad) atomicOr(c.err, 1u);
}

// ---------------------------------------------------------------------------
// Register-resident flush for the common layouts: uniform keys and values of
// 2, 4 or 8 bits, D a power of two in [8, 256], value groups of at least 8
// channels, and at most kRegRows rows of the key group per thread.  Thread
// (slice sl, 8-channel chunk c8) loads rows sl, sl + slices, ... of the group
// (keys and values, fp16) into registers in one round of requests; the
// absmax reductions work on fp16 magnitudes (max is exact in any format).
//
// Codes: rint(x / s) is taken as rint(x * rcp(s)) unless that product lies
// within 2^-13 of a rounding boundary, where the IEEE quotient decides.
// Here |x / s| <= qmax * (1 + 2^-23) < 128 (s is the rounded absmax / qmax of
// x's own group), v_rcp_f32 is within 1 ulp and the multiply rounds once, so
// the product differs from the rounded quotient by less than 128 * 2^-22 =
// 2^-15: outside the band both lie strictly between the same two
// half-integers and round to the same integer.  A NaN product takes the
// division too, so every code equals the division's.
// ---------------------------------------------------------------------------
constexpr int kRegRows = 8;
constexpr float kNearTie = 0.5f - 0x1p-13f;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ inline uint32_t max_u16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}
// per-lane max of |x| over the eight fp16 values of w (fp16 bits)
__device__ inline uint32_t absmax8(uint4 w) {
  const uint32_t m = max_u16x2(max_u16x2(w.x & 0x7FFF7FFFu, w.y & 0x7FFF7FFFu),
                               max_u16x2(w.z & 0x7FFF7FFFu, w.w & 0x7FFF7FFFu));
  return max(m & 0xFFFFu, m >> 16);
}

// Offset-binary codes of the eight fp16 values of w at BITS bits, field j at
// bit FW * j of the 64-bit result (x: fields 0..31, y: 32..63).
//
// fma(x, rc, M) with M = 1.5 * 2^23 + qmax + 1 rounds the exact product
// x * rc to an integer n (ties to even, M being even) and leaves n + qmax + 1,
// the code, in the low mantissa bits; the second fma gives x * rc - n to
// within 2^-25.  No clamp is needed: |x * rc| <= qmax * (1 + 2^-22) rounds to
// at most qmax.  v_alignbit shifts each code in from the top and drops the
// exponent bits above it.
template <int BITS, int FW>
__device__ inline uint2 encode8(uint4 w, const float* s, const float* rc) {
  constexpr int qmax = (1 << (BITS - 1)) - 1;
  constexpr float M = 12582912.0f + (float)(qmax + 1);
  const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
  float t[8];
  float dmax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float x = h2f((uint16_t)(wv[j >> 1] >> (16 * (j & 1))));
    t[j] = __builtin_fmaf(x, rc[j], M);
    dmax = fmaxf(dmax, fabsf(__builtin_fmaf(x, rc[j], -(t[j] - M))));
  }
  if (!(dmax < kNearTie)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = h2f((uint16_t)(wv[j >> 1] >> (16 * (j & 1))));
      t[j] = rintf(__fdiv_rn(x, s[j])) + M;
    }
  }
  uint32_t acc[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int word = FW * j / 32;
    acc[word] = __builtin_amdgcn_alignbit(__builtin_bit_cast(uint32_t, t[j]), acc[word], FW);
  }
  // eight 2-bit fields fill only the top half of the word
  if (FW * 8 < 32) acc[0] >>= 32 - FW * 8;
  return make_uint2(acc[0], acc[1]);
}

// max of m over aligned groups of 2^lg lanes (lg <= 5), every lane active
__device__ inline uint32_t group_max_lanes(uint32_t m, int lg) {
  if (lg > 0) m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
  if (lg > 1) m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
  if (lg > 2) m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false));
  if (lg > 3) m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x140, 0xF, 0xF, false));
  if (lg > 4) m = max(m, (uint32_t)__shfl_xor((int)m, 16));
  return m;
}

// stores the eight codes of one row chunk (packed at BITS bits) at chunk c8
template <int BITS>
__device__ inline void store_codes8(uint32_t* row, int c8, uint2 code) {
  if (BITS == 2) ((uint16_t*)row)[c8] = (uint16_t)code.x;
  else if (BITS == 4) row[c8] = code.x;
  else ((uint2*)row)[c8] = code;
}

// KB = 0: mixed keys (MixKVQ): per group, the salience classes of the
// channels, bf16 rows of the class-0 channels, int4 and int2 codes of the
// others in ascending-channel order within each class; codes are staged in
// LDS by class position and packed from there.
constexpr int kMixBf16Stage = 4096;  // halves: G * n_bf16 bf16 keys of a group
template <int KB, int VB>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(4)))
flush_reg_kernel(CacheDev c, FlushSrc f, int lg_cpr, int lg_gv8) {
  __shared__ __align__(16) uint16_t kmag[kThreads * 8];         // [slice][channel] |k| maxima
  __shared__ __align__(16) float ksc[kMaxD];                    // key scale per channel
  __shared__ __align__(16) uint8_t vst[kRegRows * kThreads * 8];  // codes [row][channel or position]
  constexpr int qk = KB > 0 ? (1 << (KB - 1)) - 1 : 0, qv = (1 << (VB - 1)) - 1;
  const int tid = threadIdx.x;
  const int D = c.D, G = c.G;
  const int slices = kThreads >> lg_cpr;
  const int c8 = tid & ((1 << lg_cpr) - 1), sl = tid >> lg_cpr;
  const int64_t st = (int64_t)blockIdx.z * c.H + blockIdx.y;
  const int64_t grp = f.nq_old / G + blockIdx.x;
  const int64_t p0 = grp * G;
  // rows p < ring_end sit in the tail ring (R is a multiple of G, so the
  // group's ring rows are contiguous from slot p0 % R); later ones in the input
  const int64_t ring_end = f.nq_old + f.nt_old;
  const int64_t ring0 = st * c.s_tail + (p0 % c.R) * D + 8 * c8;
  const int64_t in0 = (st * f.n_new + f.take + (p0 - ring_end)) * D + 8 * c8;
  // rows past the group's end load its last row again: a repeated row leaves
  // every maximum unchanged, and its codes are not stored
  uint4 kr[kRegRows], vr[kRegRows];
#pragma unroll
  for (int k = 0; k < kRegRows; ++k) {
    const int r = min(sl + k * slices, G - 1);
    const bool ring = p0 + r < ring_end;
    const int64_t at = (ring ? ring0 : in0) + (int64_t)r * D;
    kr[k] = *(const uint4*)((ring ? c.tail_k : f.k_in) + at);
    vr[k] = *(const uint4*)((ring ? c.tail_v : f.v_in) + at);
  }
  // ---- keys, pass 1: per-channel absmax over the group
  {
    uint32_t m[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < kRegRows; ++k) {
      m[0] = max_u16x2(m[0], kr[k].x & 0x7FFF7FFFu);
      m[1] = max_u16x2(m[1], kr[k].y & 0x7FFF7FFFu);
      m[2] = max_u16x2(m[2], kr[k].z & 0x7FFF7FFFu);
      m[3] = max_u16x2(m[3], kr[k].w & 0x7FFF7FFFu);
    }
    *(uint4*)&kmag[sl * D + 8 * c8] = make_uint4(m[0], m[1], m[2], m[3]);
  }
  __syncthreads();
  bool bad = false;
  uint32_t kmbits = 0;  // this channel's |k| maximum (fp16 bits), tid < D
  if (tid < D) {
    for (int q = 0; q < slices; ++q) kmbits = max(kmbits, (uint32_t)kmag[q * D + tid]);
    bad = kmbits >= 0x7C00u;
  }
  if constexpr (KB > 0) {
    if (tid < D) {
      const float s = group_scale(h2f((uint16_t)kmbits), qk);
      ksc[tid] = s;
      c.k_scales[st * c.s_k_scales + grp * D + tid] = s;
    }
    __syncthreads();
    // bound on |k_hat| / code of the group: the largest channel scale
    if (tid < 64) {
      float g = 0.0f;
      for (int ch = tid; ch < D; ch += 64) g = fmaxf(g, ksc[ch]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) g = fmaxf(g, __shfl_xor(g, o));
      if (tid == 0) c.k_gmax[st * c.s_k_gmax + grp] = g;
    }
    // ---- keys, pass 2
    float s[8], rc[8];
    const float4 a = *(const float4*)&ksc[8 * c8], b = *(const float4*)&ksc[8 * c8 + 4];
    s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w;
    s[4] = b.x; s[5] = b.y; s[6] = b.z; s[7] = b.w;
#pragma unroll
    for (int j = 0; j < 8; ++j) rc[j] = __builtin_amdgcn_rcpf(s[j]);
    const int wk = D * KB / 32;
    uint32_t* krow = c.k_codes + st * c.s_k_codes + p0 * wk;
#pragma unroll
    for (int k = 0; k < kRegRows; ++k) {
      const int r = sl + k * slices;
      if (r < G) store_codes8<KB>(krow + (int64_t)r * wk, c8, encode8<KB, KB>(kr[k], s, rc));
    }
  } else {
    // ---- MixKVQ classes: A_d = I_d * S_d (float64), ranked by (-A, d)
    __shared__ double A[kMaxD];
    __shared__ float kmx[kMaxD];
    __shared__ int kcls[kMaxD], kpos[kMaxD];
    __shared__ __align__(16) uint16_t bst[kMixBf16Stage];  // [row][bf16 position]
    const int nb = c.n_bf16, n4 = c.n_int4, n2 = D - nb - n4, nint = D - nb;
    if (tid < D) {
      kmx[tid] = h2f((uint16_t)kmbits);
      A[tid] = c.I[st * D + tid] * (double)kmx[tid];
    }
    __syncthreads();
    __shared__ int wcount[kThreads / 64][3];  // channels of each class per wave
    int cl = 0;
    if (tid < D) {
      const double av = A[tid];
      int rank = 0;
#pragma unroll 8
      for (int e = 0; e < D; ++e) {
        const double bv = A[e];
        rank += (bv > av) || (bv == av && e < tid);
      }
      cl = rank < nb ? 0 : (rank < nb + n4 ? 1 : 2);
      kcls[tid] = cl;
    }
    // position within the class: same-class channels of lower index, from
    // per-wave ballots (channel = thread index)
    const int lane = tid & 63, wave = tid >> 6;
    uint64_t bal[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) bal[k] = __ballot(tid < D && cl == k);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < 3; ++k) wcount[wave][k] = __popcll(bal[k]);
    }
    __syncthreads();
    if (tid < D) {
      int before = __popcll(bal[cl] & ((1ull << lane) - 1ull));
      for (int w = 0; w < wave; ++w) before += wcount[w][cl];
      const int pos = (cl == 0 ? 0 : (cl == 1 ? nb : nb + n4)) + before;
      kpos[tid] = pos;
      c.k_pos[st * c.s_k_pos + grp * D + tid] = (uint8_t)pos;
      if (cl != 0) {
        const float sc = group_scale(kmx[tid], cl == 1 ? 7 : 1);
        ksc[tid] = sc;
        c.k_scales[st * c.s_k_scales + grp * nint + (pos - nb)] = sc;
      } else {
        ksc[tid] = 1.0f;
      }
    }
    __syncthreads();
    // bound on |k_hat| / code: the largest scale, |K| itself for bf16 channels
    if (tid < 64) {
      float g = 0.0f;
      for (int ch = tid; ch < D; ch += 64) g = fmaxf(g, kcls[ch] == 0 ? kmx[ch] : ksc[ch]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) g = fmaxf(g, __shfl_xor(g, o));
      if (tid == 0) c.k_gmax[st * c.s_k_gmax + grp] = g;
    }
    // ---- keys, pass 2: codes by class position into LDS (offset code in
    // the low mantissa bits as in encode8, per-channel qmax), bf16 rows
    // per channel of the thread: class << 8 | position, 1 / scale
    constexpr float kM4 = 12582912.0f + 8.0f, kM2 = 12582912.0f + 2.0f;
    uint32_t cp[8];
    float rc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ch = 8 * c8 + j;
      cp[j] = ((uint32_t)kcls[ch] << 8) | (uint32_t)kpos[ch];
      rc[j] = __builtin_amdgcn_rcpf(ksc[ch]);
    }
#pragma unroll
    for (int k = 0; k < kRegRows; ++k) {
      const int r = sl + k * slices;
      if (r < G) {
        const uint32_t wv[4] = {kr[k].x, kr[k].y, kr[k].z, kr[k].w};
        float x[8], t[8];
        float dmax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float mg = (cp[j] >> 8) == 1 ? kM4 : kM2;
          x[j] = h2f((uint16_t)(wv[j >> 1] >> (16 * (j & 1))));
          t[j] = __builtin_fmaf(x[j], rc[j], mg);
          const float dj = fabsf(__builtin_fmaf(x[j], rc[j], -(t[j] - mg)));
          if ((cp[j] >> 8) != 0) dmax = fmaxf(dmax, dj);
        }
        if (!(dmax < kNearTie)) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            t[j] = rintf(__fdiv_rn(x[j], ksc[8 * c8 + j])) + ((cp[j] >> 8) == 1 ? kM4 : kM2);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int pj = (int)(cp[j] & 0xFFu);
          if ((cp[j] >> 8) == 0)
            bst[r * nb + pj] = f32_to_bf16_rne(x[j]);
          else
            vst[r * nint + pj - nb] = (uint8_t)(__builtin_bit_cast(uint32_t, t[j]) & 0xFFu);
        }
      }
    }
    __syncthreads();
    const int w4 = words_of(n4, 4), w2 = words_of(n2, 2), wt = w4 + w2;
    for (int i = tid; i < G * wt; i += kThreads) {
      const int r = i / wt;
      int w = i - r * wt;
      const uint8_t* cr = vst + r * nint;
      uint32_t word = 0;
      if (w < w4) {
        for (int j = 0; j < 8; ++j)
          if (w * 8 + j < n4) word |= (uint32_t)cr[w * 8 + j] << (4 * j);
        c.k_int4[st * c.s_k_int4 + (p0 + r) * w4 + w] = word;
      } else {
        w -= w4;
        for (int j = 0; j < 16; ++j)
          if (w * 16 + j < n2) word |= (uint32_t)cr[n4 + w * 16 + j] << (2 * j);
        c.k_int2[st * c.s_k_int2 + (p0 + r) * w2 + w] = word;
      }
    }
    for (int i = tid; i < G * nb; i += kThreads)
      c.k_bf16[st * c.s_k_bf16 + (p0 + i / nb) * nb + i % nb] = bst[i];
    __syncthreads();  // the value tiles reuse the code staging
  }
  // ---- values: per-token group scales over 2^lg_gv8 adjacent lanes
  const bool tiles = c.v_layout == KVQ_V_TILE32;
  const int ngv = D / c.Gv, wv = D * VB / 32;
  const int gmask = (1 << lg_gv8) - 1;
  uint32_t vbad = 0;
#pragma unroll
  for (int k = 0; k < kRegRows; ++k) {
    const int r = sl + k * slices;
    uint32_t m = absmax8(vr[k]);
    if (r < G) vbad = max(vbad, m);
    m = group_max_lanes(m, lg_gv8);
    if (r < G) {
      const float mf = h2f((uint16_t)m);
      const float sv = qv == 1 ? (mf == 0.0f ? 1.0f : mf) : group_scale(mf, qv);
      const float rv = __builtin_amdgcn_rcpf(sv);
      const float s[8] = {sv, sv, sv, sv, sv, sv, sv, sv};
      const float rc[8] = {rv, rv, rv, rv, rv, rv, rv, rv};
      const int64_t p = p0 + r;
      if ((c8 & gmask) == 0) c.v_scales[st * c.s_v_scales + p * ngv + (c8 >> lg_gv8)] = sv;
      if (tiles)
        *(uint2*)&vst[r * D + 8 * c8] = encode8<VB, 8>(vr[k], s, rc);
      else
        store_codes8<VB>(c.v_codes + st * c.s_v_codes + p * wv, c8, encode8<VB, VB>(vr[k], s, rc));
    }
  }
  bad |= vbad >= 0x7C00u;
  if (tiles) {
    // 32-token tiles of the group (G and p0 are multiples of 32): word w of
    // lane l holds the fields that v_tile_field places there
    __syncthreads();
    const int lg_nw = lg_cpr + 3 + (VB == 4 ? 2 : 1);  // log2(D * VB)
    const int Wl = D * VB / 64;
    const int lg_c = Wl >= 4 ? 2 : (Wl == 2 ? 1 : 0);  // C = min(Wl, 4)
    const int n = (G >> 5) << lg_nw;
    uint32_t* tile0 = c.v_codes + st * c.s_v_codes + (p0 >> 5) * (int64_t)(D * VB);
    for (int i = tid; i < n; i += kThreads) {
      const int T = i >> lg_nw, rem = i & ((1 << lg_nw) - 1);
      const int chunk = rem >> (6 + lg_c), rr = rem & ((64 << lg_c) - 1);
      const int l = rr >> lg_c, w = (chunk << lg_c) + (rr & ((1 << lg_c) - 1));
      const uint8_t* base = vst + T * 32 * D;
      uint32_t word = 0;
#pragma unroll
      for (int p = 0; p < 32 / VB; ++p) {
        int tau, ch;
        v_tile_field(l, w, p, VB, &tau, &ch);
        word |= (uint32_t)base[tau * D + ch] << (p * VB);
      }
      tile0[i] = word;
    }
  }
  if (bad) atomicOr(c.err, 1u);
}

// I[b][kvh][d] = sum over rows r and grouped heads h of |q_win[b][r][h][d]|,
// in float64.  One workgroup per (kvh, b, block of kSalCh channels): the
// block's columns of the window rows of the group's g heads are staged in
// LDS (as many rows as fit 64 KB at a time) with coalesced loads, 16-byte
// ones when the rows allow.
//
// Each |q| is a multiple of 2^-24 (the fp16 grain) below 2^16, so with at
// most 8192 terms every partial sum is a multiple of 2^-24 below 2^29 and
// exact in float64: the result does not depend on the order of the
// additions.  The terms of a channel are then spread over eight threads and
// four accumulators each.  Longer windows keep the sequential order (rows
// ascending, heads ascending within a row) on one thread per channel.
constexpr int kSalCh = 32;          // channels per workgroup
constexpr int kSalLds = 65536;      // bytes of staged window columns
constexpr int kSalExactTerms = 8192;
__global__ void __launch_bounds__(256) salience_kernel(CacheDev c, const uint16_t* __restrict__ q,
                                                       int w_rows, int Hq) {
  __shared__ __align__(16) uint16_t st[kSalLds / 2];
  const int tid = threadIdx.x, D = c.D;
  const int h = blockIdx.x, b = blockIdx.y, d0 = blockIdx.z * kSalCh;
  const int nc = min(kSalCh, D - d0);          // channels of this block
  const int g = Hq / c.H;
  const int seg = g * kSalCh;                  // staged halves per window row
  const int rows = kSalLds / 2 / seg;          // rows per chunk (>= 1: checked on the host)
  const uint16_t* base = q + ((int64_t)b * w_rows * Hq + (int64_t)h * g) * D + d0;
  const int64_t rstride = (int64_t)Hq * D;     // halves between window rows
  const bool vec = nc == kSalCh && D % 8 == 0 && ((uintptr_t)base % 16) == 0;
  const int P = (int64_t)w_rows * g <= kSalExactTerms ? 256 / kSalCh : 1;
  const int cl = tid % kSalCh, part = tid / kSalCh;
  const bool active = part < P && cl < nc;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  bool bad = false;
  for (int r0 = 0; r0 < w_rows; r0 += rows) {
    const int n = min(rows, w_rows - r0);
    // item (r, hh, piece) of the chunk: window row r0 + r, head hh
    if (vec) {
      const int total = n * g * (kSalCh / 8);
      for (int i0 = tid; i0 < total; i0 += 8 * 256) {
        uint4 x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int i = i0 + k * 256;
          if (i < total) {
            const int p8 = i % (kSalCh / 8), t = i / (kSalCh / 8);  // t = r * g + hh
            x[k] = *(const uint4*)(base + (int64_t)(r0 + t / g) * rstride + (t % g) * D + 8 * p8);
          }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int i = i0 + k * 256;
          if (i < total) *(uint4*)&st[8 * i] = x[k];
        }
      }
    } else {
      const int total = n * g * kSalCh;
      for (int i = tid; i < total; i += 256) {
        const int e = i % kSalCh, t = i / kSalCh;
        st[i] = e < nc ? base[(int64_t)(r0 + t / g) * rstride + (t % g) * D + e] : (uint16_t)0;
      }
    }
    __syncthreads();
    // term t = r * g + hh of the chunk sits at st[t * kSalCh + cl]
    const int nt = n * g;
    if (active && P == 1) {
      for (int t = 0; t < nt; ++t) {
        const float v = h2f(st[t * kSalCh + cl]);
        bad |= !finite(v);
        acc[0] += fabs((double)v);
      }
    } else if (active) {
      int t = part;
      for (; t + 3 * P < nt; t += 4 * P) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float v = h2f(st[(t + k * P) * kSalCh + cl]);
          bad |= !finite(v);
          acc[k] += fabs((double)v);
        }
      }
      for (; t < nt; t += P) {
        const float v = h2f(st[t * kSalCh + cl]);
        bad |= !finite(v);
        acc[0] += fabs((double)v);
      }
    }
    __syncthreads();
  }
  // combine the parts of each channel (exact when P > 1)
  double* red = (double*)st;
  red[tid] = active ? (acc[0] + acc[1]) + (acc[2] + acc[3]) : 0.0;
  __syncthreads();
  if (tid < nc) {
    double t = red[tid];
    for (int p = 1; p < P; ++p) t += red[p * kSalCh + tid];
    c.I[((int64_t)b * c.H + h) * D + d0 + tid] = t;
  }
  if (bad) atomicOr(c.err, 1u);
}

// ---------------------------------------------------------------------------
// Key rotation ("Quantize What Counts: More for Keys, Less for Values",
// rotation integration; the Walsh-Hadamard step of the KQV scheme in
// "Statistical Inference and Quality Measures of KV Cache Quantisations
// Inspired by TurboQuant"): y = H x / sqrt(d) per row, H the Sylvester
// Walsh-Hadamard matrix, by the fast transform in float32: stages h = 1,
// 2, 4, ..., d/2 replace (x[i], x[i + h]) (bit h of i clear) with
// (x[i] + x[i + h], x[i] - x[i + h]), then every element is multiplied by
// float32(1 / sqrt(d)); a float16 output is that value rounded to nearest
// even.  Every step is one IEEE operation, so the bits are fixed.
// ---------------------------------------------------------------------------
template <typename T> __device__ inline float to_f(T v);
template <> __device__ inline float to_f<float>(float v) { return v; }
template <> __device__ inline float to_f<uint16_t>(uint16_t v) { return h2f(v); }
// One float32 multiply, rounded to float32.  Written as the instruction so
// that the compiler cannot merge it with a following float16 conversion into
// a mixed-precision fma, which would round once instead of twice.
__device__ inline float mul_f32(float a, float b) {
  float y;
  asm volatile("v_mul_f32 %0, %1, %2" : "=v"(y) : "v"(a), "v"(b));
  return y;
}
__device__ inline void put(float* p, float v) { *p = v; }
__device__ inline void load8(const uint16_t* p, float* x) {
  const uint4 w = *(const uint4*)p;
  const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = h2f((uint16_t)(wv[j >> 1] >> (16 * (j & 1))));
}
__device__ inline void load8(const float* p, float* x) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ inline uint32_t f16_bits(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }
__device__ inline void store8(uint16_t* p, const float* x) {
  *(uint4*)p = make_uint4(f16_bits(x[0]) | f16_bits(x[1]) << 16, f16_bits(x[2]) | f16_bits(x[3]) << 16,
                          f16_bits(x[4]) | f16_bits(x[5]) << 16, f16_bits(x[6]) | f16_bits(x[7]) << 16);
}
__device__ inline void store8(float* p, const float* x) {
  *(float4*)p = make_float4(x[0], x[1], x[2], x[3]);
  *(float4*)(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
// x of lane (this lane xor c), c < 32: ds_swizzle in bit-mask mode
// (and-mask 0x1F, or-mask 0, xor-mask c, within 32-lane halves)
__device__ inline float xor_lane(float x, int c) {
  const int v = __builtin_bit_cast(int, x);
  int r;
  switch (c) {
    case 1: r = __builtin_amdgcn_ds_swizzle(v, 0x041F); break;
    case 2: r = __builtin_amdgcn_ds_swizzle(v, 0x081F); break;
    case 4: r = __builtin_amdgcn_ds_swizzle(v, 0x101F); break;
    case 8: r = __builtin_amdgcn_ds_swizzle(v, 0x201F); break;
    default: r = __builtin_amdgcn_ds_swizzle(v, 0x401F); break;  // 16
  }
  return __builtin_bit_cast(float, r);
}
__device__ inline void put(uint16_t* p, float v) {
  *p = __builtin_bit_cast(uint16_t, (_Float16)v);
}

// Lane group of d / 8 lanes per row, eight consecutive elements per lane
// (stages 1, 2, 4 in registers, the rest across lanes).  Rows and lanes:
// thread t of the grid covers row t / (d / 8), elements 8 (t % (d / 8)) ..
template <typename TI, typename TO>
__global__ void __launch_bounds__(256) hadamard_vec_kernel(const TI* __restrict__ in, TO* __restrict__ out,
                                                           int64_t n_rows, int lg_cpr, float scale) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = 1 << lg_cpr, d = 8 * cpr;
  const int64_t row = t >> lg_cpr;
  const int c8 = (int)(t & (cpr - 1));
  const bool ok = row < n_rows;
  const int64_t base = (ok ? row : 0) * d + 8 * c8;
  // the launcher passes 16-byte aligned rows (8 * sizeof(T) bytes a lane)
  float x[8];
  load8(in + base, x);
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j & h) continue;
      const float u = x[j], v = x[j + h];
      x[j] = u + v;
      x[j + h] = u - v;
    }
  }
  // stages h = 8 c: partner lane c8 ^ c; the lane with that bit clear keeps
  // the sum, the other the difference (its own value subtracted from the
  // partner's)
#pragma unroll
  for (int c = 1; c < 32; c <<= 1) {
    if (c >= cpr) break;
    const bool upper = c8 & c;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = xor_lane(x[j], c);
      x[j] = upper ? p - x[j] : x[j] + p;
    }
  }
  if (ok) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = mul_f32(x[j], scale);
    store8(out + base, x);
  }
}

// d >= 32: thirty-two consecutive elements per lane, d / 32 lanes per row
// (stages 1 .. 16 in registers; 32, 64, 128 across lanes: DPP quad
// permutations for lane xor 1 and 2, a swizzle for xor 4).
__device__ inline float lane_xor1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}
__device__ inline float lane_xor2(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
}
template <typename TI, typename TO>
__global__ void __launch_bounds__(256) hadamard_vec32_kernel(const TI* __restrict__ in, TO* __restrict__ out,
                                                             int64_t n_rows, int lg_lpr, float scale) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int lpr = 1 << lg_lpr, d = 32 * lpr;
  const int64_t row = t >> lg_lpr;
  const int part = (int)(t & (lpr - 1));
  const bool ok = row < n_rows;
  const int64_t base = (ok ? row : 0) * d + 32 * part;
  float x[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) load8(in + base + 8 * q, x + 8 * q);
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (j & h) continue;
      const float u = x[j], v = x[j + h];
      x[j] = u + v;
      x[j + h] = u - v;
    }
  }
  // stages 32 c: partner lane part ^ c (every lane of the wave takes part)
#pragma unroll
  for (int c = 1; c < 8; c <<= 1) {
    if (c >= lpr) break;
    const bool upper = part & c;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float p = c == 1 ? lane_xor1(x[j]) : (c == 2 ? lane_xor2(x[j]) : xor_lane(x[j], 4));
      x[j] = upper ? p - x[j] : x[j] + p;
    }
  }
  if (ok) {
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] = mul_f32(x[j], scale);
#pragma unroll
    for (int q = 0; q < 4; ++q) store8(out + base + 8 * q, x + 8 * q);
  }
}

// Any power of two d <= 256, any alignment: one row per thread.
template <typename TI, typename TO>
__global__ void __launch_bounds__(256) hadamard_row_kernel(const TI* __restrict__ in, TO* __restrict__ out,
                                                           int64_t n_rows, int d, float scale) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= n_rows) return;
  float x[kMaxD];
  for (int i = 0; i < d; ++i) x[i] = to_f<TI>(in[row * d + i]);
  for (int h = 1; h < d; h <<= 1)
    for (int i = 0; i < d; ++i) {
      if (i & h) continue;
      const float u = x[i], v = x[i + h];
      x[i] = u + v;
      x[i + h] = u - v;
    }
  for (int i = 0; i < d; ++i) put(out + row * d + i, mul_f32(x[i], scale));
}

// ---------------------------------------------------------------------------
// Export: strided copies into dense per-stream arrays, tail ring -> token
// order, value tiles -> rows, key positions -> classes.
// ---------------------------------------------------------------------------
__global__ void copy_streams_u16(const uint16_t* __restrict__ src,
                                 int64_t src_stride, int64_t src_off,
                                 uint16_t* __restrict__ dst, int64_t n_per,
                                 int64_t n_streams) {
  const int64_t total = n_per * n_streams;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t s = i / n_per, j = i % n_per;
    dst[i] = src[s * src_stride + src_off + j];
  }
}
__global__ void copy_streams_u32(const uint32_t* __restrict__ src,
                                 int64_t src_stride, uint32_t* __restrict__ dst,
                                 int64_t n_per, int64_t n_streams) {
  const int64_t total = n_per * n_streams;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t s = i / n_per, j = i % n_per;
    dst[i] = src[s * src_stride + j];
  }
}
__global__ void export_tail(const uint16_t* __restrict__ ring, int64_t stride,
                            int R, int D, int64_t nq, int64_t nt,
                            uint16_t* __restrict__ dst, int64_t n_streams) {
  const int64_t total = nt * D * n_streams;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t s = i / (nt * D), rem = i % (nt * D);
    int64_t t = rem / D;
    int d = (int)(rem % D);
    dst[i] = ring[s * stride + ((nq + t) % R) * D + d];
  }
}
__global__ void export_v_tiles(const uint32_t* __restrict__ tiles,
                               int64_t stride, int D, int vb, int64_t nq,
                               uint32_t* __restrict__ dst, int64_t n_streams) {
  const int wv = words_of(D, vb), pw = fields_per_word(vb);
  const int64_t total = nq * wv * n_streams;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t s = i / (nq * wv), rem = i % (nq * wv);
    int64_t t = rem / wv;
    int w = (int)(rem % wv);
    uint32_t word = 0;
    for (int j = 0; j < pw; ++j) {
      int d = w * pw + j;
      if (d >= D) break;
      int64_t widx;
      int bit;
      v_tile_pos(t, d, D, vb, &widx, &bit);
      uint32_t u = (tiles[s * stride + widx] >> bit) & ((1u << vb) - 1u);
      word |= u << (j * vb);
    }
    dst[i] = word;
  }
}
__global__ void export_classes(const uint8_t* __restrict__ pos, int64_t stride,
                               int64_t n_per, int nb, int n4,
                               uint8_t* __restrict__ dst, int64_t n_streams) {
  const int64_t total = n_per * n_streams;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t s = i / n_per, j = i % n_per;
    int p = pos[s * stride + j];
    dst[i] = (uint8_t)(p < nb ? 0 : (p < nb + n4 ? 1 : 2));
  }
}

// ---------------------------------------------------------------------------
// Counter-based synthetic fp16 (SplitMix64 output function over
// seed + (counter + 1) * golden gamma; Irwin-Hall sum of four 16-bit lanes).
// ---------------------------------------------------------------------------
// float32 -> float16 bits, round to nearest even, subnormal results kept
// (integer arithmetic, so independent of the hardware denormal mode).
// Finite |f| < 65520 only, which the generator guarantees.
__device__ inline uint16_t f2h_rne_int(float f) {
  const uint32_t x = __builtin_bit_cast(uint32_t, f);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7FFFFFFFu;
  uint32_t r;
  if (ax < 0x38800000u) {  // below 2^-14: float16 subnormal (or zero)
    const uint32_t e = ax >> 23;
    const uint32_t mant = (ax & 0x7FFFFFu) | 0x800000u;
    const uint32_t sh = 126u - e;  // value / 2^-24 = mant >> sh
    if (e == 0 || sh > 24u) return (uint16_t)sign;
    r = mant >> sh;
    const uint32_t rem = mant & ((1u << sh) - 1u), half = 1u << (sh - 1u);
    if (rem > half || (rem == half && (r & 1u))) ++r;
  } else {
    r = (ax >> 13) - (112u << 10);
    const uint32_t rem = ax & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) ++r;
  }
  return (uint16_t)(sign | r);
}

__device__ inline uint64_t splitmix_out(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void synth_kernel(uint16_t* __restrict__ out, uint64_t seed,
                             int tensor, int layer, int head0, int n_heads,
                             int64_t t0, int64_t n_tok, int d,
                             int64_t head_stride) {
  const int64_t per = n_tok * d;
  const int64_t total = per * n_heads;
  // float32 nearest to 1/sqrt((2^32 - 1)/3)
  const float kScale = 0x1.bb67aep-16f;  // 2.642899744e-05
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int64_t hh = i / per, rem = i % per;
    int64_t t = t0 + rem / d;
    uint64_t ch = (uint64_t)(rem % d);
    uint64_t hi = (uint64_t)(((int64_t)tensor * 256 + layer) * 256 + head0 + hh);
    uint64_t ctr = ((hi << 32) + (uint64_t)t) * 256ull + ch;
    uint64_t h = splitmix_out(seed + (ctr + 1ull) * 0x9E3779B97F4A7C15ull);
    int64_t s = (int64_t)(h & 0xFFFF) + (int64_t)((h >> 16) & 0xFFFF) +
                (int64_t)((h >> 32) & 0xFFFF) + (int64_t)(h >> 48) - 131070;
    float x = __fmul_rn((float)s, kScale);
    out[hh * head_stride + rem] = f2h_rne_int(x);
  }
}

inline dim3 grid_for(int64_t n, int threads) {
  int64_t b = (n + threads - 1) / threads;
  if (b < 1) b = 1;
  if (b > 65536) b = 65536;
  return dim3((unsigned)b);
}

}  // namespace

hipError_t launch_quantize_k(const void* k, int f16, int64_t n_mats,
                             int64_t n_tok, int d, int bits, int G,
                             uint32_t* codes, float* scales, uint32_t* err,
                             hipStream_t s) {
  int64_t ng = (n_tok + G - 1) / G;
  dim3 grid((unsigned)ng, (unsigned)n_mats);
  if (f16)
    quantize_k_kernel<uint16_t><<<grid, kThreads, 0, s>>>(
        (const uint16_t*)k, n_tok, d, bits, G, codes, scales, err);
  else
    quantize_k_kernel<float><<<grid, kThreads, 0, s>>>(
        (const float*)k, n_tok, d, bits, G, codes, scales, err);
  return hipGetLastError();
}

hipError_t launch_quantize_v(const void* v, int f16, int64_t n_mats,
                             int64_t n_tok, int d, int bits, int Gv,
                             uint32_t* codes, float* scales, uint32_t* err,
                             hipStream_t s) {
  dim3 grid((unsigned)((n_tok + kChunk - 1) / kChunk), (unsigned)n_mats);
  if (f16)
    quantize_v_kernel<uint16_t><<<grid, kThreads, 0, s>>>(
        (const uint16_t*)v, n_tok, d, bits, Gv, codes, scales, err);
  else
    quantize_v_kernel<float><<<grid, kThreads, 0, s>>>(
        (const float*)v, n_tok, d, bits, Gv, codes, scales, err);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint32_t* codes, const float* scales,
                          int64_t n_mats, int64_t n_tok, int d, int bits,
                          int axis, int group, float* out, hipStream_t s) {
  dequant_kernel<<<grid_for(n_mats * n_tok * d, 256), 256, 0, s>>>(
      codes, scales, n_mats, n_tok, d, bits, axis, group, out);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* dst, uint32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_u32_kernel<<<grid_for(n, 256), 256, 0, s>>>(dst, v, n);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s) {
  if (bytes <= 0) return hipSuccess;
  stream_read_kernel<<<kStreamReadBlocks, 256, 0, s>>>((const u32x4v*)src, bytes / 16, sink);
  return hipGetLastError();
}

template <typename TI, typename TO>
hipError_t hadamard_t(const void* in, void* out, int64_t n_rows, int d, hipStream_t s) {
  const float scale = (float)(1.0 / __builtin_sqrt((double)d));
  const bool vec = d >= 8 && ((uintptr_t)in % (8 * sizeof(TI))) == 0 &&
                   ((uintptr_t)out % (8 * sizeof(TO))) == 0;
  if (vec && d >= 32) {
    const int lg_lpr = __builtin_ctz(d / 32);
    const int64_t threads = n_rows << lg_lpr;
    hadamard_vec32_kernel<TI, TO><<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(
        (const TI*)in, (TO*)out, n_rows, lg_lpr, scale);
  } else if (vec) {
    const int lg_cpr = __builtin_ctz(d / 8);
    const int64_t threads = n_rows << lg_cpr;
    hadamard_vec_kernel<TI, TO><<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(
        (const TI*)in, (TO*)out, n_rows, lg_cpr, scale);
  } else {
    hadamard_row_kernel<TI, TO><<<(unsigned)((n_rows + 255) / 256), 256, 0, s>>>(
        (const TI*)in, (TO*)out, n_rows, d, scale);
  }
  return hipGetLastError();
}

hipError_t launch_hadamard(const void* in, int in_f16, void* out, int out_f16, int64_t n_rows,
                           int d, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  if (in_f16)
    return out_f16 ? hadamard_t<uint16_t, uint16_t>(in, out, n_rows, d, s)
                   : hadamard_t<uint16_t, float>(in, out, n_rows, d, s);
  return out_f16 ? hadamard_t<float, uint16_t>(in, out, n_rows, d, s)
                 : hadamard_t<float, float>(in, out, n_rows, d, s);
}

hipError_t launch_fill_f64(double* dst, double v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_f64_kernel<<<grid_for(n, 256), 256, 0, s>>>(dst, v, n);
  return hipGetLastError();
}

hipError_t launch_append_rows(const CacheDev& c, const uint16_t* k_in,
                              const uint16_t* v_in, int64_t n_new,
                              int64_t ns_old, int64_t take, int64_t in_lo,
                              int64_t in_hi, int64_t p_lo, hipStream_t s) {
  int64_t rows = take + (in_hi - in_lo);
  if (rows <= 0) return hipSuccess;
  int64_t per = rows * c.D;
  int64_t bx = (per + 255) / 256;
  if (bx > 4096) bx = 4096;
  dim3 grid((unsigned)bx, (unsigned)(c.B * c.H));
  append_rows_kernel<<<grid, 256, 0, s>>>(c, k_in, v_in, n_new, ns_old, take,
                                          in_lo, in_hi, p_lo);
  return hipGetLastError();
}

hipError_t launch_flush(const CacheDev& c, const uint16_t* k_in,
                        const uint16_t* v_in, int64_t n_new, int64_t take,
                        int64_t nq_old, int64_t nt_old, int64_t n_groups,
                        hipStream_t s) {
  if (n_groups <= 0) return hipSuccess;
  FlushSrc f{k_in, v_in, n_new, take, nq_old, nt_old};
  dim3 grid((unsigned)n_groups, (unsigned)c.H, (unsigned)c.B);
  auto b248 = [](int b) { return b == 2 || b == 4 || b == 8; };
  const int D = c.D;
  if ((c.mixed ? c.G * c.n_bf16 <= kMixBf16Stage : b248(c.k_bits)) && b248(c.v_bits) && D >= 8 &&
      (D & (D - 1)) == 0 && c.Gv >= 8 && c.G <= kRegRows * (kThreads / (D / 8)) &&
      (((uintptr_t)k_in | (uintptr_t)v_in) % 16) == 0) {
    const int lg_cpr = __builtin_ctz(D / 8), lg_gv8 = __builtin_ctz(c.Gv / 8);
#define KVQ_FLUSH_REG(KB, VB)                                                   \
  if (c.k_bits == KB && c.v_bits == VB) {                                       \
    flush_reg_kernel<KB, VB><<<grid, kThreads, 0, s>>>(c, f, lg_cpr, lg_gv8);   \
    return hipGetLastError();                                                   \
  }
    if (c.mixed) {
      if (c.v_bits == 2) KVQ_FLUSH_REG(0, 2)
      if (c.v_bits == 4) KVQ_FLUSH_REG(0, 4)
      if (c.v_bits == 8) KVQ_FLUSH_REG(0, 8)
    }
    KVQ_FLUSH_REG(2, 2) KVQ_FLUSH_REG(2, 4) KVQ_FLUSH_REG(2, 8)
    KVQ_FLUSH_REG(4, 2) KVQ_FLUSH_REG(4, 4) KVQ_FLUSH_REG(4, 8)
    KVQ_FLUSH_REG(8, 2) KVQ_FLUSH_REG(8, 4) KVQ_FLUSH_REG(8, 8)
#undef KVQ_FLUSH_REG
  }
  if (c.D <= 128)
    flush_kernel<128><<<grid, kThreads, 0, s>>>(c, f);
  else
    flush_kernel<kMaxD><<<grid, kThreads, 0, s>>>(c, f);
  return hipGetLastError();
}

hipError_t launch_salience(const CacheDev& c, const uint16_t* q_win, int w_rows,
                           int n_q_heads, hipStream_t s) {
  // one window row of a channel block of a KV head's query heads must fit
  // the staging buffer
  if ((int64_t)(n_q_heads / c.H) * kSalCh * 2 > kSalLds) return hipErrorInvalidValue;
  dim3 grid((unsigned)c.H, (unsigned)c.B, (unsigned)((c.D + kSalCh - 1) / kSalCh));
  salience_kernel<<<grid, 256, 0, s>>>(c, q_win, w_rows, n_q_heads);
  return hipGetLastError();
}

hipError_t launch_export(const kvq_kv_view& v, const kvq_export_bufs& o,
                         hipStream_t s) {
  const int64_t ns = (int64_t)v.batch * v.kv_heads;
  const int D = v.head_dim;
  const int64_t nq = v.n_quant, ng = v.group_tok > 0 ? nq / v.group_tok : 0;
  auto g = [](int64_t n) { return grid_for(n, 256); };
  if (v.n_sink > 0) {
    int64_t n = v.n_sink * D;
    if (o.sink_k) copy_streams_u16<<<g(n * ns), 256, 0, s>>>(v.sink_k, v.sink_stride, 0, (uint16_t*)o.sink_k, n, ns);
    if (o.sink_v) copy_streams_u16<<<g(n * ns), 256, 0, s>>>(v.sink_v, v.sink_stride, 0, (uint16_t*)o.sink_v, n, ns);
  }
  if (v.n_tail > 0) {
    int64_t n = v.n_tail * D * ns;
    if (o.tail_k) export_tail<<<g(n), 256, 0, s>>>(v.tail_k, v.tail_stride, v.residual, D, nq, v.n_tail, (uint16_t*)o.tail_k, ns);
    if (o.tail_v) export_tail<<<g(n), 256, 0, s>>>(v.tail_v, v.tail_stride, v.residual, D, nq, v.n_tail, (uint16_t*)o.tail_v, ns);
  }
  if (nq > 0) {
    if (!v.k_mixed) {
      int64_t n = nq * words_of(D, v.k_bits);
      if (o.k_codes) copy_streams_u32<<<g(n * ns), 256, 0, s>>>(v.k_codes, v.k_codes_stride, o.k_codes, n, ns);
      if (o.k_scales) copy_streams_u32<<<g(ng * D * ns), 256, 0, s>>>((const uint32_t*)v.k_scales, v.k_scales_stride, (uint32_t*)o.k_scales, ng * D, ns);
    } else {
      const int nb = v.n_bf16, n4 = v.n_int4, n2 = D - nb - n4;
      if (o.k_class) export_classes<<<g(ng * D * ns), 256, 0, s>>>(v.k_pos, v.k_pos_stride, ng * D, nb, n4, o.k_class, ns);
      if (o.k_bf16 && nb) copy_streams_u16<<<g(nq * nb * ns), 256, 0, s>>>(v.k_bf16, v.k_bf16_stride, 0, o.k_bf16, nq * nb, ns);
      if (o.k_int4 && n4) copy_streams_u32<<<g(nq * words_of(n4, 4) * ns), 256, 0, s>>>(v.k_int4, v.k_int4_stride, o.k_int4, nq * words_of(n4, 4), ns);
      if (o.k_int2 && n2) copy_streams_u32<<<g(nq * words_of(n2, 2) * ns), 256, 0, s>>>(v.k_int2, v.k_int2_stride, o.k_int2, nq * words_of(n2, 2), ns);
      if (o.k_scales) copy_streams_u32<<<g(ng * (n4 + n2) * ns), 256, 0, s>>>((const uint32_t*)v.k_scales, v.k_scales_stride, (uint32_t*)o.k_scales, ng * (n4 + n2), ns);
    }
    if (o.v_codes) {
      int64_t n = nq * words_of(D, v.v_bits);
      if (v.v_layout == KVQ_V_ROWS)
        copy_streams_u32<<<g(n * ns), 256, 0, s>>>(v.v_codes, v.v_codes_stride, o.v_codes, n, ns);
      else
        export_v_tiles<<<g(n * ns), 256, 0, s>>>(v.v_codes, v.v_codes_stride, D, v.v_bits, nq, o.v_codes, ns);
    }
    if (o.v_scales) {
      int64_t n = nq * (D / v.group_ch);
      copy_streams_u32<<<g(n * ns), 256, 0, s>>>((const uint32_t*)v.v_scales, v.v_scales_stride, (uint32_t*)o.v_scales, n, ns);
    }
  }
  return hipGetLastError();
}

hipError_t launch_synth(uint16_t* out, uint64_t seed, int tensor, int layer,
                        int head0, int n_heads, int64_t t0, int64_t n_tok,
                        int d, int64_t head_stride, hipStream_t s) {
  int64_t n = n_tok * d * n_heads;
  if (n <= 0) return hipSuccess;
  synth_kernel<<<grid_for(n, 256), 256, 0, s>>>(out, seed, tensor, layer,
                                                head0, n_heads, t0, n_tok, d,
                                                head_stride);
  return hipGetLastError();
}

}  // namespace kvq
