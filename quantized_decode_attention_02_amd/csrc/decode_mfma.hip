// Matrix-core decode attention of libkvq for gfx950 (uniform int4/int2 keys,
// int2/int4 value tiles, head_dim 128, up to 16 query heads per KV head).
//
// The two matvecs over the quantized cache ("KVQuant ...", key results: key
// and value matvec kernels; "KV quantization axes ...", "Separate the two
// error paths") are run as 16x16x32 fp16 MFMA tiles:
//
//   scores  S^T[token][head] = sum_d code[token][d] * Q'[head][d]
//           Q'[h][d] = q[h][d] * k_scale[group][d] * sm_scale * log2(e)
//   output  O^T[d][head]    += sum_t vcode[t][d] * P'[head][t]
//           P'[h][t] = 2^(s[h][t] - m[h]) * v_scale[t][d / Gv]
//
// Integer codes become exact fp16 numbers with one AND-OR against the fp16
// pattern of 1024 (0x6400) and one packed subtract; a field at a higher bit
// position arrives multiplied by 4^i or 16, which the other operand divides
// back out (powers of two, exact).  Q' is split into a high and a low fp16
// part (two MFMAs) so the scores keep float32-level accuracy; P' is a single
// fp16 (its rounding error averages out in the weighted sum).  Q' is scaled
// per key group by a power of two chosen from the group's largest |K| so it
// stays inside the fp16 range.
//
// One workgroup = 4 wavefronts = one (batch, KV head, split).  Each wave
// walks 32-token tiles i = wave, wave+4, ... of the split with its own
// online-softmax state; the four states are merged in LDS at the end.  Lane
// l = 16*q + n works on query head n (the B operand column) and on the
// MFMA k-slots 8q..8q+7.  fp16 sink and tail rows go through the general
// kernel as extra partials.
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kD = 128;
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float h2f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }

// Four fp16 pairs (one MFMA operand) from one 32-bit word of int4 codes:
// pair i holds nibbles (i, 4 + i) of the word times f_i = (1, 16, 1, 16),
// minus the offset 8: the exact values f_i * code.
__device__ inline half8 int4_operand(uint32_t w) {
  const uint32_t w8 = w >> 8;
  u32x4 r;
  r[0] = (w & 0x000F000Fu) | 0x64006400u;
  r[1] = (w & 0x00F000F0u) | 0x64006400u;
  r[2] = (w8 & 0x000F000Fu) | 0x64006400u;
  r[3] = (w8 & 0x00F000F0u) | 0x64006400u;
  half8 h = __builtin_bit_cast(half8, r);
  const half8 off = {(_Float16)1032.0f, (_Float16)1032.0f, (_Float16)1152.0f,
                     (_Float16)1152.0f, (_Float16)1032.0f, (_Float16)1032.0f,
                     (_Float16)1152.0f, (_Float16)1152.0f};
  return h - off;
}

// Four fp16 pairs from 16 bits of int2 codes (the low or high byte pair of
// a word, selected by shifting by 8 first): pair i holds fields (i, 8 + i)
// times 4^i, minus the offset 2.
__device__ inline half8 int2_operand(uint32_t ws) {
  u32x4 r;
  r[0] = (ws & 0x00030003u) | 0x64006400u;
  r[1] = (ws & 0x000C000Cu) | 0x64006400u;
  r[2] = (ws & 0x00300030u) | 0x64006400u;
  r[3] = (ws & 0x00C000C0u) | 0x64006400u;
  half8 h = __builtin_bit_cast(half8, r);
  const half8 off = {(_Float16)1026.0f, (_Float16)1026.0f, (_Float16)1032.0f,
                     (_Float16)1032.0f, (_Float16)1056.0f, (_Float16)1056.0f,
                     (_Float16)1152.0f, (_Float16)1152.0f};
  return h - off;
}

// Local channel (0..31 within the lane group's 32 channels) of k-slot
// pair i, element e, of key MFMA kb, and the factor that slot carries.
template <int KB>
__device__ inline int k_slot_channel(int kb, int i, int e) {
  if (KB == 4) return 8 * kb + i + 4 * e;
  return 16 * (kb >> 1) + 4 * (kb & 1) + i + 8 * e;
}
template <int BITS>
__device__ inline float slot_factor_inv(int i) {
  if (BITS == 4) return (i & 1) ? 0.0625f : 1.0f;
  return i == 0 ? 1.0f : (i == 1 ? 0.25f : (i == 2 ? 0.0625f : 0.015625f));
}

struct MfmaArgs {
  kvq_kv_view v;
  const void* q;
  int q_f16;
  int Hq;
  float qscale;        // sm_scale * log2(e)
  float* partials;     // [B][Hq][n_parts][D + 2]
  int n_parts;
  int n_splits;
};

template <int KB, int VB, int NC>
__global__ void __launch_bounds__(kThreads)
decode_mfma_kernel(MfmaArgs a) {
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];
  __shared__ float sm_o[kWaves][16][kD + 1];

  const kvq_kv_view& v = a.v;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lq = lane >> 4, ln = lane & 15;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int g = a.Hq / v.kv_heads;
  const int64_t s = (int64_t)b * v.kv_heads + kvh;
  const bool head_ok = ln < g;
  const int G = v.group_tok;
  const int qmax_k = (1 << (KB - 1)) - 1;

  // this lane's 32 query channels 32*lq .. 32*lq + 31 of head ln
  float qv[32];
  float qabs = 0.0f;
  {
    const int64_t base = ((int64_t)b * a.Hq + kvh * g + (head_ok ? ln : 0)) * kD + 32 * lq;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      float x = 0.0f;
      if (head_ok)
        x = a.q_f16 ? h2f(((const uint16_t*)a.q)[base + c]) : ((const float*)a.q)[base + c];
      qv[c] = x * a.qscale;
      qabs = fmaxf(qabs, fabsf(qv[c]));
    }
  }
  qabs = fmaxf(qabs, __shfl_xor(qabs, 16));
  qabs = fmaxf(qabs, __shfl_xor(qabs, 32));

  const int64_t n_tiles = v.n_quant / 32;
  const int64_t per = (n_tiles + a.n_splits - 1) / a.n_splits;
  const int64_t t_lo = min(n_tiles, (int64_t)split * per);
  const int64_t t_hi = min(n_tiles, t_lo + per);

  const uint32_t* kc = v.k_codes + s * v.k_codes_stride;
  const float* ks = v.k_scales + s * v.k_scales_stride;
  const float* kg = v.k_gmax + s * v.k_gmax_stride;
  const uint32_t* vc = v.v_codes + s * v.v_codes_stride;
  const float* vs = v.v_scales + s * v.v_scales_stride;

  half8 qhi[4], qlo[4];
  float inv_sigma = 1.0f;
  int64_t cur_group = -1;

  float m_run = -INFINITY, l_run = 0.0f;
  float4v o[8];
#pragma unroll
  for (int jb = 0; jb < 8; ++jb) o[jb] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  for (int64_t tile = t_lo + wave; tile < t_hi; tile += kWaves) {
    const int64_t tok0 = tile * 32;
    const int64_t grp = tok0 / G;
    if (grp != cur_group) {
      cur_group = grp;
      // power-of-two prescale keeping |Q'| below 2^14
      const float bound = qabs * kg[grp] / (float)qmax_k;
      int ex = (int)((__builtin_bit_cast(uint32_t, bound) >> 23) & 0xFF) - 127;
      ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
      const float sigma = __builtin_bit_cast(float, (uint32_t)(127 + 13 - ex) << 23);
      inv_sigma = __builtin_bit_cast(float, (uint32_t)(127 - 13 + ex) << 23);
      const float* kss = ks + grp * kD + 32 * lq;
      float ksv[32];
#pragma unroll
      for (int c = 0; c < 32; c += 4) {
        float4v t4 = *(const float4v*)(kss + c);
        ksv[c] = t4[0]; ksv[c + 1] = t4[1]; ksv[c + 2] = t4[2]; ksv[c + 3] = t4[3];
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int c = k_slot_channel<KB>(kb, i, e);
            const float x = qv[c] * ksv[c] * sigma * slot_factor_inv<KB>(i);
            const _Float16 hi = (_Float16)x;
            qhi[kb][2 * i + e] = hi;
            qlo[kb][2 * i + e] = (_Float16)(x - (float)hi);
          }
        }
      }
    }

    // ---- scores for the 32 tokens: two 16-token halves
    float sc[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t tok = tok0 + 16 * h + ln;
      float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
      if (KB == 4) {
        const u32x4 w = *(const u32x4*)(kc + tok * 16 + 4 * lq);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const half8 A = int4_operand(w[kb]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qhi[kb], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qlo[kb], acc, 0, 0, 0);
        }
      } else {
        const u32x2 w = *(const u32x2*)(kc + tok * 8 + 2 * lq);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const uint32_t word = w[kb >> 1];
          const half8 A = int2_operand((kb & 1) ? (word >> 8) : word);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qhi[kb], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qlo[kb], acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[4 * h + j] = acc[j] * inv_sigma;
    }

    // ---- online softmax; slot sigma of this lane is token
    //      (sigma % 4) + 4*lq + 16*(sigma / 4) of the tile, head ln
    float tmax = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, sc[i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float p[8];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = exp2f(sc[i] - m_new);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) o[jb] *= alpha;

    // ---- values
    float vsc[8][NC];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* row = vs + (tok0 + 16 * r + 4 * lq + j) * NC;
#pragma unroll
        for (int c = 0; c < NC; ++c) vsc[4 * r + j][c] = row[c];
      }
    }
    half8 pb[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int sl = 0; sl < 8; ++sl)
        pb[c][sl] = (_Float16)(p[sl] * vsc[sl][c] * slot_factor_inv<VB>(sl >> 1));
    }
    if (VB == 2) {
      const u32x4 w = *(const u32x4*)(vc + tile * 256 + lane * 4);
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) {
        const uint32_t word = w[jb >> 1];
        const half8 A = int2_operand((jb & 1) ? (word >> 8) : word);
        o[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, pb[(jb * 16 * NC) / kD], o[jb], 0, 0, 0);
      }
    } else {
      const u32x4 w0 = *(const u32x4*)(vc + tile * 512 + lane * 4);
      const u32x4 w1 = *(const u32x4*)(vc + tile * 512 + 256 + lane * 4);
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) {
        const uint32_t word = jb < 4 ? w0[jb] : w1[jb - 4];
        const half8 A = int4_operand(word);
        o[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, pb[(jb * 16 * NC) / kD], o[jb], 0, 0, 0);
      }
    }
  }

  // ---- per-wave state to LDS: m, l (summed over the 4 lane groups), O
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (lq == 0) {
    sm_m[wave][ln] = m_run;
    sm_l[wave][ln] = l_run;
  }
#pragma unroll
  for (int jb = 0; jb < 8; ++jb)
#pragma unroll
    for (int j = 0; j < 4; ++j) sm_o[wave][ln][16 * jb + 4 * lq + j] = o[jb][j];
  __syncthreads();

  // ---- merge the four waves into this split's partial
  for (int i = threadIdx.x; i < g * (kD + 2); i += kThreads) {
    const int h = i / (kD + 2), jx = i % (kD + 2);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (sm_l[w][h] > 0.0f) M = fmaxf(M, sm_m[w][h]);
    float val = 0.0f;
    if (jx == 0) {
      val = M;
    } else {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        if (sm_l[w][h] > 0.0f) {
          const float sc_w = exp2f(sm_m[w][h] - M);
          val += (jx == 1 ? sm_l[w][h] : sm_o[w][h][jx - 2]) * sc_w;
        }
      }
    }
    a.partials[(((int64_t)b * a.Hq + kvh * g + h) * a.n_parts + split) * (kD + 2) + jx] = val;
  }
}

int auto_splits(const kvq_kv_view& v) {
  const int64_t n_tiles = v.n_quant / 32;
  const int64_t streams = (int64_t)v.batch * v.kv_heads;
  int64_t sp = (2048 + streams - 1) / streams;
  int64_t by_len = n_tiles / 8;  // at least two tiles per wave
  if (sp > by_len) sp = by_len;
  if (sp < 1) sp = 1;
  if (sp > 65535) sp = 65535;
  return (int)sp;
}

int fp16_parts(const kvq_kv_view& v) {
  return (v.n_sink > 0 ? 1 : 0) + (int)((v.n_tail + 63) / 64);
}

template <int KB, int VB, int NC>
hipError_t launch_t(const MfmaArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.n_splits, (unsigned)a.v.kv_heads, (unsigned)a.v.batch);
  decode_mfma_kernel<KB, VB, NC><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_nc(const MfmaArgs& a, int nc, hipStream_t s) {
  switch (nc) {
    case 1: return launch_t<KB, VB, 1>(a, s);
    case 2: return launch_t<KB, VB, 2>(a, s);
    case 4: return launch_t<KB, VB, 4>(a, s);
    case 8: return launch_t<KB, VB, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool mfma_decode_eligible(const kvq_kv_view& v, int Hq) {
  if (v.head_dim != kD || v.k_mixed) return false;
  if (v.k_bits != 4 && v.k_bits != 2) return false;
  if (v.v_bits != 4 && v.v_bits != 2) return false;
  if (v.v_layout != KVQ_V_TILE32 || v.group_tok % 32 || v.n_quant % 32) return false;
  if (v.n_quant < 32 || !v.k_gmax) return false;
  const int nc = kD / v.group_ch;
  if (nc != 1 && nc != 2 && nc != 4 && nc != 8) return false;
  const int g = Hq / v.kv_heads;
  return g >= 1 && g <= 16;
}

int mfma_decode_parts(const kvq_kv_view& v, int Hq, int n_splits) {
  (void)Hq;
  const int sp = n_splits > 0 ? n_splits : auto_splits(v);
  return sp + fp16_parts(v);
}

hipError_t launch_decode_mfma(const kvq_kv_view& v, const void* q, int f16, int Hq,
                              float sm_scale, float* partials, int n_parts,
                              hipStream_t s) {
  const int fp = fp16_parts(v);
  const int n_splits = n_parts - fp;
  MfmaArgs a{v, q, f16, Hq, sm_scale * kLog2e, partials, n_parts, n_splits};
  const int nc = kD / v.group_ch;
  hipError_t e;
  if (v.k_bits == 4 && v.v_bits == 2) e = launch_nc<4, 2>(a, nc, s);
  else if (v.k_bits == 4 && v.v_bits == 4) e = launch_nc<4, 4>(a, nc, s);
  else if (v.k_bits == 2 && v.v_bits == 2) e = launch_nc<2, 2>(a, nc, s);
  else e = launch_nc<2, 4>(a, nc, s);
  if (e != hipSuccess) return e;
  // fp16 rows: the sink as one partial, the tail in 64-token partials
  int part = n_splits;
  if (v.n_sink > 0) {
    e = launch_decode_generic_range(v, q, f16, Hq, sm_scale, partials, 0, v.n_sink, 1, part,
                                    n_parts, s);
    if (e != hipSuccess) return e;
    part += 1;
  }
  if (v.n_tail > 0) {
    const int tp = (int)((v.n_tail + 63) / 64);
    const int64_t lo = v.n_sink + v.n_quant;
    e = launch_decode_generic_range(v, q, f16, Hq, sm_scale, partials, lo, lo + v.n_tail, tp,
                                    part, n_parts, s);
  }
  return e;
}

}  // namespace kvq
