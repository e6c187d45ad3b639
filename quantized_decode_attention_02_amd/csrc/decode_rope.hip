// Decode attention over keys cached before the rotary position embedding
// ("KVQuant: Towards 10 Million Context Length LLM Inference with KV Cache
// Quantization", "Approach": per-channel key quantization before RoPE), for
// uniform int8 / int4 / int2 keys or mixed bf16 / int4 / int2 keys (the
// MixKVQ layout), int4 / int2 value tiles and D = 128.
//
// Cache-order token i sits at position pos0 + i.  Writing the position of a
// quantized token as t0 + j, with t0 the position of the first token of its
// 32-token tile, the two rotations compose:
//     q . R(t0 + j) k = (R(-t0) q) . (R(j) k),
// so the query turns back by t0 once per tile, and the turn by j uses the
// cosines and sines of j * theta_f (j = 0..31): one table in LDS for the
// whole workgroup.  For channel d with pair partner e and sign sigma (+1 for
// the first channel of its pair, -1 for the second), a key with codes c_d
// and per-channel group scales s_d scores
//     sum_d c_d * (cos(j theta_f) Q1_d + sin(j theta_f) Q2_d),
//     Q1_d = s_d (R(-t0) q)_d,   Q2_d = sigma s_d (R(-t0) q)_e,
// in float32: two multiply-adds form a code's weight, a third adds it in.
// Scores are in log2 units (q carries sm_scale * log2(e)).
//
// Work split: a 256-thread workgroup takes a range of 32-token tiles of one
// (batch, KV head) stream; its four waves take every fourth tile and keep
// their own running max, sum and output, combined in LDS at the end into
// one partial (m, l, o).  In a tile, lane 16 r + c scores eight channels of
// the tokens 4 s + r (s = 0..7): 8c .. 8c + 7 for interleaved pairs,
// 4c .. 4c + 3 and 64 + 4c .. 64 + 4c + 3 for half pairs (both members of
// four pairs either way), and 16-lane DPP sums complete the scores.  Values
// keep the value-tile layout: lane 16 q + m
// holds channel 16 jb + m at eight tokens of the tile and reads their
// softmax weights, times the token's value scale, from LDS.  The fp16 sink
// and tail tokens go through the general kernel as one range, 32 tokens per
// partial.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kvq_internal.h"
#include "rope_math.h"

namespace kvq {
namespace {

constexpr int kRWaves = 4;
constexpr int kRThreads = 64 * kRWaves;
constexpr int kRD = 128;             // head_dim of this kernel
constexpr int kRNF = kRD / 2;        // frequencies
constexpr int kRTile = 32;           // tokens per tile
constexpr int kRSteps = 8;           // wave steps per tile, 4 tokens each
constexpr int kRBlocks = kRD / 16;   // value channel blocks
constexpr int kRMaxGroups = 8;       // value groups per token (Gv >= 16)
constexpr float kRLog2e = 1.4426950408889634f;

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streamed once per call: nontemporal loads keep the codes out of the caches.
template <typename T>
__device__ inline T ldnt(const T* p) { return __builtin_nontemporal_load(p); }

// Two codes sitting 16 bits apart in x (low bits of each half) as exact
// fp16 values u - 2^(BITS-1): OR-ing 0x6400 makes 1024 + u, then one packed
// subtract removes 1024 + 2^(BITS-1).
template <int BITS>
__device__ inline half2v code_pair(uint32_t x) {
  constexpr uint32_t mask = (BITS == 8 ? 0xFFu : BITS == 4 ? 0xFu : 0x3u) * 0x00010001u;
  const half2v h = __builtin_bit_cast(half2v, (x & mask) | 0x64006400u);
  constexpr _Float16 off = (_Float16)(1024 + (1 << (BITS - 1)));
  return h - half2v{off, off};
}

template <int CTRL>
__device__ inline float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a row (row_ror 8, 4, 2, 1): every lane gets it.
__device__ inline float row_sum16(float x) {
  x += dpp_f<0x128>(x);
  x += dpp_f<0x124>(x);
  x += dpp_f<0x122>(x);
  x += dpp_f<0x121>(x);
  return x;
}
// Max over the 16 lanes of a row (every lane gets it).
__device__ inline float row_max16(float x) {
  x = fmaxf(x, dpp_f<0x128>(x));
  x = fmaxf(x, dpp_f<0x124>(x));
  x = fmaxf(x, dpp_f<0x122>(x));
  x = fmaxf(x, dpp_f<0x121>(x));
  return x;
}
// Reduce-scatter of eight per-lane partial sums over the 16 lanes of a row:
// lane c ends with the full sum of entry 4 b3 + 2 b1 + b0 (bits of c), as
// does lane c ^ 4.  Partners c ^ 8 (DPP row_ror 8), c ^ 2 and c ^ 1 (DPP
// quad permutations) each take the half the lane keeps; c ^ 4 (swizzle)
// completes the sum.
__device__ inline float row_reduce_scatter8(const float a[8], int c) {
  const bool b3 = c & 8, b1 = c & 2, b0 = c & 1;
  float t1[4], t2[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float keep = b3 ? a[k + 4] : a[k], give = b3 ? a[k] : a[k + 4];
    t1[k] = keep + dpp_f<0x128>(give);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float keep = b1 ? t1[k + 2] : t1[k], give = b1 ? t1[k] : t1[k + 2];
    t2[k] = keep + dpp_f<0x4E>(give);  // quad_perm [2, 3, 0, 1]: lane ^ 2
  }
  const float keep = b0 ? t2[1] : t2[0], give = b0 ? t2[0] : t2[1];
  const float t3 = keep + dpp_f<0xB1>(give);  // quad_perm [1, 0, 3, 2]: lane ^ 1
  return t3 + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(
                                            __builtin_bit_cast(int, t3), (4 << 10) | 0x1F));
}
__device__ inline float lane_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// Key codes of one lane's 8 channels: pair i holds channels (lo_e(i), hi_e(i)).
template <int KB>
__device__ constexpr int lo_e(int i) { return KB == 8 ? (i & 1) + 4 * (i >> 1) : i; }
template <int KB>
__device__ constexpr int hi_e(int i) { return KB == 8 ? lo_e<KB>(i) + 2 : i + 4; }

// Key words one lane loads per token.  Interleaved pairs: channels
// 8c .. 8c + 7, one or two consecutive words.  Half pairs: channels
// 4c .. 4c + 3 and 64 + 4c .. 64 + 4c + 3 (both members of four pairs), from
// two words; lane channel e < 4 is 4c + e, e >= 4 is 64 + 4c + e - 4.
template <int KB, bool INTER>
struct KWords {
  typedef typename std::conditional<
      KB == 0, u32x4, typename std::conditional<KB == 8 || !INTER, u32x2, uint32_t>::type>::type T;
};

// The lane's 8 codes as 4 fp16 pairs; pair i holds lane channels
// (lo_e(i), hi_e(i)).
template <int KB, bool INTER>
__device__ inline void key_pairs(typename KWords<KB, INTER>::T w, int c, half2v p[4]) {
  if constexpr (KB == 0) {
    (void)w;
    (void)c;
  } else if constexpr (KB == 8) {
    p[0] = code_pair<8>(w[0]);
    p[1] = code_pair<8>(w[0] >> 8);
    p[2] = code_pair<8>(w[1]);
    p[3] = code_pair<8>(w[1] >> 8);
  } else {
    uint32_t z;
    if constexpr (KB == 4) {
      if constexpr (INTER) {
        z = w;
      } else {
        const int sh = 16 * (c & 1);
        z = ((w[0] >> sh) & 0xFFFFu) | ((w[1] >> sh) << 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = code_pair<4>(z >> (4 * i));
    } else {
      uint32_t y;
      if constexpr (INTER) {
        y = w >> (16 * (c & 1));
      } else {
        const int sh = 8 * (c & 3);
        y = ((w[0] >> sh) & 0xFFu) | (((w[1] >> sh) & 0xFFu) << 8);
      }
      z = (y & 0xFFu) | ((y << 8) & 0x00FF0000u);
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = code_pair<2>(z >> (2 * i));
    }
  }
}

// Weight slots per token in LDS: RS kernels write one per value group,
// the others one per key lane (groups past D/Gv are never read).
template <bool RS>
constexpr int pv_slots() { return RS ? kRMaxGroups : 16; }

template <int GQ, bool RS>
struct RopeLds {
  double phi[kRNF];                       // turns per position
  float2 tab[kRTile][kRNF];               // (cos, sin) of j * theta_f
  float2 qs[GQ][kRD];                     // (q_d, sigma q_e) * qscale
  float2 base[kRWaves][kRNF];             // (cos, sin) of t0 * theta_f
  uint8_t inv[kRWaves][kRD];              // mixed keys: channel of each class position
  float pv[kRWaves][GQ][pv_slots<RS>()][kRTile];  // weight * value scale
  float comb[kRWaves][GQ][kRD + 2];       // per-wave (m, l, o)
};

// GQ query heads h_off .. h_off + GQ - 1 of each KV head's g = Hq / Hkv.
// RS: scores summed by a reduce-scatter (one token per lane afterwards: one
// exp per lane and tile); otherwise every lane gets all eight row sums.
// The one-head kernel keeps the latter: it then fits three waves per SIMD.
template <int KB, int VB, int GQ, bool INTER, typename QT, bool RS = (GQ >= 2)>
__global__ void __launch_bounds__(kRThreads)
__attribute__((amdgpu_waves_per_eu((RS || KB == 0) ? 2 : 3)))
decode_rope_kernel(kvq_kv_view v, const QT* __restrict__ q, int Hq, float qscale,
                   RopeDev rope, float* __restrict__ partials, int n_parts, int part_stride,
                   int gv_shift, int h_off) {
  __shared__ RopeLds<GQ, RS> L;
  constexpr int kSlots = pv_slots<RS>();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int64_t s = (int64_t)b * v.kv_heads + kvh;
  const int c = lane & 15, r = lane >> 4;  // key role: channel chunk, token
  const int q4 = r, m16 = c;               // value role: token quarter, channel
  const int NG = kRD >> gv_shift;

  for (int f = tid; f < kRNF; f += kRThreads) L.phi[f] = rope.phi[f];
  for (int i = tid; i < GQ * kRD; i += kRThreads) {
    const int h = i / kRD, d = i % kRD;
    const int e = INTER ? (d ^ 1) : (d < kRNF ? d + kRNF : d - kRNF);
    const float sg = (INTER ? (d & 1) : (d >= kRNF)) ? -1.0f : 1.0f;
    const int64_t qrow = ((int64_t)b * Hq + (int64_t)kvh * (Hq / v.kv_heads) + h_off + h) * kRD;
    float qd, qe;
    if constexpr (sizeof(QT) == 2) {
      qd = (float)__builtin_bit_cast(_Float16, q[qrow + d]);
      qe = (float)__builtin_bit_cast(_Float16, q[qrow + e]);
    } else {
      qd = q[qrow + d];
      qe = q[qrow + e];
    }
    L.qs[h][d] = make_float2(qd * qscale, sg * qe * qscale);
  }
  __syncthreads();
  for (int i = tid; i < kRTile * kRNF; i += kRThreads) {
    const int j = i / kRNF, f = i % kRNF;
    L.tab[j][f] = rope_cos_sin(rope_turns((double)j, L.phi[f]));
  }
  __syncthreads();

  // this workgroup's tiles; wave w takes tiles t_lo + w, t_lo + w + 4, ...
  const int64_t n_tiles = v.n_quant / kRTile;
  const int64_t per = (n_tiles + n_parts - 1) / n_parts;
  const int64_t t_lo = (int64_t)part * per < n_tiles ? (int64_t)part * per : n_tiles;
  const int64_t t_hi = t_lo + per < n_tiles ? t_lo + per : n_tiles;

  const uint32_t* kc = v.k_codes + s * v.k_codes_stride;
  const float* ksc = v.k_scales + s * v.k_scales_stride;
  const uint32_t* vc = v.v_codes + s * v.v_codes_stride;
  const float* vsc_base = v.v_scales + s * v.v_scales_stride;
  constexpr uint32_t KWD = kRD * KB / 32;  // key words per token
  // first key word of the lane, and (half pairs) the second one
  const uint32_t kcol = INTER ? (KB == 4 ? c : KB == 8 ? 2 * c : (c >> 1))
                              : (KB == 4 ? (c >> 1) : KB == 8 ? c : (c >> 2));
  constexpr uint32_t kcol2 = KWD / 2;
  // after the score reduce-scatter this lane holds token 4 ks_tok + r
  const int ks_tok = ((c >> 3) & 1) * 4 + ((c >> 1) & 1) * 2 + (c & 1);
  const int fbase = 4 * c;                 // the lane's four frequencies
  // lane channel e: its channel, and its frequency's offset from fbase
  auto chan = [&](int e) { return INTER ? 8 * c + e : (e < 4 ? 4 * c + e : kRNF + 4 * c + e - 4); };
  auto fi = [](int e) { return INTER ? e >> 1 : e & 3; };
  // Mixed keys (KB == 0): a score is a sum over channels in any order, so
  // lane c takes the class positions 8 c .. 8 c + 7 (bf16 positions first,
  // then int4, then int2; every class a multiple of eight positions): eight
  // consecutive entries of one class row, one load per token.  Per key
  // group the lane looks up the channel and frequency of each position
  // (the inverse of the group's class map) and the int positions' scales.
  constexpr bool KM = KB == 0;
  const int NB = KM ? v.n_bf16 : 0, N4 = KM ? v.n_int4 : 0, N2 = kRD - NB - N4;
  const int kp0 = 8 * c;
  const int kcls = kp0 < NB ? 0 : (kp0 < NB + N4 ? 1 : 2);  // bf16, int4, int2
  const uint32_t* kmb = nullptr;  // the lane's class array (this stream)
  uint32_t krw = 0, kwo = 0;      // its row words, the lane's first word
  int k2sh = 0;                   // int2: bit offset of the lane's 16 bits
  if constexpr (KM) {
    if (kcls == 0) {
      kmb = (const uint32_t*)(v.k_bf16 + s * v.k_bf16_stride);
      krw = (uint32_t)NB / 2;
      kwo = (uint32_t)kp0 / 2;
    } else if (kcls == 1) {
      kmb = v.k_int4 + s * v.k_int4_stride;
      krw = (uint32_t)N4 / 8;
      kwo = (uint32_t)(kp0 - NB) / 8;
    } else {
      kmb = v.k_int2 + s * v.k_int2_stride;
      krw = (uint32_t)(N2 + 15) / 16;
      kwo = (uint32_t)(kp0 - NB - N4) / 16;
      k2sh = 16 * (((kp0 - NB - N4) / 8) & 1);
    }
  }
  const uint8_t* kpos = KM ? v.k_pos + s * v.k_pos_stride : nullptr;
  int dch[KM ? 8 : 1], dfr[KM ? 8 : 1];  // channel and frequency of each position

  float m_run[GQ], l_run[GQ], o[GQ][kRBlocks];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.0f;
#pragma unroll
    for (int jb = 0; jb < kRBlocks; ++jb) o[h][jb] = 0.0f;
  }

  // One register buffer per kind, refilled for the wave's next tile right
  // after its last use in the current one (offsets within a stream are
  // 32-bit: the view's eligibility bounds them).
  typedef typename KWords<KB, INTER>::T KW;
  KW kw[kRSteps];
  u32x4 vw[VB == 4 ? 2 : 1];
  float vs[RS ? kRMaxGroups : kRSteps];
  auto load_k = [&](int64_t T) {
    const uint32_t row0 = (uint32_t)T * kRTile + r;
#pragma unroll
    for (int st = 0; st < kRSteps; ++st) {
      const uint32_t off = (row0 + 4 * st) * KWD + kcol;
      if constexpr (KM) {
        const uint32_t o2 = (row0 + 4 * st) * krw + kwo;
        if (kcls == 0)
          kw[st] = ldnt((const u32x4*)(kmb + o2));
        else
          kw[st][0] = ldnt(kmb + o2);
      } else if constexpr (!INTER) {
        kw[st][0] = ldnt(kc + off);
        kw[st][1] = ldnt(kc + off + kcol2);
      } else if constexpr (KB == 8) {
        kw[st] = ldnt((const u32x2*)(kc + off));
      } else {
        kw[st] = ldnt(kc + off);
      }
    }
  };
  auto load_vs = [&](int64_t T) {
    if constexpr (RS) {
      const uint32_t row = (uint32_t)T * kRTile + 4 * ks_tok + r;
#pragma unroll
      for (int g = 0; g < kRMaxGroups; ++g)
        if (g < NG) vs[g] = ldnt(vsc_base + row * NG + g);
    } else {
      const uint32_t row0 = (uint32_t)T * kRTile + r;
#pragma unroll
      for (int st = 0; st < kRSteps; ++st)
        vs[st] = ldnt(vsc_base + (row0 + 4 * st) * NG + (c & (NG - 1)));
    }
  };
  auto load_v = [&](int64_t T) {
    const uint32_t* tw = vc + (uint32_t)T * (uint32_t)(kRD * VB);
    vw[0] = ldnt((const u32x4*)(tw + lane * 4));
    if constexpr (VB == 4) vw[VB == 4 ? 1 : 0] = ldnt((const u32x4*)(tw + 256 + lane * 4));
  };

  int64_t cur_grp = -1;
  float ks[8];
  int64_t T = t_lo + wave;
  if (T < t_hi) {
    load_k(T);
    load_vs(T);
    load_v(T);
  }
  for (; T < t_hi; T += kRWaves) {
    const bool more = T + kRWaves < t_hi;
    const int64_t qt0 = T * kRTile;
    const int64_t grp = (uint32_t)qt0 / (uint32_t)v.group_tok;  // qt0 < 2^26
    if (KM && grp != cur_grp) {
      cur_grp = grp;
      for (int d = lane; d < kRD; d += 64) L.inv[wave][kpos[grp * kRD + d]] = (uint8_t)d;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dch[KM ? e : 0] = L.inv[wave][kp0 + e];
        dfr[KM ? e : 0] = INTER ? dch[KM ? e : 0] >> 1 : dch[KM ? e : 0] & (kRNF - 1);
        ks[e] = kcls == 0 ? 1.0f : ksc[grp * (N4 + N2) + kp0 + e - NB];
      }
      __builtin_amdgcn_wave_barrier();
    } else if (!KM && grp != cur_grp) {
      cur_grp = grp;
      const float4v a = *(const float4v*)(ksc + grp * kRD + chan(0));
      const float4v bq = *(const float4v*)(ksc + grp * kRD + chan(4));
      ks[0] = a[0]; ks[1] = a[1]; ks[2] = a[2]; ks[3] = a[3];
      ks[4] = bq[0]; ks[5] = bq[1]; ks[6] = bq[2]; ks[7] = bq[3];
    }
    // (cos, sin) of the tile's first position at every frequency
    const double p0 = (double)(rope.pos0 + v.n_sink + qt0);
    L.base[wave][lane] = rope_cos_sin(rope_turns(p0, L.phi[lane]));
    __builtin_amdgcn_wave_barrier();

    float sc[GQ][kRSteps];
    // Q1, Q2 of this lane's channels for the tile
    float Q1[GQ][8], Q2[GQ][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 cs = L.base[wave][KM ? dfr[KM ? e : 0] : fbase + fi(e)];
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float2 qq = L.qs[h][KM ? dch[KM ? e : 0] : chan(e)];
        Q1[h][e] = ks[e] * (cs.x * qq.x + cs.y * qq.y);
        Q2[h][e] = ks[e] * (cs.x * qq.y - cs.y * qq.x);
      }
    }
    // scores of the tile's 32 tokens: code times weight
#pragma unroll
    for (int st = 0; st < kRSteps; ++st) {
      const int j = 4 * st + r;
      if constexpr (KM) {
        // the lane's eight entries as floats (exact): bf16 values, or
        // int4 / int2 codes minus their offsets
        float x[8];
        float2 t8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t8[e] = L.tab[j][dfr[KM ? e : 0]];
        const u32x4 w = kw[st];
        if (kcls == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
            x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
          }
        } else if (kcls == 1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = (float)(int)((w[0] >> (4 * e)) & 0xFu) - 8.0f;
        } else {
          const uint32_t y = w[0] >> k2sh;
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = (float)(int)((y >> (2 * e)) & 0x3u) - 2.0f;
        }
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
          float acc = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc = __builtin_fmaf(x[e], t8[e].x * Q1[h][e] + t8[e].y * Q2[h][e], acc);
          sc[h][st] = RS ? acc : row_sum16(acc);
        }
        continue;
      }
      float2 t[4];
      const float4v* tp = (const float4v*)&L.tab[j][fbase];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float4v x = tp[k];
        t[2 * k] = make_float2(x[0], x[1]);
        t[2 * k + 1] = make_float2(x[2], x[3]);
      }
      half2v pr[4];
      key_pairs<KB, INTER>(kw[st], c, pr);
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int el = lo_e<KB>(i), eh = hi_e<KB>(i);
          const float2 tl = t[fi(el)], th = t[fi(eh)];
          const float wl = tl.x * Q1[h][el] + tl.y * Q2[h][el];
          const float wh = th.x * Q1[h][eh] + th.y * Q2[h][eh];
          acc = __builtin_fmaf((float)pr[i][0], wl, acc);
          acc = __builtin_fmaf((float)pr[i][1], wh, acc);
        }
        sc[h][st] = RS ? acc : row_sum16(acc);  // RS: summed below
      }
    }
    if (more) load_k(T + kRWaves);

    // online softmax over the tile; weights times value scales into LDS.
    // RS: lane 16 r + c holds the score of token 4 ks + r (ks = 4 b3 + 2 b1
    // + b0 of c; lanes c and c ^ 4 alike); otherwise all eight of its row.
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      float mx, sv = 0.0f;
      if constexpr (RS) {
        sv = row_reduce_scatter8(sc[h], c);
        mx = row_max16(sv);
      } else {
        mx = sc[h][0];
#pragma unroll
        for (int st = 1; st < kRSteps; ++st) mx = fmaxf(mx, sc[h][st]);
      }
      mx = fmaxf(fmaxf(lane_f(mx, 0), lane_f(mx, 16)), fmaxf(lane_f(mx, 32), lane_f(mx, 48)));
      const float mnew = fmaxf(m_run[h], mx);
      // v_exp_f32 flushes results below 2^-126 to zero: such a weight next
      // to the running maximum's weight 1 cannot change a float32 sum
      const float alpha = __builtin_amdgcn_exp2f(m_run[h] - mnew);
      m_run[h] = mnew;
      float psum = 0.0f;
      if constexpr (RS) {
        const float p = __builtin_amdgcn_exp2f(sv - mnew);
#pragma unroll
        for (int g = 0; g < kRMaxGroups; ++g)
          if (g < NG) L.pv[wave][h][g][4 * ks_tok + r] = p * vs[g];
        psum = (c & 4) ? 0.0f : p;  // each token counted once
      } else {
#pragma unroll
        for (int st = 0; st < kRSteps; ++st) {
          const float p = __builtin_amdgcn_exp2f(sc[h][st] - mnew);
          psum += p;
          L.pv[wave][h][c][4 * st + r] = p * vs[st];
        }
      }
      l_run[h] = l_run[h] * alpha + psum;
#pragma unroll
      for (int jb = 0; jb < kRBlocks; ++jb) o[h][jb] *= alpha;
    }
    if (more) load_vs(T + kRWaves);
    __builtin_amdgcn_wave_barrier();

    // values: channel 16 jb + m16 at tokens tau(q4, s), s = 0..7
#pragma unroll
    for (int jb = 0; jb < kRBlocks; ++jb) {
      const float* pw = &L.pv[wave][0][(16 * jb) >> gv_shift][4 * q4];
      float4v wlo[GQ], whi[GQ];
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        wlo[h] = *(const float4v*)(pw + h * kSlots * kRTile);
        whi[h] = *(const float4v*)(pw + h * kSlots * kRTile + 16);
      }
      half2v pr[4];
      if constexpr (VB == 2) {
        const uint32_t w = vw[0][jb >> 1];
        const int sh = (jb & 1) ? 8 : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = code_pair<2>(w >> (sh + 2 * i));
      } else {
        const uint32_t w = vw[jb >> 2][jb & 3];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = code_pair<4>(w >> (4 * i));
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        float acc = o[h][jb];
        acc = __builtin_fmaf((float)pr[0][0], wlo[h][0], acc);
        acc = __builtin_fmaf((float)pr[0][1], wlo[h][1], acc);
        acc = __builtin_fmaf((float)pr[1][0], wlo[h][2], acc);
        acc = __builtin_fmaf((float)pr[1][1], wlo[h][3], acc);
        acc = __builtin_fmaf((float)pr[2][0], whi[h][0], acc);
        acc = __builtin_fmaf((float)pr[2][1], whi[h][1], acc);
        acc = __builtin_fmaf((float)pr[3][0], whi[h][2], acc);
        acc = __builtin_fmaf((float)pr[3][1], whi[h][3], acc);
        o[h][jb] = acc;
      }
    }
    if (more) load_v(T + kRWaves);
  }

  // per wave: l over the four token rows, o over the four token quarters
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    // RS: lanes hold their own tokens' sums; otherwise every lane its row's
    const float lrow = RS ? row_sum16(l_run[h]) : l_run[h];
    const float lw = lane_f(lrow, 0) + lane_f(lrow, 16) + lane_f(lrow, 32) + lane_f(lrow, 48);
#pragma unroll
    for (int jb = 0; jb < kRBlocks; ++jb) {
      float x = o[h][jb];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      if (q4 == 0) L.comb[wave][h][2 + 16 * jb + m16] = x;
    }
    if (lane == 0) {
      L.comb[wave][h][0] = m_run[h];
      L.comb[wave][h][1] = lw;
    }
  }
  __syncthreads();
  for (int i = tid; i < GQ * (kRD + 2); i += kRThreads) {
    const int h = i / (kRD + 2), j = i % (kRD + 2);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kRWaves; ++w)
      if (L.comb[w][h][1] > 0.0f) M = fmaxf(M, L.comb[w][h][0]);
    float val = 0.0f;
    if (j == 0) {
      val = M;
    } else {
#pragma unroll
      for (int w = 0; w < kRWaves; ++w)
        if (L.comb[w][h][1] > 0.0f) val += L.comb[w][h][j] * exp2f(L.comb[w][h][0] - M);
    }
    partials[(((int64_t)b * Hq + (int64_t)kvh * (Hq / v.kv_heads) + h_off + h) * part_stride +
              part) * (kRD + 2) + j] =
        val;
  }
}

template <int KB, int VB, int GQ, bool INTER>
hipError_t launch_rope_t(const kvq_kv_view& v, const void* q, int f16, int Hq, float qscale,
                         const RopeDev& rope, float* partials, int n_parts, int part_stride,
                         int gv_shift, int h_off, hipStream_t s) {
  dim3 grid((unsigned)n_parts, (unsigned)v.kv_heads, (unsigned)v.batch);
  if (f16)
    decode_rope_kernel<KB, VB, GQ, INTER, uint16_t><<<grid, kRThreads, 0, s>>>(
        v, (const uint16_t*)q, Hq, qscale, rope, partials, n_parts, part_stride, gv_shift,
        h_off);
  else
    decode_rope_kernel<KB, VB, GQ, INTER, float><<<grid, kRThreads, 0, s>>>(
        v, (const float*)q, Hq, qscale, rope, partials, n_parts, part_stride, gv_shift, h_off);
  return hipGetLastError();
}

// Query heads per KV head taken two at a time (the last alone when their
// count is odd); each launch reads the cache once.
template <int KB, int VB>
hipError_t launch_rope_g(const kvq_kv_view& v, const void* q, int f16, int Hq, float qscale,
                         const RopeDev& rope, float* partials, int n_parts, int part_stride,
                         int gv_shift, hipStream_t s) {
  const int g = Hq / v.kv_heads;
  if constexpr (KB == 0) {
    // mixed keys: one query head per launch (the per-lane channel map
    // leaves no registers for a second head)
    for (int h = 0; h < g; ++h) {
      const hipError_t e =
          rope.interleaved
              ? launch_rope_t<KB, VB, 1, true>(v, q, f16, Hq, qscale, rope, partials, n_parts,
                                               part_stride, gv_shift, h, s)
              : launch_rope_t<KB, VB, 1, false>(v, q, f16, Hq, qscale, rope, partials, n_parts,
                                                part_stride, gv_shift, h, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  } else {
    for (int h0 = 0; h0 < g; h0 += 2) {
      hipError_t e;
      if (h0 + 2 > g)
        e = rope.interleaved
                ? launch_rope_t<KB, VB, 1, true>(v, q, f16, Hq, qscale, rope, partials, n_parts,
                                                 part_stride, gv_shift, h0, s)
                : launch_rope_t<KB, VB, 1, false>(v, q, f16, Hq, qscale, rope, partials,
                                                  n_parts, part_stride, gv_shift, h0, s);
      else
        e = rope.interleaved
                ? launch_rope_t<KB, VB, 2, true>(v, q, f16, Hq, qscale, rope, partials, n_parts,
                                                 part_stride, gv_shift, h0, s)
                : launch_rope_t<KB, VB, 2, false>(v, q, f16, Hq, qscale, rope, partials,
                                                  n_parts, part_stride, gv_shift, h0, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
}

bool aligned_to(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

bool rope_fast_eligible(const kvq_kv_view& v, int Hq) {
  const int g = Hq / v.kv_heads;
  if (v.head_dim != kRD) return false;
  if (v.k_mixed) {
    // whole eight-position lanes per class; 16-byte bf16 loads
    const int nb = v.n_bf16, n4 = v.n_int4;
    if (nb < 0 || n4 < 0 || nb % 8 || n4 % 8 || nb + n4 > kRD || !v.k_pos) return false;
    if (nb && !(aligned_to(v.k_bf16, 16) && v.k_bf16_stride % 8 == 0)) return false;
    if (n4 && !v.k_int4) return false;
    if (nb + n4 < kRD && !v.k_int2) return false;
  } else {
    if (v.k_bits != 2 && v.k_bits != 4 && v.k_bits != 8) return false;
    if (!(aligned_to(v.k_codes, 16) && v.k_codes_stride % 4 == 0 && aligned_to(v.k_scales, 16) &&
          v.k_scales_stride % 4 == 0))
      return false;
  }
  if (v.v_bits != 2 && v.v_bits != 4) return false;
  if (v.v_layout != KVQ_V_TILE32 || v.group_tok % kRTile || v.group_ch < 16) return false;
  if (g < 1 || g > 8) return false;
  if (v.n_quant < kRTile || v.n_quant >= ((int64_t)1 << 26)) return false;  // 32-bit offsets
  return aligned_to(v.v_codes, 16) && v.v_codes_stride % 4 == 0 && aligned_to(v.v_scales, 4);
}

int rope_fast_parts(const kvq_kv_view& v, int Hq, int n_splits) {
  (void)Hq;
  const int64_t tiles = v.n_quant / kRTile;
  int64_t p;
  if (n_splits > 0) {
    p = n_splits;
  } else {
    const int64_t streams = (int64_t)v.batch * v.kv_heads;
    p = (2048 + streams - 1) / streams;          // about 8 workgroups per CU
    const int64_t cap = (tiles + 7) / 8;         // at least 2 tiles per wave
    if (p > cap) p = cap;
  }
  if (p > tiles) p = tiles;
  if (p < 1) p = 1;
  return (int)p;
}

int rope_fp16_parts(const kvq_kv_view& v) {
  const int64_t n = v.n_sink + v.n_tail;
  return n > 0 ? (int)((n + 31) / 32) : 0;
}

hipError_t launch_decode_rope(const kvq_kv_view& v, const void* q, int f16, int Hq,
                              float sm_scale, const RopeDev& rope, float* partials,
                              int n_parts, hipStream_t s) {
  const int64_t ns = v.n_sink, nq = v.n_quant, nf = ns + v.n_tail;
  const int fp = rope_fp16_parts(v);
  const int stride = n_parts + fp;
  const float qscale = sm_scale * kRLog2e;
  int gv_shift = 0;
  while ((1 << gv_shift) < v.group_ch) ++gv_shift;
  hipError_t e;
#define KVQ_ROPE_CASE(KB, VB)                                                               \
  if (v.k_bits == KB && v.v_bits == VB)                                                     \
    e = launch_rope_g<KB, VB>(v, q, f16, Hq, qscale, rope, partials, n_parts, stride, gv_shift, \
                              s);                                                           \
  else
  if (v.k_mixed)
    e = v.v_bits == 4 ? launch_rope_g<0, 4>(v, q, f16, Hq, qscale, rope, partials, n_parts, stride,
                                            gv_shift, s)
                      : launch_rope_g<0, 2>(v, q, f16, Hq, qscale, rope, partials, n_parts, stride,
                                            gv_shift, s);
  else
  KVQ_ROPE_CASE(8, 4) KVQ_ROPE_CASE(8, 2) KVQ_ROPE_CASE(4, 4) KVQ_ROPE_CASE(4, 2)
  KVQ_ROPE_CASE(2, 4) KVQ_ROPE_CASE(2, 2) e = hipErrorInvalidValue;
#undef KVQ_ROPE_CASE
  if (e != hipSuccess || fp == 0) return e;
  // the fp16 sink and tail tokens as one range that skips the quantized
  // ones, 32 tokens per partial
  return launch_decode_generic_range(v, q, f16, Hq, sm_scale, partials, 0, nf, fp, n_parts,
                                     stride, &rope, s, ns, nq);
}

}  // namespace kvq
