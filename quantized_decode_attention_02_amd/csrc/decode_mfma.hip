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
// One workgroup = 4 wavefronts = one (batch, KV head, split).  A split is
// cut into units of up to four 32-token tiles inside one key group; wave w
// takes units w, w+4, ... with its own online-softmax state (Q' is rebuilt
// only when the key group changes), and the four states are merged in LDS
// at the end.  The output is rescaled only when a running max grows.  Lane
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
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kD = 128;
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float h2f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
// The packed cache is read once per call: its loads carry the nontemporal
// hint, which streams them past the caches instead of filling them (a plain
// read of several GiB runs about 13% faster that way on gfx950).
template <typename T>
__device__ inline T ldnt(const T* p) { return __builtin_nontemporal_load(p); }

// v_and_or_b32: (a & mask) | magic in one instruction (the mask travels in
// an SGPR, the magic in a VGPR: gfx9 VOP3 takes no literal and at most one
// scalar operand).
__device__ inline uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(magic));
  return r;
}

// Four fp16 pairs (one MFMA operand) from one 32-bit word of int4 codes:
// pair i holds nibbles (i, 4 + i) of the word times f_i = (1, 16, 1, 16),
// minus the offset 8: the exact values f_i * code.
__device__ inline half8 int4_operand(uint32_t w, uint32_t magic) {
  const uint32_t w8 = w >> 8;
  u32x4 r;
  r[0] = and_or(w, 0x000F000Fu, magic);
  r[1] = and_or(w, 0x00F000F0u, magic);
  r[2] = and_or(w8, 0x000F000Fu, magic);
  r[3] = and_or(w8, 0x00F000F0u, magic);
  half8 h = __builtin_bit_cast(half8, r);
  const half8 off = {(_Float16)1032.0f, (_Float16)1032.0f, (_Float16)1152.0f,
                     (_Float16)1152.0f, (_Float16)1032.0f, (_Float16)1032.0f,
                     (_Float16)1152.0f, (_Float16)1152.0f};
  return h - off;
}

// Four fp16 pairs from 16 bits of int2 codes (the low or high byte pair of
// a word, selected by shifting by 8 first): pair i holds fields (i, 8 + i)
// times 4^i, minus the offset 2.
__device__ inline half8 int2_operand(uint32_t ws, uint32_t magic) {
  u32x4 r;
  r[0] = and_or(ws, 0x00030003u, magic);
  r[1] = and_or(ws, 0x000C000Cu, magic);
  r[2] = and_or(ws, 0x00300030u, magic);
  r[3] = and_or(ws, 0x00C000C0u, magic);
  half8 h = __builtin_bit_cast(half8, r);
  const half8 off = {(_Float16)1026.0f, (_Float16)1026.0f, (_Float16)1032.0f,
                     (_Float16)1032.0f, (_Float16)1056.0f, (_Float16)1056.0f,
                     (_Float16)1152.0f, (_Float16)1152.0f};
  return h - off;
}

// Key operands as fp16 denormals: a field masked in place is the exact fp16
// value f * u * 2^-24 (no implicit leading one, so nothing to subtract per
// code); the code offset is removed once per key group through the MFMA
// accumulator (see k_offset_operand).  The MFMA keeps fp16 denormal inputs
// exact.
__device__ inline half8 int4_key_operand(uint32_t w) {
  const uint32_t w8 = w >> 8;
  u32x4 r;
  r[0] = w & 0x000F000Fu;
  r[1] = w & 0x00F000F0u;
  r[2] = w8 & 0x000F000Fu;
  r[3] = w8 & 0x00F000F0u;
  return __builtin_bit_cast(half8, r);
}
__device__ inline half8 int2_key_operand(uint32_t ws) {
  u32x4 r;
  r[0] = ws & 0x00030003u;
  r[1] = ws & 0x000C000Cu;
  r[2] = ws & 0x00300030u;
  r[3] = ws & 0x00C000C0u;
  return __builtin_bit_cast(half8, r);
}
// The denormal operand of the code offsets (8 for int4, 2 for int2) with
// each slot pair's factor: sum_k off_k * B_k is the group's offset term.
template <int KB>
__device__ inline half8 k_offset_operand() {
  u32x4 r;
  if (KB == 4) {
    r[0] = 0x00080008u; r[1] = 0x00800080u; r[2] = 0x00080008u; r[3] = 0x00800080u;
  } else {
    r[0] = 0x00020002u; r[1] = 0x00080008u; r[2] = 0x00200020u; r[3] = 0x00800080u;
  }
  return __builtin_bit_cast(half8, r);
}

// Local channel (0..31 within the lane group's 32 channels) of k-slot
// pair i, element e, of key MFMA kb.
template <int KB>
__device__ inline int k_slot_channel(int kb, int i, int e) {
  if (KB == 4) return 8 * kb + i + 4 * e;
  return 16 * (kb >> 1) + 4 * (kb & 1) + i + 8 * e;
}
// log2 of the factor carried by slot pair i of an operand of BITS-bit codes.
template <int BITS>
__host__ __device__ constexpr int slot_log2f(int i) {
  return BITS == 4 ? ((i & 1) ? 4 : 0) : 2 * i;
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
  int fp_last;         // grid order: the fp16-row parts after the splits
};

// One-dimensional grid: the short fp16-row parts of every stream first
// (dispatched first, so that none of them trails the long quantized
// splits), then the splits; or, when the workgroups overflow one resident
// round by no more than the fp16-row parts (fp_last), the splits first, so
// that every split starts at once and the short parts take the slots of
// the first splits to finish.  Partial slot = fp16 chunk, or n_fp + split.
struct PartIndex {
  int part, kvh, b;
};
__device__ inline PartIndex part_index(const MfmaArgs& a) {
  // 32-bit arithmetic: the launcher keeps the grid below 2^31 blocks
  const uint32_t L = blockIdx.x;
  const uint32_t n_sp = (uint32_t)a.n_splits, n_fp = (uint32_t)a.n_parts - n_sp;
  const uint32_t streams = (uint32_t)a.v.batch * (uint32_t)a.v.kv_heads;
  const uint32_t first = a.fp_last ? streams * n_sp : streams * n_fp;  // blocks of the first region
  const bool in_first = L < first;
  const bool is_fp = in_first != (bool)a.fp_last;
  const uint32_t idx = in_first ? L : L - first;
  const uint32_t per = is_fp ? n_fp : n_sp;
  const uint32_t s = idx / per;
  const uint32_t r = idx - s * per;
  const uint32_t H = (uint32_t)a.v.kv_heads;
  const uint32_t bb = s / H;
  return PartIndex{(int)(is_fp ? r : n_fp + r), (int)(s - bb * H), (int)bb};
}

// A work unit of one wave: up to 4 tiles (128 tokens) of one key group.
constexpr int kUnitTiles = 4;
constexpr int kRowsPerChunk = 64;  // fp16 sink/tail rows per extra workgroup

// LDS of the matrix-core path and of the fp16-rows path (one buffer).
template <int NC>
struct MainLds {
  float vs[kWaves][kUnitTiles * 32 * NC];
  float ks[kWaves][kD];
  float4v qf[8][64];   // lane l's 32 query values, 4 per entry
  float m[kWaves][16];
  float l[kWaves][16];
  float o[kWaves][16][kD + 1];
};
struct RowsLds {
  uint16_t k[kRowsPerChunk][kD + 8];  // fp16 rows (padded: 16-byte rows, fewer conflicts)
  uint16_t v[kRowsPerChunk][kD + 8];
  float q[16][kD];
  float p[16][kRowsPerChunk];
};
template <int NC>
constexpr size_t lds_bytes() {
  return sizeof(MainLds<NC>) > sizeof(RowsLds) ? sizeof(MainLds<NC>) : sizeof(RowsLds);
}

// fp16 rows (sink rows, then tail rows in token order) chunk `chunk` of one
// (batch, KV head): exact fp32 attention over up to 64 rows; writes one
// partial.  Rows arrive with 16-byte loads; each wave takes 16 rows, a lane
// one row and a quarter of the channels; softmax and the weighted sum of
// the values are spread over the workgroup.
__device__ void fp16_rows_partial(const MfmaArgs& a, int chunk, int part, int kvh, int b,
                                  RowsLds& L) {
  const kvq_kv_view& v = a.v;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = a.Hq / v.kv_heads;
  const int64_t s = (int64_t)b * v.kv_heads + kvh;
  const int64_t nr = v.n_sink + v.n_tail;
  const int r0 = chunk * kRowsPerChunk;
  const int n = (int)min((int64_t)kRowsPerChunk, nr - r0);
  // rows: 16 threads per row, 16 bytes each
  for (int i = tid; i < n * 16; i += kThreads) {
    const int r = i >> 4, c8 = (i & 15) * 8;
    const int64_t j = r0 + r;
    int64_t off;
    const uint16_t *kp, *vp;
    if (j < v.n_sink) {
      off = s * v.sink_stride + j * kD;
      kp = v.sink_k; vp = v.sink_v;
    } else {
      off = s * v.tail_stride + ((v.n_quant + j - v.n_sink) % v.residual) * kD;
      kp = v.tail_k; vp = v.tail_v;
    }
    *(u32x4*)&L.k[r][c8] = *(const u32x4*)(kp + off + c8);
    *(u32x4*)&L.v[r][c8] = *(const u32x4*)(vp + off + c8);
  }
  for (int i = tid; i < g * kD; i += kThreads) {
    const int h = i / kD, d = i % kD;
    const int64_t qi = ((int64_t)b * a.Hq + kvh * g + h) * kD + d;
    L.q[h][d] = (a.q_f16 ? h2f(((const uint16_t*)a.q)[qi]) : ((const float*)a.q)[qi]) * a.qscale;
  }
  __syncthreads();
  // scores: wave w takes rows 16 w .. 16 w + 15; lane (row ln, channel
  // quarter lq) sums 32 channels, then the quarters are added
  {
    const int ln = lane & 15, lq = lane >> 4, r = 16 * wave + ln;
    float kf[32];
    if (r < n) {
#pragma unroll
      for (int c = 0; c < 32; c += 8) {
        const half8 h8 = *(const half8*)&L.k[r][32 * lq + c];
#pragma unroll
        for (int j = 0; j < 8; ++j) kf[c + j] = (float)h8[j];
      }
    }
    for (int h = 0; h < g; ++h) {
      float acc = 0.0f;
      if (r < n) {
#pragma unroll
        for (int c = 0; c < 32; c += 4) {
          const float4v q4 = *(const float4v*)&L.q[h][32 * lq + c];
          acc = __builtin_fmaf(q4[0], kf[c], acc);
          acc = __builtin_fmaf(q4[1], kf[c + 1], acc);
          acc = __builtin_fmaf(q4[2], kf[c + 2], acc);
          acc = __builtin_fmaf(q4[3], kf[c + 3], acc);
        }
      }
      acc += __shfl_xor(acc, 16);
      acc += __shfl_xor(acc, 32);
      if (lq == 0 && r < n) L.p[h][r] = acc;
    }
  }
  __syncthreads();
  float* out = a.partials + (((int64_t)b * a.Hq + kvh * g) * a.n_parts + part) * (kD + 2);
  const int64_t hstride = (int64_t)a.n_parts * (kD + 2);
  // softmax per head: wave w takes heads w, w + 4, ...; lane = row
  for (int h = wave; h < g; h += kWaves) {
    const float x = lane < n ? L.p[h][lane] : -INFINITY;
    float m = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float e = lane < n ? exp2f(x - m) : 0.0f;
    float l = e;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) l += __shfl_xor(l, o);
    if (lane < n) L.p[h][lane] = e;
    if (lane == 0) {
      out[h * hstride] = m;
      out[h * hstride + 1] = l;
    }
  }
  __syncthreads();
  // weighted sum of the value rows: thread (head, channel pair)
  for (int i = tid; i < g * (kD / 2); i += kThreads) {
    const int h = i / (kD / 2), d2 = 2 * (i % (kD / 2));
    float o0 = 0.0f, o1 = 0.0f;
    for (int r = 0; r < n; ++r) {
      const float pr = L.p[h][r];
      const uint32_t w = *(const uint32_t*)&L.v[r][d2];
      o0 = __builtin_fmaf(pr, h2f((uint16_t)(w & 0xFFFF)), o0);
      o1 = __builtin_fmaf(pr, h2f((uint16_t)(w >> 16)), o1);
    }
    out[h * hstride + 2 + d2] = o0;
    out[h * hstride + 3 + d2] = o1;
  }
}

template <int CTRL>
__device__ inline float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// Max / sum over the 16 lanes of a row (row_ror 8, 4, 2, 1).  The max is
// one v_max_f32 with a DPP source per step (the builtin form adds a copy
// and a canonicalizing max); the s_nop covers the VALU-write-to-DPP-read
// wait states.
template <int ROR>
__device__ inline float max_ror(float x) {
  float r;
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_ror:%2 row_mask:0xf bank_mask:0xf"
      : "=v"(r)
      : "v"(x), "i"(ROR));
  return r;
}
__device__ inline float row_max16(float x) {
  return max_ror<1>(max_ror<2>(max_ror<4>(max_ror<8>(x))));
}
// Largest of a scale row held as float4s by lanes 0-31 (lanes 32-63 hold
// zeros; scales are >= 0).
__device__ inline float row_max_lanes32(float4v x) {
  const float m = row_max16(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  return fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m), 0)),
               __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m), 16)));
}
__device__ inline float row_sum16(float x) {
  x += dpp_f<0x128>(x);
  x += dpp_f<0x124>(x);
  x += dpp_f<0x122>(x);
  x += dpp_f<0x121>(x);
  return x;
}

// Lazy softmax rescale.  The running maximum m moves only when a tile's
// largest score exceeds it by more than kLazy (log2 units), so most tiles
// skip the rescale of the output accumulators; p = 2^(s - m) is then at
// most 2^kLazy.  The result is the same function of (m, l, o): every
// partial is exact with respect to the m it reports.
constexpr int kLazy = 3;
// Value prescale.  P' = p * v_scale / f is rounded to one fp16 number, so
// a unit's value scales are multiplied by a power of two
// sigma_v = 2^(14 - kLazy - e) before P' is formed, e being the exponent of
// a recent unit's largest value scale: the largest scale times sigma_v
// stays in [2^(8 - kLazy), 2^(15 - kLazy)), which keeps P' (p <= 2^kLazy)
// below the fp16 maximum and, down to p * v_scale / v_max = 2^(kLazy - 16),
// in the normal range (relative rounding 2^-11).  The output accumulators
// carry the same factor: when a unit's scales leave that window, e moves to
// the unit's exponent and the accumulators are multiplied by the (exact)
// power of two between the two factors; at the end they are divided by
// sigma_v.
constexpr int kVTop = 14 - kLazy;
// Exponent of the largest of the n value scales a wave holds (float4 j of
// lane l is scale group l + 64 j); the result is wave-uniform.
template <int K>
__device__ inline int unit_vscale_exp(const float4v (&vsn)[K], int lane, int n) {
  float mx = 0.0f;
#pragma unroll
  for (int j = 0; j < K; ++j)
    if (lane + 64 * j < n)
      mx = fmaxf(mx, fmaxf(fmaxf(vsn[j][0], vsn[j][1]), fmaxf(vsn[j][2], vsn[j][3])));
  mx = row_max16(mx);
  const uint32_t b = __builtin_bit_cast(uint32_t, mx);
  const uint32_t r0 = __builtin_amdgcn_readlane(b, 0), r1 = __builtin_amdgcn_readlane(b, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(b, 32), r3 = __builtin_amdgcn_readlane(b, 48);
  const uint32_t m = max(max(r0, r1), max(r2, r3));  // positive floats order as integers
  int e = (int)(m >> 23) - 127;
  return e < -100 ? -100 : e;
}
__device__ inline float pow2f(int k) { return __builtin_bit_cast(float, (uint32_t)(127 + k) << 23); }

// Value of the next lane of the 16-lane row (DPP row_shl:1); lane 15 gets 0.
__device__ inline float from_next_lane(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x101, 0xF, 0xF, false));
}

// PACKED (2 * g * NC <= 16): MFMA column n = 2 * (h * NC + c) + part.  On the
// key side column n carries the high (part 0) or low (part 1) fp16 limb of
// Q'_h, so one MFMA gives both limbs and a row shift adds them; on the value
// side the even columns carry P'_h for value-channel group c.  Otherwise
// column n is query head n, with separate high/low MFMAs and every value
// group's P' built in every lane.
template <int KB, int VB, int NC, bool PACKED>
__global__ void __launch_bounds__(kThreads, (PACKED && NC <= 4 && !(KB == 4 && VB == 4)) ? 3 : 2)
decode_mfma_kernel(MfmaArgs a) {
  __shared__ __align__(16) unsigned char lds_raw[lds_bytes<NC>()];
  const PartIndex pi = part_index(a);
  const int slot = pi.part, kvh = pi.kvh, b = pi.b;
  const int n_fp = a.n_parts - a.n_splits;
  if (slot < n_fp) {
    fp16_rows_partial(a, slot, slot, kvh, b, *(RowsLds*)lds_raw);
    return;
  }
  const int split = slot - n_fp;
  MainLds<NC>& S = *(MainLds<NC>*)lds_raw;
  auto& sm_vs = S.vs;
  auto& sm_qf = S.qf;
  auto& sm_m = S.m;
  auto& sm_l = S.l;
  auto& sm_o = S.o;

  const kvq_kv_view& v = a.v;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lq = lane >> 4, ln = lane & 15;
  const int g = a.Hq / v.kv_heads;
  const int64_t s = (int64_t)b * v.kv_heads + kvh;
  // this lane's column: query head hh, value group cc, limb part
  const int hh = PACKED ? (ln >> 1) / NC : ln;
  const int cc = PACKED ? (ln >> 1) % NC : 0;
  const int part = PACKED ? (ln & 1) : 0;
  const bool head_ok = hh < g;
  const bool col_valid = head_ok && part == 0;  // value-side column in use
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(magic));  // keep the fp16 magic in a VGPR

  const int tpg = v.group_tok / 32;                 // tiles per key group
  const int ut = tpg < kUnitTiles ? tpg : kUnitTiles;  // tiles per unit
  const int upg = tpg / ut;                         // units per group
  const int n_units = (int)(v.n_quant / (32 * ut));
  // units split as evenly as possible over the splits
  const int u_lo = (int)((int64_t)split * n_units / a.n_splits);
  const int u_hi = (int)((int64_t)(split + 1) * n_units / a.n_splits);

  // This lane's query values on its key MFMA k-slots, times the inverse of
  // each slot's factor, sm_scale * log2(e) and a power of two sigma_q that
  // brings them below 2 in magnitude: qf[kb][2i + e], kept in LDS (every
  // wave uses the same values; wave 0 writes them).  Each key group's scale
  // row is multiplied by its own power of two sigma_g (largest scale below
  // 2^13) when it is committed to LDS, so |Q'| < 2^14 stays in fp16 range.
  float inv_sigma_q;
  {
    float qv[32];
    const int64_t base = ((int64_t)b * a.Hq + kvh * g + (head_ok ? hh : 0)) * kD + 32 * lq;
    if (a.q_f16) {
#pragma unroll
      for (int c = 0; c < 32; c += 8) {
        const half8 h8 = *(const half8*)((const uint16_t*)a.q + base + c);
#pragma unroll
        for (int j = 0; j < 8; ++j) qv[c + j] = (float)h8[j];
      }
    } else {
#pragma unroll
      for (int c = 0; c < 32; c += 4) {
        const float4v f4 = *(const float4v*)((const float*)a.q + base + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) qv[c + j] = f4[j];
      }
    }
    float qabs = 0.0f;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      qv[c] = head_ok ? qv[c] * a.qscale : 0.0f;
      qabs = fmaxf(qabs, fabsf(qv[c]));
    }
    qabs = fmaxf(qabs, __shfl_xor(qabs, 16));
    qabs = fmaxf(qabs, __shfl_xor(qabs, 32));
    int ex = (int)((__builtin_bit_cast(uint32_t, qabs) >> 23) & 0xFF) - 127;
    ex = ex < -100 ? -100 : ex;
    const float sigma_q = __builtin_bit_cast(float, (uint32_t)(127 - ex) << 23);
    inv_sigma_q = __builtin_bit_cast(float, (uint32_t)(127 + ex) << 23);
    if (wave == 0) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float qf[8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 2; ++e)
            qf[2 * i + e] = qv[k_slot_channel<KB>(kb, i, e)] * sigma_q *
                            (1.0f / (float)(1 << slot_log2f<KB>(i)));
        sm_qf[2 * kb][lane] = (float4v){qf[0], qf[1], qf[2], qf[3]};
        sm_qf[2 * kb + 1][lane] = (float4v){qf[4], qf[5], qf[6], qf[7]};
      }
    }
  }
  __syncthreads();

  const uint32_t* kc = v.k_codes + s * v.k_codes_stride;
  const float* ks = v.k_scales + s * v.k_scales_stride;
  const uint32_t* vc = v.v_codes + s * v.v_codes_stride;
  const float* vs = v.v_scales + s * v.v_scales_stride;
  float* my_vs = sm_vs[wave];

  half8 qhi[4], qlo[PACKED ? 1 : 4];
  float4v negcorr_hi, negcorr_lo;  // minus the group's offset terms
  int cur_group = -1;
  float inv_sigma_k = 0.0f;  // undoes sigma_q * sigma_g and the 2^-24

  float m_run = -INFINITY, l_run = 0.0f;
  float4v o[8];
#pragma unroll
  for (int jb = 0; jb < 8; ++jb) o[jb] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

  // Rolling prefetch: the codes of tile i of the wave's next unit are loaded
  // into tile i's registers as soon as tile i of the current unit is done;
  // the next unit's value scales and key-scale row wait in registers and are
  // committed to this wave's LDS slice at the unit boundary.
  constexpr int kVs4 = (kUnitTiles * 32 * NC / 4 + 63) / 64;  // float4 per lane
  const int n_vs4 = ut * 32 * NC / 4;
  u32x4 kw[kUnitTiles][2];
  u32x4 vw[kUnitTiles][VB == 4 ? 2 : 1];
  float4v vsn[kVs4];
  float4v ksn = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
  auto load_tile = [&](int unit, int i) {
    const int64_t t32 = (int64_t)(unit * ut + i) * 32;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t tok = t32 + 16 * h + ln;
      if (KB == 4) {
        kw[i][h] = ldnt((const u32x4*)(kc + tok * 16 + 4 * lq));
      } else {
        const u32x2 w2 = ldnt((const u32x2*)(kc + tok * 8 + 2 * lq));
        kw[i][h] = (u32x4){w2[0], w2[1], 0u, 0u};
      }
    }
    const int64_t tw = (int64_t)(unit * ut + i) * (32 * VB * kD / 32);
    vw[i][0] = ldnt((const u32x4*)(vc + tw + lane * 4));
    if (VB == 4) vw[i][VB == 4 ? 1 : 0] = ldnt((const u32x4*)(vc + tw + 256 + lane * 4));
  };
  auto load_scales = [&](int unit) {
    const float4v* src = (const float4v*)(vs + (int64_t)unit * ut * 32 * NC);
#pragma unroll
    for (int j = 0; j < kVs4; ++j) {
      const int idx = lane + 64 * j;
      if (idx < n_vs4) vsn[j] = ldnt(src + idx);
    }
    // (the group's largest scale is taken from this row when it is
    // committed: a separate uniform load of it would be moved to a scalar
    // register at once, and that move waits for every load in flight, the
    // prefetched tiles included)
    if (lane < kD / 4) ksn = ((const float4v*)(ks + (int64_t)(unit / upg) * kD))[lane];
  };
  float* my_ks = S.ks[wave];
  const int u_first = u_lo + wave;
  if (u_first < u_hi) {
    // scales first, then the tiles: the order of the loop's own requests
    load_scales(u_first);
#pragma unroll
    for (int i = 0; i < kUnitTiles; ++i)
      if (i < ut) load_tile(u_first, i);
  }

  int ev = 0;            // sigma_v = 2^(kVTop - ev) (see unit_vscale_exp)
  bool ev_set = false;
  for (int u = u_first; u < u_hi; u += kWaves) {
    const int grp = u / upg;
    // ---- commit this unit's scales to LDS (times sigma_v), then fetch the
    //      next unit's
    {
      const int e = unit_vscale_exp(vsn, lane, n_vs4);
      if (!ev_set || e > ev || e < ev - 6) {
        if (ev_set) {
          const float r = pow2f(ev - e);
#pragma unroll
          for (int jb = 0; jb < 8; ++jb) o[jb] *= r;
        }
        ev = e;
        ev_set = true;
      }
    }
    const float sig_v = pow2f(kVTop - ev);
#pragma unroll
    for (int j = 0; j < kVs4; ++j) {
      const int idx = lane + 64 * j;
      if (idx < n_vs4) ((float4v*)my_vs)[idx] = vsn[j] * sig_v;
    }
    // sigma_g: power of two bringing the group's largest scale below 2^13
    // (the group's largest scale, from the scale row itself)
    const float kgv = row_max_lanes32(ksn);
    int exg = (int)((__builtin_bit_cast(uint32_t, kgv) >> 23) & 0xFF) - 127;
    exg = exg < -100 ? -100 : exg;
    const float sigma_g = __builtin_bit_cast(float, (uint32_t)(127 + 12 - exg) << 23);
    const float inv_sigma_g = __builtin_bit_cast(float, (uint32_t)(127 - 12 + exg) << 23);
    if (lane < kD / 4) ((float4v*)my_ks)[lane] = ksn * sigma_g;
    __builtin_amdgcn_wave_barrier();
    const int un = u + kWaves;
    const bool has_next = un < u_hi;
    if (has_next) load_scales(un);
    if (grp != cur_group) {
      cur_group = grp;
      inv_sigma_k = inv_sigma_q * inv_sigma_g * 16777216.0f;
      const float* kss = my_ks + 32 * lq;
      float ksv[32];
#pragma unroll
      for (int c = 0; c < 32; c += 4) {
        const float4v t4 = *(const float4v*)(kss + c);
        ksv[c] = t4[0]; ksv[c + 1] = t4[1]; ksv[c + 2] = t4[2]; ksv[c + 3] = t4[3];
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float4v q0 = sm_qf[2 * kb][lane], q1 = sm_qf[2 * kb + 1][lane];
        const float qk[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float x = qk[2 * i + e] * ksv[k_slot_channel<KB>(kb, i, e)];
            const _Float16 hi = (_Float16)x;
            const _Float16 lo = (_Float16)(x - (float)hi);
            if (PACKED) {
              qhi[kb][2 * i + e] = part ? lo : hi;
            } else {
              qhi[kb][2 * i + e] = hi;
              qlo[PACKED ? 0 : kb][2 * i + e] = lo;
            }
          }
      }
      const half8 aoff = k_offset_operand<KB>();
      float4v c_hi = (float4v){0.0f, 0.0f, 0.0f, 0.0f}, c_lo = c_hi;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        c_hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(aoff, qhi[kb], c_hi, 0, 0, 0);
        if (!PACKED)
          c_lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(aoff, qlo[PACKED ? 0 : kb], c_lo, 0, 0, 0);
      }
      negcorr_hi = -c_hi;
      negcorr_lo = -c_lo;
    }
    __builtin_amdgcn_wave_barrier();

#pragma unroll
    for (int i = 0; i < kUnitTiles; ++i) {
      if (i >= ut) break;
      // ---- scores of the tile's 32 tokens (two 16-token halves)
      float4v acc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float4v acc_lo = negcorr_lo;
        acc[h] = negcorr_hi;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          half8 A;
          if (KB == 4) {
            A = int4_key_operand(kw[i][h][kb]);
          } else {
            const uint32_t word = kw[i][h][kb >> 1];
            A = int2_key_operand((kb & 1) ? (word >> 8) : word);
          }
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qhi[kb], acc[h], 0, 0, 0);
          if (!PACKED)
            acc_lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qlo[PACKED ? 0 : kb], acc_lo, 0, 0, 0);
        }
        if (PACKED) {
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[h][j] += from_next_lane(acc[h][j]);
        } else {
          acc[h] += acc_lo;
        }
      }
      // ---- online softmax; slot sl = 4h + j of this lane is token
      //      j + 4*lq + 16*h of the tile, query head hh
      float amax = fmaxf(fmaxf(fmaxf(acc[0][0], acc[0][1]), fmaxf(acc[0][2], acc[0][3])),
                         fmaxf(fmaxf(acc[1][0], acc[1][1]), fmaxf(acc[1][2], acc[1][3])));
      float tmax = amax * inv_sigma_k;
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      if (__any(tmax > m_run + (float)kLazy)) {
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) o[jb] *= alpha;
      }
      // p / f(slot pair) for the value operand (0 in unused columns); psum of
      // the unscaled p
      const float neg_m = (PACKED && !col_valid) ? -INFINITY : -m_run;
      float p[8];
      float psum = 0.0f;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) {
        const int lf = slot_log2f<VB>(sl >> 1);
        p[sl] = __builtin_amdgcn_exp2f(
            __builtin_fmaf(acc[sl >> 2][sl & 3], inv_sigma_k, neg_m - (float)lf));
        psum = __builtin_fmaf(p[sl], (float)(1 << lf), psum);
      }
      l_run += psum;
      // ---- P' operands and the value MFMAs
      if (PACKED) {
        half8 pb;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int tau = (sl & 3) + 4 * lq + 16 * (sl >> 2);
          pb[sl] = (_Float16)(p[sl] * my_vs[(i * 32 + tau) * NC + cc]);
        }
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) {
          half8 A;
          if (VB == 2) {
            const uint32_t word = vw[i][0][jb >> 1];
            A = int2_operand((jb & 1) ? (word >> 8) : word, magic);
          } else {
            A = int4_operand(vw[i][jb >> 2][jb & 3], magic);
          }
          o[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, pb, o[jb], 0, 0, 0);
        }
      } else {
        half8 pb[NC];
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const int tau = (sl & 3) + 4 * lq + 16 * (sl >> 2);
          const float* row = my_vs + (i * 32 + tau) * NC;
#pragma unroll
          for (int c = 0; c < NC; ++c) pb[c][sl] = (_Float16)(p[sl] * row[c]);
        }
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) {
          half8 A;
          if (VB == 2) {
            const uint32_t word = vw[i][0][jb >> 1];
            A = int2_operand((jb & 1) ? (word >> 8) : word, magic);
          } else {
            A = int4_operand(vw[i][jb >> 2][jb & 3], magic);
          }
          o[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, pb[(jb * 16 * NC) / kD], o[jb], 0,
                                                         0, 0);
        }
      }
      if (has_next) load_tile(un, i);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- per-wave state to LDS: m, l (summed over the 4 lane groups), O
  //      (divided by sigma_v)
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (ev_set) {
    const float r = pow2f(ev - kVTop);
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) o[jb] *= r;
  }
  if (PACKED) {
    if (lq == 0 && col_valid && cc == 0) {
      sm_m[wave][hh] = m_run;
      sm_l[wave][hh] = l_run;
    }
    if (col_valid) {
#pragma unroll
      for (int jb = 0; jb < 8; ++jb)
        if ((jb * 16 * NC) / kD == cc)
#pragma unroll
          for (int j = 0; j < 4; ++j) sm_o[wave][hh][16 * jb + 4 * lq + j] = o[jb][j];
    }
  } else {
    if (lq == 0) {
      sm_m[wave][ln] = m_run;
      sm_l[wave][ln] = l_run;
    }
#pragma unroll
    for (int jb = 0; jb < 8; ++jb)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm_o[wave][ln][16 * jb + 4 * lq + j] = o[jb][j];
  }
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
    a.partials[(((int64_t)b * a.Hq + kvh * g + h) * a.n_parts + slot) * (kD + 2) + jx] = val;
  }
}

// ---------------------------------------------------------------------------
// Row-score kernel: up to 8 query heads per KV head and g * NC <= 16.
//
// The scores are computed transposed, S[row][token] = Q'[row] . code[token],
// with the rows of Q' (head, limb) as the MFMA A operand and the key codes
// as B.  Lane 16r + t then holds, for token t of each 16-token half, the
// high and low limb sums of the two heads of row group r, so every lane
// owns whole scores of distinct tokens and the softmax costs one exp per
// (head, token) and lane group instead of one per MFMA output column.  Row
// groups that would hold the same heads (g <= 4) split the value groups
// between them.  The fp16 P' values go through a per-wave LDS buffer into
// the value MFMA's B layout, whose columns are (head, value group).
//
// Value operands are exact centred fp16 codes (AND-OR with the pattern of
// 1024, packed subtract).  Removing the value offset through an extra MFMA
// against a constant operand, as on the key side, is not used here: the
// offset term has the same sign for every token and the MFMA accumulation
// does not round it away without bias over thousands of tiles.
constexpr int kPlStride = 40;  // halves per P' row: 32 + 8 against bank conflicts

// Requests of the row-score kernel past the wave's last unit read this block
// of zeros (8 KB: the largest span a request's lane offsets cover is a
// unit's value scales, 4 KB).  Every path then issues the same requests, so
// the compiler's wait counts stay exact (a skipped request makes it fall
// back to waiting for every load in flight at each unit start), and the
// block stays in cache.  (Not const: the compiler would fold loads from a
// known-zero array away and bring the skipped requests back.  Nothing
// writes it; a device variable starts zeroed.)
__device__ __align__(16) uint32_t kPastZeros[2048];

template <int NC, bool KM, int QR>
struct RsLds {
  float vs[kWaves][kUnitTiles * 32 * NC];
  float ks[kWaves][kD];
  // lane l's query values at column l + l / 16: the Q' build reads one
  // column of each lane group per lane, and the padding puts the four lane
  // groups in distinct banks
  float4v qf[8][64 + 4];
  // mixed keys: q * sm_scale * log2(e) * sigma_q by channel; rows padded
  // to 132 floats so that the heads of one channel fall in distinct banks
  // (the Q' gather reads one channel of up to eight heads per instruction)
  float qs[KM ? 8 : 1][kD + 4];
  uint16_t inv[kWaves][KM ? kD + 8 : 8];  // mixed keys: 4 x channel of each slot, then bf16 ones
  float m[kWaves][8];
  float l[kWaves][8];
  union alignas(16) {
    float o[kWaves][8][kD + 1];
    struct {
      _Float16 pl[kWaves][16][kPlStride];
      // uniform keys: each wave's Q' limbs in the A layout, by key MFMA,
      // lane group and distinct row (2 head + limb; QR rows), four words
      // of fp16 pairs per entry; 16 rows are padded to 17 so that the four
      // lane groups' stores fall in distinct banks
      u32x4 qp[KM ? 1 : kWaves][4][4][KM ? 1 : (QR == 16 ? 17 : QR)];
    } t;
  } u;
};
template <int NC, bool KM, int QR>
constexpr size_t rs_lds_bytes() {
  return sizeof(RsLds<NC, KM, QR>) > sizeof(RowsLds) ? sizeof(RsLds<NC, KM, QR>) : sizeof(RowsLds);
}

// KB: uniform key bits (4 or 2), or 0 for mixed keys (bf16 / int4 / int2
// channels per group, the MixKVQ layout).  HS: head slots per score lane
// (1 when g == 1, else 2).  Three waves per SIMD (168 registers) where the
// variant fits without spilling, else two.
template <int KB, int VB, int NC, int HS>
constexpr int rs_waves() {
  return (KB == 0 || (KB == 4 && VB == 4) || NC == 8 ||
          (NC == 4 && (KB == 4 || VB == 4) && !(KB == 2 && HS == 1)))
             ? 2
             : 3;
}
template <int KB, int VB, int NC, int HS, int UT>
__global__ void __launch_bounds__(kThreads, (rs_waves<KB, VB, NC, HS>())) decode_rs_kernel(MfmaArgs a) {
  constexpr bool KM = KB == 0;  // mixed-precision keys
  constexpr int QR = HS == 1 ? 2 : 16;  // distinct Q' rows (head, limb)
  __shared__ __align__(16) unsigned char lds_raw[rs_lds_bytes<NC, KM, QR>()];
  const PartIndex pi = part_index(a);
  const int part = pi.part, kvh = pi.kvh, b = pi.b;
  const int n_fp = a.n_parts - a.n_splits;
  if (part < n_fp) {
    fp16_rows_partial(a, part, part, kvh, b, *(RowsLds*)lds_raw);
    return;
  }
  const int split = part - n_fp;
  RsLds<NC, KM, QR>& S = *(RsLds<NC, KM, QR>*)lds_raw;
  const kvq_kv_view& v = a.v;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lq = lane >> 4, ln = lane & 15;
  const int g = a.Hq / v.kv_heads;
  const int64_t s = (int64_t)b * v.kv_heads + kvh;
  // row groups with distinct heads; each is repeated rep times
  const int rgd = HS == 1 ? 1 : (g <= 2 ? 1 : (g <= 4 ? 2 : 4));
  const int rep = HS == 1 ? 4 : 4 / rgd;
  // A layout: Q' row ln = 4r + 2hl + limb is head 2(r mod rgd) + hl
  const int a_head = HS == 1 ? 0 : 2 * ((ln >> 2) % rgd) + ((ln >> 1) & 1);
  const int limb = ln & 1;
  // score layout: lane holds rows 4lq .. 4lq + 3 of token ln of each half
  int s_head[HS];
#pragma unroll
  for (int hl = 0; hl < HS; ++hl) s_head[hl] = HS == 1 ? 0 : 2 * (lq % rgd) + hl;
  const int rep_idx = lq / rgd;
  // value layout: column ln = head * NC + value group
  const int v_head = ln / NC, v_cc = ln % NC;
  const bool v_valid = v_head < g;

  const int tpg = v.group_tok / 32;                    // tiles per key group
  constexpr int ut = UT;                               // tiles per unit
  const int upg = tpg / ut;                            // units per group
  const int n_units = (int)(v.n_quant / (32 * ut));
  // units split as evenly as possible over the splits
  const int u_lo = (int)((int64_t)split * n_units / a.n_splits);
  const int u_hi = (int)((int64_t)(split + 1) * n_units / a.n_splits);
  const float* kg = v.k_gmax + s * v.k_gmax_stride;

  const uint32_t* kc = v.k_codes + s * v.k_codes_stride;
  const float* ks = v.k_scales + s * v.k_scales_stride;
  const uint32_t* vc = v.v_codes + s * v.v_codes_stride;
  const float* vs = v.v_scales + s * v.v_scales_stride;
  float* my_vs = S.vs[wave];
  float* my_ks = S.ks[wave];
  _Float16(*my_pl)[kPlStride] = S.u.t.pl[wave];
  // mixed keys: class sizes, packed row words, and the MFMA blocks (the
  // first n4b take int4 positions, the rest int2 positions, 32 each)
  const int NB = KM ? v.n_bf16 : 0, N4 = KM ? v.n_int4 : 0, N2 = kD - NB - N4;
  const int w4 = (N4 + 7) / 8, w2 = (N2 + 15) / 16;
  const int n4b = (N4 + 31) / 32;
  const int ksrow = KM ? kD - NB : kD;  // key scales per group
  const uint32_t* k4p = KM ? v.k_int4 + s * v.k_int4_stride : nullptr;
  const uint32_t* k2p = KM ? v.k_int2 + s * v.k_int2_stride : nullptr;
  const uint16_t* kbp = KM ? v.k_bf16 + s * v.k_bf16_stride : nullptr;
  const uint8_t* kpp = KM ? v.k_pos + s * v.k_pos_stride : nullptr;
  uint16_t* my_inv = S.inv[wave];
  // mixed keys, per MFMA block kb: row array, row words and this lane's
  // word (clamped into the row: a padding slot's code is never used, its
  // scale is zero); int2 words are shifted so the lane's 8 fields sit in
  // the low bytes
  const uint32_t* kbase[4];
  int kstride[4], kwi[4], kshift[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const bool b4 = kb < n4b;
    kbase[kb] = b4 ? k4p : k2p;
    kstride[kb] = b4 ? w4 : w2;
    const int wi = b4 ? 4 * kb + lq : 2 * (kb - n4b) + (lq >> 1);
    const int wmax = (b4 ? w4 : w2) - 1;
    kwi[kb] = wi < wmax ? wi : (wmax > 0 ? wmax : 0);
    kshift[kb] = b4 ? 0 : 8 * (lq & 1);
  }
  if (KM) {
    // padding slots of the scale row stay zero; unused map entries name
    // channel 0
    const bool pad = (lane >= N4 / 4 && lane < 8 * n4b) || lane >= 8 * n4b + N2 / 4;
    if (lane < kD / 4 && pad) ((float4v*)my_ks)[lane] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = lane; j < kD + 8; j += 64) my_inv[j] = 0;  // channel 0
  }

  half8 qa[4];              // Q' rows (A operand), one limb per lane
  float4v negc;             // minus the group's offset terms, per row
  float isk = 0.0f;         // undoes sigma_q * sigma_g and the 2^-24

  // online softmax state per head slot (score layout)
  float m_run[HS], l_part[HS], cm[2][HS];
  // value-operand slot factor of token 16 h16 + ln: k-slot pair
  // ((ln & 3) >> 1) + 2 h16
  const int lf0 = slot_log2f<VB>((ln & 3) >> 1), lf1 = slot_log2f<VB>(((ln & 3) >> 1) + 2);
  const float f0 = (float)(1 << lf0), f1 = (float)(1 << lf1);
#pragma unroll
  for (int hl = 0; hl < HS; ++hl) {
    m_run[hl] = -INFINITY;
    l_part[hl] = 0.0f;
    cm[0][hl] = -INFINITY;
    cm[1][hl] = -INFINITY;
  }
  // P' buffer position of token 16 h16 + ln in its column (+ 4 h16)
  const int kpos = 8 * (ln >> 2) + (ln & 3);
  const int niter = (NC + rep - 1) / rep;  // value groups per score lane

  float4v o[8];
#pragma unroll
  for (int jb = 0; jb < 8; ++jb) o[jb] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(magic));  // keep the fp16 magic in a VGPR

  int ev = 0;            // sigma_v = 2^(kVTop - ev) (see unit_vscale_exp)
  bool ev_set = false;

  // Rolling prefetch (as in the column kernel above).  The first unit is
  // requested before the query prologue so the two latencies overlap.
  constexpr int kVs4 = (UT * 32 * NC / 4 + 63) / 64;
  constexpr int n_vs4 = UT * 32 * NC / 4;
  // code slots: a whole unit (tile i in slot i), or for mixed keys two
  // (tile i in slot i % 2, refilled with the tile two places later)
  constexpr int kSlots = KM ? 2 : kUnitTiles;
  u32x4 kw[kSlots][2];
  u32x4 vw[kSlots][VB == 4 ? 2 : 1];
  // mixed keys: the token's bf16 channels (0-3 and 4-7, each loaded on
  // its own into its own registers)
  u32x2 kb16lo[KM ? kSlots : 1][2], kb16hi[KM ? kSlots : 1][2];
  float4v vsn[kVs4];
  float4v ksn = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
  float kgn = 0.0f;
  uint32_t kpn = 0;  // mixed keys: class positions of channels 2 lane, 2 lane + 1
  // (a unit past the wave's last reads kPastZeros at the same lane offsets;
  // for mixed keys, whose many arrays would each need that choice, it reads
  // the split's last unit again, which its own wave reads at about the
  // same time)
  const int u_again = u_hi > 0 ? u_hi - 1 : 0;
  auto load_tile = [&](int unit, int i, int slot) {
    const bool past = unit >= u_hi;
    const int64_t t32 = (int64_t)((KM && past ? u_again : unit) * ut + i) * 32;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 16 * h + ln;  // token of the tile
      if (KM) {
        // word of MFMA block kb: int4 word 4 kb + lq, or int2 word
        // 2 (kb - n4b) + lq / 2
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          kw[slot][h][kb] = ldnt(&kbase[kb][(t32 + r) * kstride[kb] + kwi[kb]]);
        // (the class sizes act as lane conditions, so every path issues
        // the same requests and the compiler's wait counts stay exact)
        int nbv = NB;
        asm volatile("" : "+v"(nbv));
        const uint16_t* bb = kbp + (t32 + r) * nbv;
        u32x2 lo = {0u, 0u}, hi = {0u, 0u};
        if (nbv >= 4) lo = ldnt((const u32x2*)bb);
        if (nbv == 8) hi = ldnt((const u32x2*)(bb + 4));
        kb16lo[KM ? slot : 0][h] = lo;
        kb16hi[KM ? slot : 0][h] = hi;
      } else if (KB == 4) {
        const uint32_t* b = past ? kPastZeros : kc + t32 * 16;
        kw[slot][h] = ldnt((const u32x4*)(b + r * 16 + 4 * lq));
      } else {
        const uint32_t* b = past ? kPastZeros : kc + t32 * 8;
        const u32x2 w2 = ldnt((const u32x2*)(b + r * 8 + 2 * lq));
        kw[slot][h] = (u32x4){w2[0], w2[1], 0u, 0u};
      }
    }
    const uint32_t* vb = (!KM && past) ? kPastZeros : vc + t32 * (VB * kD / 32);
    vw[slot][0] = ldnt((const u32x4*)(vb + lane * 4));
    if (VB == 4) vw[slot][VB == 4 ? 1 : 0] = ldnt((const u32x4*)(vb + 256 + lane * 4));
  };
  auto load_scales = [&](int unit) {
    const bool past = !KM && unit >= u_hi;
    if (KM && unit >= u_hi) unit = u_again;
    const float4v* src =
        (const float4v*)(past ? (const float*)kPastZeros : vs + (int64_t)unit * ut * 32 * NC);
#pragma unroll
    for (int j = 0; j < kVs4; ++j) {
      const int idx = lane + 64 * j;
      if (idx < n_vs4) vsn[j] = ldnt(src + idx);
    }
    const float* ksr = past ? (const float*)kPastZeros : ks + (int64_t)(unit / upg) * ksrow;
    if (lane < ksrow / 4) ksn = ((const float4v*)ksr)[lane];
    // (uniform keys take the group's largest scale from the scale row
    // itself when it is committed: a separate uniform load of it would be
    // moved to a scalar register at once, and that move waits for every
    // load in flight, the prefetched tiles included)
    if (KM) {
      // (a lane-varying index keeps this one in a vector register)
      int gi = unit / upg;
      asm volatile("" : "+v"(gi));
      kgn = kg[gi];
      kpn = ((const uint16_t*)(kpp + (int64_t)(unit / upg) * kD))[lane];
    }
  };
  // A step of the wave covers kStep tiles: one unit, or kStep / ut units
  // (u, u + 4, ...) when units are shorter than the slot ring, so the code
  // prefetch always runs kSlots tiles ahead; tile i of a step is tile
  // i % ut of unit u + 4 (i / ut) and lives in slot i % kSlots.
  constexpr int kStep = kSlots > ut ? kSlots : ut;
  constexpr int ups = kStep / ut;  // units per step
  const int u_first = u_lo + wave;
  // Request order: the query, the first unit's scales, then its codes.
  // Loads complete in order, so the query prologue waits only for the
  // query and the first tile only for the scales and itself, not for the
  // whole prefetch burst.
  const bool q_ok = a_head < g;
  u32x4 qraw[8];
  {
    const int64_t base = ((int64_t)b * a.Hq + kvh * g + (q_ok ? a_head : 0)) * kD + 32 * lq;
    if (a.q_f16) {
#pragma unroll
      for (int c = 0; c < 4; ++c) qraw[c] = *(const u32x4*)((const uint16_t*)a.q + base + 8 * c);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) qraw[c] = *(const u32x4*)((const float*)a.q + base + 4 * c);
    }
  }
  // Every request is issued on every path (past the wave's last unit, or
  // for a wave without units, it reads kPastZeros or, for mixed keys, the
  // split's last unit), scales first, then the tiles: the order of the
  // loop's own requests.
  load_scales(u_first);
#pragma unroll
  for (int i = 0; i < kSlots; ++i) load_tile(u_first + kWaves * (i / ut), i % ut, i);

  // This lane's query values (head a_head, channels of lane group lq) on
  // its key k-slots, times the inverse slot factor, sm_scale * log2(e) and
  // a power of two sigma_q (one for all heads) that brings them below 2 in
  // magnitude; wave 0 keeps them in LDS for all waves.  Each key group's
  // scale row is multiplied by its own power of two sigma_g (largest scale
  // below 2^13) when it is committed to LDS, so |Q'| < 2^14.
  float inv_sigma_q;
  {
    const bool ok = q_ok;
    float qv[32];
    if (a.q_f16) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const half8 h8 = __builtin_bit_cast(half8, qraw[c]);
#pragma unroll
        for (int j = 0; j < 8; ++j) qv[8 * c + j] = (float)h8[j];
      }
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float4v f4 = __builtin_bit_cast(float4v, qraw[c]);
#pragma unroll
        for (int j = 0; j < 4; ++j) qv[4 * c + j] = f4[j];
      }
    }
    float qabs = 0.0f;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      qv[c] = ok ? qv[c] * a.qscale : 0.0f;
      qabs = fmaxf(qabs, fabsf(qv[c]));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) qabs = fmaxf(qabs, __shfl_xor(qabs, o));
    int ex = (int)((__builtin_bit_cast(uint32_t, qabs) >> 23) & 0xFF) - 127;
    ex = ex < -100 ? -100 : ex;
    const float sigma_q = __builtin_bit_cast(float, (uint32_t)(127 - ex) << 23);
    inv_sigma_q = __builtin_bit_cast(float, (uint32_t)(127 + ex) << 23);
    if (KM) {
      // mixed keys: the class order differs per group, so keep q by
      // channel (lanes of one row and lane group write the same values;
      // rows of heads past g are zero)
      if (wave == 0) {
        for (int j = lane; j < 8 * kD; j += 64)
          if (j / kD >= g) S.qs[j / kD][j % kD] = 0.0f;
        if (ok) {
#pragma unroll
          for (int c = 0; c < 32; c += 4)
            *(float4v*)&S.qs[a_head][32 * lq + c] =
                (float4v){qv[c], qv[c + 1], qv[c + 2], qv[c + 3]} * sigma_q;
        }
      }
    } else if (wave == 0) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float qf[8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 2; ++e)
            qf[2 * i + e] = qv[k_slot_channel<KB == 0 ? 4 : KB>(kb, i, e)] * sigma_q *
                            (1.0f / (float)(1 << slot_log2f<KB == 0 ? 4 : KB>(i)));
        S.qf[2 * kb][lane + (lane >> 4)] = (float4v){qf[0], qf[1], qf[2], qf[3]};
        S.qf[2 * kb + 1][lane + (lane >> 4)] = (float4v){qf[4], qf[5], qf[6], qf[7]};
      }
    }
  }
  __syncthreads();
  // mixed keys: A operands of the bf16-channel MFMAs (three bf16 limbs of
  // the query on the bf16 channels)
  bf16x8 qbA = {}, qbB = {};

  for (int u = u_first; u < u_hi; u += kWaves * ups) {
    const int un = u + kWaves * ups;  // first unit of the next step
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
      const int uc = u + kWaves * (i / ut);  // this tile's unit
      if (i % ut == 0) {
        // (a step's later unit past the end ends the wave's loop: the
        // next step would start past it too)
        if (i > 0 && uc >= u_hi) goto units_done;
        // ---- unit start: commit the unit's scales, request the next
        //      unit's, and build Q' for the unit's key group (every unit,
        //      so that Q' is not carried from one unit to the next, which
        //      costs registers)
        {
          const int e = unit_vscale_exp(vsn, lane, n_vs4);
          if (!ev_set || e > ev || e < ev - 6) {
            if (ev_set) {
              const float r = pow2f(ev - e);
#pragma unroll
              for (int jb = 0; jb < 8; ++jb) o[jb] *= r;
            }
            ev = e;
            ev_set = true;
          }
        }
        const float sig_v = pow2f(kVTop - ev);
#pragma unroll
        for (int j = 0; j < kVs4; ++j) {
          const int idx = lane + 64 * j;
          if (idx < n_vs4) ((float4v*)my_vs)[idx] = vsn[j] * sig_v;
        }
        const float kgv = KM ? kgn : row_max_lanes32(ksn);
        int exg = (int)((__builtin_bit_cast(uint32_t, kgv) >> 23) & 0xFF) - 127;
        exg = exg < -100 ? -100 : exg;
        const float sigma_g = __builtin_bit_cast(float, (uint32_t)(127 + 12 - exg) << 23);
        const float inv_sigma_g = __builtin_bit_cast(float, (uint32_t)(127 - 12 + exg) << 23);
        if (!KM) {
          if (lane < kD / 4) ((float4v*)my_ks)[lane] = ksn * sigma_g;
        } else {
          // padded slot layout: int4 positions at slots 0 .. 32 n4b - 1, int2
          // positions from slot 32 n4b on; padding slots keep scale 0
          if (lane < ksrow / 4) {
            // times the inverse slot factors: int4 (1, 1/16, 1, 1/16), int2
            // (1, 1/4, 1, 1/4) (a float4 of slots is one slot pair pattern)
            const bool i4 = 4 * lane < N4;
            const int dst = i4 ? lane : 8 * n4b + lane - N4 / 4;
            const float fo = i4 ? 0.0625f : 0.25f;
            ((float4v*)my_ks)[dst] = ksn * sigma_g * (float4v){1.0f, fo, 1.0f, fo};
          }
          // slot (or bf16 index) -> channel, for channels 2 lane and 2 lane + 1
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int pos = (kpn >> (8 * e)) & 0xFF;
            const int slot = pos < NB ? kD + pos : (pos < NB + N4 ? pos - NB : 32 * n4b + pos - NB - N4);
            my_inv[slot] = (uint16_t)(4 * (2 * lane + e));
          }
        }
        __builtin_amdgcn_wave_barrier();
        // scales of the wave's next unit
        load_scales(uc + kWaves);
        {
          isk = inv_sigma_q * inv_sigma_g * 16777216.0f;
          // one limb per lane: the high part, or the rounding residual
          const uint32_t lmask = limb ? 0xFFFFFFFFu : 0u;
          typedef _Float16 half2v __attribute__((ext_vector_type(2)));
          if (KM) {
            // Q' by padded slot: block kb < n4b holds int4 slots 32 kb + 8 lq +
            // nibble (slot pair i: nibbles i and i + 4, factor 1 or 16); the
            // others int2 slots 32 kb + 16 (lq / 2) + 4 (lq & 1) + field (fields
            // i and i + 8, factor 1 or 4: fields 2 and 3 are read from the word
            // shifted right by 4).  Padding slots have scale 0.
            const char* qrow = (const char*)S.qs[a_head < g ? a_head : 7];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              const bool b4 = kb < n4b;
              const int base = b4 ? 32 * kb + 8 * lq : 32 * kb + 16 * (lq >> 1) + 4 * (lq & 1);
              const int step = b4 ? 4 : 8;  // slot distance of element 1
              const float4v k0 = *(const float4v*)(my_ks + base);
              const float4v k1 = *(const float4v*)(my_ks + base + step);
              u32x4 r;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                // slot factors are already in the scale row; unused slots have
                // scale 0, rows of heads past g are zero
                const float x0 = *(const float*)(qrow + my_inv[base + i]) * k0[i];
                const float x1 = *(const float*)(qrow + my_inv[base + step + i]) * k1[i];
                const half2v hi = {(_Float16)x0, (_Float16)x1};
                const half2v hsel = __builtin_bit_cast(half2v, __builtin_bit_cast(uint32_t, hi) & lmask);
                const half2v res = {(_Float16)(x0 - (float)hsel[0]), (_Float16)(x1 - (float)hsel[1])};
                r[i] = __builtin_bit_cast(uint32_t, res);
              }
              qa[kb] = __builtin_bit_cast(half8, r);
            }
            float4v c = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              // offsets 8 (int4) or 2 (int2) times the slot pair factors
              const u32x4 o4 = {0x00080008u, 0x00800080u, 0x00080008u, 0x00800080u};
              const u32x4 o2 = {0x00020002u, 0x00080008u, 0x00020002u, 0x00080008u};
              const half8 aoff = __builtin_bit_cast(half8, kb < n4b ? o4 : o2);
              c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kb], aoff, c, 0, 0, 0);
            }
            negc = -c;
            // bf16 channels: lane group 0 holds row ln's query on bf16
            // index j (k-slot j of a bf16 MFMA whose key operand is the
            // token's bf16 row), in the integer part's units (times
            // sigma_g 2^-24, which isk undoes) and split into three bf16
            // limbs: limb-0 rows take the first and third, limb-1 rows the
            // second, so the row pair's sum carries the fp32 product
            if (NB > 0) {
              const float fg = sigma_g * __builtin_bit_cast(float, 0x33800000u);  // 2^-24
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const float x = (lq == 0 && j < NB) ? *(const float*)(qrow + my_inv[kD + j]) * fg : 0.0f;
                const __bf16 h1 = (__bf16)x;
                const float r1 = x - (float)h1;
                const __bf16 h2 = (__bf16)r1;
                const __bf16 h3 = (__bf16)(r1 - (float)h2);
                qbA[j] = limb ? h2 : h1;
                qbB[j] = limb ? (__bf16)0.0f : h3;
              }
            }
          } else {
          // Q' limbs: the A operand repeats each (head, limb) row over the
          // row groups and the limb lanes share the high part, so the wave
          // forms each distinct product once: lane (kb, lq, i) = (lane >> 4,
          // (lane >> 2) & 3, lane & 3) takes slot pair i of key MFMA kb and
          // lane group lq for every distinct head (nh of them), stores the
          // high and low limbs in LDS, and every lane then reads its four
          // operands (the same products and roundings as forming them in
          // place)
          (void)lmask;
          const int nh = HS == 1 ? 1 : 2 * rgd;
          const int bkb = lane >> 4, blq = (lane >> 2) & 3, bi = lane & 3;
          const int c0 = 32 * blq + k_slot_channel<KB == 0 ? 4 : KB>(bkb, bi, 0);
          const float k0 = my_ks[c0], k1 = my_ks[c0 + (KB == 4 ? 4 : 8)];
          const float* qsrc = (const float*)&S.qf[2 * bkb + (bi >> 1)][17 * blq] + 2 * (bi & 1);
          uint32_t* qdst = (uint32_t*)&S.u.t.qp[wave][bkb][blq][0] + bi;
          for (int hh = 0; hh < nh; ++hh) {
            // lane 2 hh of each lane group holds head hh (limb 0) in qf
            const float2 qq = *(const float2*)(qsrc + 8 * hh);
            const float x0 = qq.x * k0, x1 = qq.y * k1;
            const half2v hi = {(_Float16)x0, (_Float16)x1};
            const half2v lo = {(_Float16)(x0 - (float)hi[0]), (_Float16)(x1 - (float)hi[1])};
            qdst[8 * hh] = __builtin_bit_cast(uint32_t, hi);
            qdst[8 * hh + 4] = __builtin_bit_cast(uint32_t, lo);
          }
          __builtin_amdgcn_wave_barrier();
          const int qrow = HS == 1 ? limb : 2 * a_head + limb;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            qa[kb] = __builtin_bit_cast(half8, S.u.t.qp[wave][kb][lq][qrow]);
          const half8 aoff = k_offset_operand<KB == 0 ? 4 : KB>();
          float4v c = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kb], aoff, c, 0, 0, 0);
          negc = -c;
          }
        }
        __builtin_amdgcn_wave_barrier();
      }

      // ---- scores: rows 4lq..4lq+3 (head slots x limbs) of token ln of
      //      each 16-token half
      float4v acc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        acc[h] = negc;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          half8 B;
          if (KM) {
            // one form for both classes: int4 masks nibble pairs of the word
            // and of the word >> 8; int2 masks 2-bit pairs of the lane's 16
            // bits (the word >> kshift)
            const bool b4 = kb < n4b;
            const uint32_t w = kw[i % kSlots][h][kb] >> kshift[kb];
            const uint32_t w8 = w >> (b4 ? 8 : 4);
            u32x4 r;
            r[0] = w & (b4 ? 0x000F000Fu : 0x00030003u);
            r[1] = w & (b4 ? 0x00F000F0u : 0x000C000Cu);
            r[2] = w8 & (b4 ? 0x000F000Fu : 0x00030003u);
            r[3] = w8 & (b4 ? 0x00F000F0u : 0x000C000Cu);
            B = __builtin_bit_cast(half8, r);
          } else if (KB == 4) {
            B = int4_key_operand(kw[i % kSlots][h][kb]);
          } else {
            const uint32_t word = kw[i % kSlots][h][kb >> 1];
            B = int2_key_operand((kb & 1) ? (word >> 8) : word);
          }
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kb], B, acc[h], 0, 0, 0);
        }
        if (KM && NB > 0) {
          // the bf16 channels: the token's bf16 row is the key operand
          // (k-slots past NB, and every slot of lane groups 1-3, meet zero
          // query limbs)
          const u32x2 lo = kb16lo[KM ? i % kSlots : 0][h], hi = kb16hi[KM ? i % kSlots : 0][h];
          const bf16x8 kbf = __builtin_bit_cast(bf16x8, (u32x4){lo[0], lo[1], hi[0], hi[1]});
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qbA, kbf, acc[h], 0, 0, 0);
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qbB, kbf, acc[h], 0, 0, 0);
        }
      }
      // whole scores (head slot hl: rows 2 hl and 2 hl + 1, the limbs)
      float sc[2][HS];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int hl = 0; hl < HS; ++hl) sc[h][hl] = acc[h][2 * hl] + acc[h][2 * hl + 1];
      const float sk = isk;
      // ---- tile max per head slot, online softmax
      float tmx[HS];
      bool grow = false;
#pragma unroll
      for (int hl = 0; hl < HS; ++hl) {
        tmx[hl] = row_max16(fmaxf(sc[0][hl], sc[1][hl])) * sk;
        grow = grow || tmx[hl] > m_run[hl] + (float)kLazy;
      }
      if (__any(grow)) {
        float alpha[HS];
#pragma unroll
        for (int hl = 0; hl < HS; ++hl) {
          const float mn = fmaxf(m_run[hl], tmx[hl]);
          alpha[hl] = __builtin_amdgcn_exp2f(m_run[hl] - mn);
          m_run[hl] = mn;
          l_part[hl] *= alpha[hl];
          cm[0][hl] = -mn - (float)lf0;
          cm[1][hl] = -mn - (float)lf1;
        }
        float av;
        if (HS == 1) {
          av = alpha[0];
        } else {
          const int src = 16 * ((v_head >> 1) % rgd);
          const float a0 = __shfl(alpha[0], src), a1 = __shfl(alpha[HS - 1], src);
          av = (v_head & 1) ? a1 : a0;
        }
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) o[jb] *= av;
      }
      // p / f(slot pair) for the value operand, sums of the unscaled p
      float p[2][HS];
#pragma unroll
      for (int hl = 0; hl < HS; ++hl) {
        p[0][hl] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[0][hl], sk, cm[0][hl]));
        p[1][hl] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[1][hl], sk, cm[1][hl]));
        l_part[hl] = __builtin_fmaf(p[0][hl], f0, __builtin_fmaf(p[1][hl], f1, l_part[hl]));
      }
      // ---- P' = p * v_scale into the value B layout, with no lane
      //      conditions: rows of heads at or past g feed only output columns
      //      that are never kept, and a lane whose value group c is past NC
      //      (possible only when g * NC < 16) writes row 15, which then
      //      belongs to no head below g.  (2-bit keys with 4-bit values and
      //      two head slots keep the lane conditions: without them those
      //      variants spill at three waves per SIMD.)
      constexpr bool kNoLaneIf = !(KB == 2 && VB == 4 && HS == 2);
      const float* vrow = my_vs + ((i % ut) * 32 + ln) * NC;
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        if (j >= niter) break;
        const int c = rep_idx + j * rep;
        if (kNoLaneIf) {
          const bool cok = c < NC;
          const int cr = cok ? c : NC - 1;
          const float vs0 = vrow[cr], vs1 = vrow[16 * NC + cr];
#pragma unroll
          for (int hl = 0; hl < HS; ++hl) {
            _Float16* row = my_pl[cok ? s_head[hl] * NC + c : 15];
            row[kpos] = (_Float16)(p[0][hl] * vs0);
            row[kpos + 4] = (_Float16)(p[1][hl] * vs1);
          }
        } else if (c < NC) {
          const float vs0 = vrow[c], vs1 = vrow[16 * NC + c];
#pragma unroll
          for (int hl = 0; hl < HS; ++hl) {
            if (s_head[hl] < g) {
              _Float16* row = my_pl[s_head[hl] * NC + c];
              row[kpos] = (_Float16)(p[0][hl] * vs0);
              row[kpos + 4] = (_Float16)(p[1][hl] * vs1);
            }
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      const half8 pb = *(const half8*)&my_pl[ln][8 * lq];
      // ---- value MFMAs
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) {
        half8 A;
        if (VB == 2) {
          const uint32_t word = vw[i % kSlots][0][jb >> 1];
          A = int2_operand((jb & 1) ? (word >> 8) : word, magic);
        } else {
          A = int4_operand(vw[i % kSlots][jb >> 2][jb & 3], magic);
        }
        o[jb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, pb, o[jb], 0, 0, 0);
      }
      __builtin_amdgcn_wave_barrier();
      // refill the slot with the wave's tile kSlots places later
      if (i + kSlots < kStep) {
        const int uf = u + kWaves * ((i + kSlots) / ut);
        load_tile(uf, (i + kSlots) % ut, i % kSlots);
      } else {
        const int uf = un + kWaves * ((i + kSlots - kStep) / ut);
        load_tile(uf, (i + kSlots - kStep) % ut, i % kSlots);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
units_done:

  // ---- per-wave state to LDS (after every wave is done with its P' buffer);
  //      the output divided by sigma_v
#pragma unroll
  for (int hl = 0; hl < HS; ++hl) l_part[hl] = row_sum16(l_part[hl]);
  if (ev_set) {
    const float r = pow2f(ev - kVTop);
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) o[jb] *= r;
  }
  __syncthreads();
  if (ln == 0 && lq < rgd) {
#pragma unroll
    for (int hl = 0; hl < HS; ++hl) {
      if (s_head[hl] < g) {
        S.m[wave][s_head[hl]] = m_run[hl];
        S.l[wave][s_head[hl]] = l_part[hl];
      }
    }
  }
  if (v_valid) {
#pragma unroll
    for (int jb = 0; jb < 8; ++jb)
      if ((jb * NC) / 8 == v_cc)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          S.u.o[wave][v_head][16 * jb + 4 * lq + j] = o[jb][j];
  }
  __syncthreads();

  // ---- merge the four waves into this split's partial
  for (int i = threadIdx.x; i < g * (kD + 2); i += kThreads) {
    const int h = i / (kD + 2), jx = i % (kD + 2);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (S.l[w][h] > 0.0f) M = fmaxf(M, S.m[w][h]);
    float val = 0.0f;
    if (jx == 0) {
      val = M;
    } else {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        if (S.l[w][h] > 0.0f) {
          const float sc_w = exp2f(S.m[w][h] - M);
          val += (jx == 1 ? S.l[w][h] : S.u.o[w][h][jx - 2]) * sc_w;
        }
      }
    }
    a.partials[(((int64_t)b * a.Hq + kvh * g + h) * a.n_parts + part) * (kD + 2) + jx] = val;
  }
}


// Whether the row-score kernel runs for this view (else the column kernel).
bool rows_kernel(const kvq_kv_view& v, int Hq) {
  const int g = Hq / v.kv_heads, nc = kD / v.group_ch;
  return g <= 8 && g * nc <= 16;
}

// Resident workgroups per compute unit of a row-score variant (the
// occupancy the compiler's register and LDS use allows), cached.
// Tiles per unit of the row-score kernel: four, or two or one when the key
// group is shorter or not a multiple of four tiles.
int rs_unit_tiles(const kvq_kv_view& v) {
  const int tpg = v.group_tok / 32;
  return tpg % 4 == 0 ? 4 : (tpg % 2 == 0 ? 2 : 1);
}

template <int KB, int VB, int NC, int HS>
int rs_wgs_ut(int ut) {
  static int cached[3] = {0, 0, 0};
  int& c = cached[ut == 4 ? 2 : ut - 1];
  if (c == 0) {
    int n = 0;
    const hipError_t e =
        ut == 4 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_rs_kernel<KB, VB, NC, HS, 4>, kThreads, 0)
        : ut == 2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_rs_kernel<KB, VB, NC, HS, 2>, kThreads, 0)
                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_rs_kernel<KB, VB, NC, HS, 1>, kThreads, 0);
    c = (e == hipSuccess && n > 0) ? n : 2;
  }
  return c;
}
template <int KB, int VB, int NC>
int rs_wgs_per_cu(int g, int ut) {
  return g == 1 ? rs_wgs_ut<KB, VB, NC, 1>(ut) : rs_wgs_ut<KB, VB, NC, 2>(ut);
}
template <int KB, int VB>
int rs_wgs_nc(int nc, int g, int ut) {
  switch (nc) {
    case 1: return rs_wgs_per_cu<KB, VB, 1>(g, ut);
    case 2: return rs_wgs_per_cu<KB, VB, 2>(g, ut);
    case 4: return rs_wgs_per_cu<KB, VB, 4>(g, ut);
    default: return rs_wgs_per_cu<KB, VB, 8>(g, ut);
  }
}
int rs_wgs(const kvq_kv_view& v, int Hq) {
  const int nc = kD / v.group_ch, g = Hq / v.kv_heads, ut = rs_unit_tiles(v);
  if (v.k_mixed) return v.v_bits == 2 ? rs_wgs_nc<0, 2>(nc, g, ut) : rs_wgs_nc<0, 4>(nc, g, ut);
  if (v.k_bits == 4) return v.v_bits == 2 ? rs_wgs_nc<4, 2>(nc, g, ut) : rs_wgs_nc<4, 4>(nc, g, ut);
  return v.v_bits == 2 ? rs_wgs_nc<2, 2>(nc, g, ut) : rs_wgs_nc<2, 4>(nc, g, ut);
}
int n_cus() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cached = n;
    else
      cached = 256;
  }
  return cached;
}

int fp16_parts(const kvq_kv_view& v);

// Splits per (batch, KV head).  Column kernel: about four workgroups per
// compute unit (two resident, two rounds) and at least eight units per
// wave.  Row-score kernel: the resident workgroups (compute units x
// resident per unit, fp16-row parts included) in one round, or in four
// rounds when one round would leave more than 48 tiles per wave (smaller
// workgroups balance better over the compute units: at 1M tokens 3072 beat
// 768, 1024 and 6144), and at least one unit per wave.  In one round the
// fp16-row parts either take slots of their own, so that every workgroup is
// resident at once, or keep none: the splits are then dispatched first and
// the fp16-row parts take the slots of the first splits to finish (see
// part_index).  The second is taken when the shorter splits save more than
// a trailing fp16-row part adds (estimates: 2 us per tile per wave, 5 us per
// trailing part, which mostly overlaps the spread of the split ends; at
// MixKVQ 32K x 8 with one part per stream, 8 splits and a trailing part
// take 87 us, 7 splits and a slot of its own 100 us).
int auto_splits(const kvq_kv_view& v, int Hq) {
  const int64_t streams = (int64_t)v.batch * v.kv_heads;
  int64_t sp, by_len;
  const int tpg = v.group_tok / 32;
  const int ut = rows_kernel(v, Hq) ? rs_unit_tiles(v) : (tpg < kUnitTiles ? tpg : kUnitTiles);
  const int64_t n_units = v.n_quant / (32 * ut);
  if (rows_kernel(v, Hq)) {
    const int64_t round = (int64_t)n_cus() * rs_wgs(v, Hq);
    const int64_t fp = fp16_parts(v);
    const double tiles = (double)(v.n_quant / 32);
    auto wave_tiles = [&](int64_t n) { return tiles / (double)(n * kWaves); };
    const int64_t slots = round / streams > 1 ? round / streams : 1;
    sp = slots - fp;
    if (sp < 1 || (fp > 0 && 2.0 * (wave_tiles(sp) - wave_tiles(slots)) > 5.0)) sp = slots;
    if (wave_tiles(sp) > 48.0) {
      sp = 4 * round / streams - fp;
      if (sp < 1) sp = 1;
    }
    by_len = n_units / kWaves;
  } else {
    sp = (1024 + streams - 1) / streams;
    by_len = n_units / (8 * kWaves);
  }
  if (sp > by_len) sp = by_len;
  if (sp < 1) sp = 1;
  if (sp > 16000) sp = 16000;
  return (int)sp;
}

int fp16_parts(const kvq_kv_view& v) {
  return (int)((v.n_sink + v.n_tail + kRowsPerChunk - 1) / kRowsPerChunk);
}

template <int KB, int VB, int NC, int HS>
void launch_rs(const MfmaArgs& a, int ut, dim3 grid, hipStream_t s) {
  if (ut == 4)
    decode_rs_kernel<KB, VB, NC, HS, 4><<<grid, kThreads, 0, s>>>(a);
  else if (ut == 2)
    decode_rs_kernel<KB, VB, NC, HS, 2><<<grid, kThreads, 0, s>>>(a);
  else
    decode_rs_kernel<KB, VB, NC, HS, 1><<<grid, kThreads, 0, s>>>(a);
}

template <int KB, int VB, int NC>
hipError_t launch_t(const MfmaArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((int64_t)a.n_parts * a.v.kv_heads * a.v.batch));
  const int g = a.Hq / a.v.kv_heads;
  if (rows_kernel(a.v, a.Hq)) {
    const int ut = rs_unit_tiles(a.v);
    if (g == 1)
      launch_rs<KB, VB, NC, 1>(a, ut, grid, s);
    else
      launch_rs<KB, VB, NC, 2>(a, ut, grid, s);
  } else if constexpr (KB != 0)  // mixed keys run only in the row-score kernel
    decode_mfma_kernel<KB, VB, NC, false><<<grid, kThreads, 0, s>>>(a);
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
  if (v.head_dim != kD || Hq < v.kv_heads || Hq % v.kv_heads) return false;
  if (v.k_mixed) {
    // row-score kernel only, groups of at least two tiles; 0, 4 or 8 bf16
    // channels, whole int4 words, and the int4 and int2 positions in at
    // most four 32-position blocks
    if (!rows_kernel(v, Hq) || v.group_tok < 64) return false;
    if (v.n_bf16 != 0 && v.n_bf16 != 4 && v.n_bf16 != 8) return false;
    const int n2 = kD - v.n_bf16 - v.n_int4;
    if (v.n_int4 < 0 || v.n_int4 % 8 || n2 < 0) return false;
    if ((v.n_int4 + 31) / 32 + (n2 + 31) / 32 > 4) return false;
  } else if (v.k_bits != 4 && v.k_bits != 2) {
    return false;
  }
  if (v.v_bits != 4 && v.v_bits != 2) return false;
  // whole key groups only: a work unit never spans a partial group
  if (v.v_layout != KVQ_V_TILE32 || v.group_tok % 32 || v.n_quant % v.group_tok) return false;
  // the column kernel's units need groups of at most four tiles or whole
  // multiples of four (the row-score kernel takes any multiple of a tile)
  if (!rows_kernel(v, Hq) && v.group_tok > 32 * kUnitTiles && v.group_tok % (32 * kUnitTiles))
    return false;
  if (v.n_quant < 32 || !v.k_gmax || v.n_quant / 32 > 0x7FFFFFFF) return false;
  const int nc = kD / v.group_ch;
  if (nc != 1 && nc != 2 && nc != 4 && nc != 8) return false;
  const int g = Hq / v.kv_heads;
  return g >= 1 && g <= 16;
}

int mfma_decode_parts(const kvq_kv_view& v, int Hq, int n_splits) {
  const int sp = n_splits > 0 ? n_splits : auto_splits(v, Hq);
  return sp + fp16_parts(v);
}

hipError_t launch_decode_mfma(const kvq_kv_view& v, const void* q, int f16, int Hq,
                              float sm_scale, float* partials, int n_parts,
                              hipStream_t s) {
  const int fp = fp16_parts(v);
  const int n_splits = n_parts - fp;
  if ((int64_t)n_parts * v.kv_heads * v.batch > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  // resident workgroups of one round (row-score kernel)
  const int64_t streams = (int64_t)v.batch * v.kv_heads;
  const int64_t total = (int64_t)n_parts * streams;
  const int64_t round = rows_kernel(v, Hq) ? (int64_t)n_cus() * rs_wgs(v, Hq) : 0;
  const int fp_last = fp > 0 && round > 0 && total > round && total - round <= streams * fp;
  MfmaArgs a{v, q, f16, Hq, sm_scale * kLog2e, partials, n_parts, n_splits, fp_last};
  const int nc = kD / v.group_ch;
  hipError_t e;
  if (v.k_mixed) e = v.v_bits == 2 ? launch_nc<0, 2>(a, nc, s) : launch_nc<0, 4>(a, nc, s);
  else if (v.k_bits == 4 && v.v_bits == 2) e = launch_nc<4, 2>(a, nc, s);
  else if (v.k_bits == 4 && v.v_bits == 4) e = launch_nc<4, 4>(a, nc, s);
  else if (v.k_bits == 2 && v.v_bits == 2) e = launch_nc<2, 2>(a, nc, s);
  else e = launch_nc<2, 4>(a, nc, s);
  return e;
}

}  // namespace kvq
