// Rotary position embedding arithmetic of libkvq's decode kernels (keys
// cached before the embedding: "KVQuant: Towards 10 Million Context Length
// LLM Inference with KV Cache Quantization", "Approach").
//
// Frequency f = 0 .. D/2 - 1 turns by theta_f = base^(-2f/D) radians per
// position.  Angles are kept in turns (fractions of a full turn): the turns
// of position p are p * phi_f with phi_f = theta_f / (2 pi) in float64, and
// only the fractional part, |x| <= 1/2, goes on to float32.  Positions up to
// 2^40 keep that fraction accurate to about 1e-10 turns.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kRopeMaxFreq = 128;  // D / 2 for D <= 256

struct RopeDev {
  double base;                     // theta_f = base^(-2f/D)
  int interleaved;                 // 0: channel f pairs with f + D/2; 1: 2f with 2f + 1
  int64_t pos0;                    // position of cache-order token 0
  double phi[kRopeMaxFreq];        // theta_f / (2 pi): turns per position
};

// Fractional turns of p * phi, in [-1/2, 1/2].
__device__ inline float rope_turns(double p, double phi) {
  const double a = p * phi;
  return (float)(a - rint(a));
}

// (cos, sin) of 2 pi x for |x| <= 1/2.  x drops whole quarter turns first
// (an exact subtraction); the rest, |a| <= pi/4 radians, goes through the
// Taylor series of sin to the a^11 term and of cos to the a^12 term
// (truncation below 1e-11), and the quarter turns are put back by swapping
// and negating.
__device__ inline float2 rope_cos_sin(float x) {
  const float qf = rintf(4.0f * x);
  const float r = __builtin_fmaf(-0.25f, qf, x);
  const float a = r * 6.28318530717958647692f;
  const float u = a * a;
  float s = -2.50521083854417188e-8f;        // -1/11!
  s = __builtin_fmaf(s, u, 2.75573192239858907e-6f);   // 1/9!
  s = __builtin_fmaf(s, u, -1.98412698412698413e-4f);  // -1/7!
  s = __builtin_fmaf(s, u, 8.33333333333333333e-3f);   // 1/5!
  s = __builtin_fmaf(s, u, -1.66666666666666667e-1f);  // -1/3!
  s = __builtin_fmaf(s * u, a, a);
  float c = 2.08767569878680990e-9f;         // 1/12!
  c = __builtin_fmaf(c, u, -2.75573192239858907e-7f);  // -1/10!
  c = __builtin_fmaf(c, u, 2.48015873015873016e-5f);   // 1/8!
  c = __builtin_fmaf(c, u, -1.38888888888888889e-3f);  // -1/6!
  c = __builtin_fmaf(c, u, 4.16666666666666667e-2f);   // 1/4!
  c = __builtin_fmaf(c, u, -0.5f);
  c = __builtin_fmaf(c, u, 1.0f);
  const int qd = (int)qf & 3;
  float2 r2;
  r2.x = (qd == 0) ? c : (qd == 1) ? -s : (qd == 2) ? -c : s;
  r2.y = (qd == 0) ? s : (qd == 1) ? c : (qd == 2) ? -s : -c;
  return r2;
}

}  // namespace kvq
