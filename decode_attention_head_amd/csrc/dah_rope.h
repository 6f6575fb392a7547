// RoPE angles for the decode kernels: cos and sin of pos * theta^(-2i/128)
// (node attn.rope of the "Qwen3-0.6B" Model Spec page, "Compute-graph
// nodes"), to float32 accuracy for any position of the shape domain
// (pos < 40,960) and beyond.
//
// Method.
//  * theta^(-i/64) for i < 64 is the product of the precomputed powers
//    theta^(-2^k/64) selected by the bits of i (at most 6 float64 products,
//    relative error below 1e-14).
//  * The angle phi = pos * theta^(-i/64) is formed in float64 and reduced by
//    pi/2 with the Cody-Waite method: n = round(phi * 2/pi), and
//    r = (phi - n*P1) - n*P1t, where P1 holds the leading 33 bits of pi/2 (so
//    n*P1 is exact for |n| < 2^20) and P1t the next 53.  |r| <= pi/4.
//  * cos and sin of r come from their Taylor polynomials in float32 (through
//    r^10 and r^9: truncation below 1.2e-10 and 1.7e-9 on |r| <= pi/4), and
//    the quadrant n mod 4 maps (sin r, cos r) to (sin phi, cos phi).
// No part of the platform's math library is involved, so this header also
// builds as plain host C++ for tests.
#pragma once

#include <math.h>

#if defined(__HIPCC__)
#define DAH_HD __host__ __device__
#else
#define DAH_HD
#endif

namespace dah {

// theta^(-2^k/64), k = 0..5
struct RopePowers {
  double p[6];
};

inline RopePowers rope_powers(double theta) {
  RopePowers r;
  for (int k = 0; k < 6; ++k) r.p[k] = pow(theta, -(double)(1 << k) / 64.0);
  return r;
}

DAH_HD inline double rope_inv_freq(int i, const RopePowers& r) {
  double f = 1.0;
  for (int k = 0; k < 6; ++k) f = ((i >> k) & 1) ? f * r.p[k] : f;
  return f;
}

DAH_HD inline void rope_cos_sin(double phi, float* c, float* s) {
  const double kTwoOverPi = 0.63661977236758134308;
  const double kP1 = 1.57079632673412561417e+00;   // leading 33 bits of pi/2
  const double kP1t = 6.07710050650619224932e-11;  // pi/2 - kP1
  const double n = rint(phi * kTwoOverPi);
  const double r = fma(-n, kP1t, phi - n * kP1);
  const float x = (float)r;
  const float x2 = x * x;
  const float sn = x + x * x2 * (-1.0f / 6 + x2 * (1.0f / 120 + x2 * (-1.0f / 5040 + x2 * (1.0f / 362880))));
  const float cs = 1.0f + x2 * (-0.5f + x2 * (1.0f / 24 + x2 * (-1.0f / 720 +
                   x2 * (1.0f / 40320 + x2 * (-1.0f / 3628800)))));
  const int q = (int)((long long)n & 3);
  *s = q == 0 ? sn : q == 1 ? cs : q == 2 ? -sn : -cs;
  *c = q == 0 ? cs : q == 1 ? -sn : q == 2 ? -cs : sn;
}

}  // namespace dah
