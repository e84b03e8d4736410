// RoPE angle in double precision, written with plain arithmetic so that the
// same code compiles for the host (where a CPU test pins its accuracy) and
// for gfx950 (where it replaces the much longer library exp2/log2 chains on
// the critical path of the compressor and attention epilogues).
//
// Pair i of a rope_dim-wide slice at position p turns by p * base^(-2i/rope_dim)
// ("DeepSeek-V4-Flash 架构：一个 token 的旅程", section "压缩是逐通道的 learned
// pooling": the trailing channels carry the position).  log2(base) is formed
// once on the host and handed to the kernels.
#pragma once

#ifndef __HIPCC__
#include <cmath>
#define CSA_HD
#else
#define CSA_HD __host__ __device__
#endif

namespace csa {

constexpr double kLn2d = 0.6931471805599453094;  // ln 2, rounded to double
constexpr double kTwoPiHi = 6.283185307179586;    // 2*pi rounded to double
constexpr double kTwoPiLo = 2.4492935982947064e-16;  // 2*pi - kTwoPiHi

// 2^x for |x| < 1000.  Argument reduction x = n + f, n = rint(x), |f| <= 1/2
// (f is exact); 2^f = e^t with t = f ln 2, |t| <= 0.347, from the Taylor
// series of e^t summed to t^12 by Horner's rule (the first omitted term is
// below 2e-16 of the result); the power of two is applied with ldexp.
CSA_HD inline double exp2_taylor(double x) {
  const double n = rint(x);
  const double t = (x - n) * kLn2d;
  double q = 1.0 / 479001600.0;  // 1/12!
  q = fma(q, t, 1.0 / 39916800.0);
  q = fma(q, t, 1.0 / 3628800.0);
  q = fma(q, t, 1.0 / 362880.0);
  q = fma(q, t, 1.0 / 40320.0);
  q = fma(q, t, 1.0 / 5040.0);
  q = fma(q, t, 1.0 / 720.0);
  q = fma(q, t, 1.0 / 120.0);
  q = fma(q, t, 1.0 / 24.0);
  q = fma(q, t, 1.0 / 6.0);
  q = fma(q, t, 0.5);
  q = fma(q, t, 1.0);
  q = fma(q, t, 1.0);
  return ldexp(q, int(n));
}

// Rotation angle of pair i at position p, reduced into [-pi, pi] with a
// two-term split of 2*pi, so that positions near 2^20 keep an absolute error
// of a few 1e-10 rad.
CSA_HD inline double rope_angle(long long p, int i, int rope_dim, double log2_base) {
  const double theta = exp2_taylor(-2.0 * double(i) / double(rope_dim) * log2_base);
  const double x = double(p) * theta;
  const double k = rint(x * (1.0 / kTwoPiHi));
  const double r = fma(-k, kTwoPiHi, x);
  return fma(-k, kTwoPiLo, r);
}

}  // namespace csa

#undef CSA_HD
