// fp64 exponential used by the draw kernels; also compiled by a plain host
// compiler for its unit test.
#pragma once

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#else
#define __host__
#define __device__
#endif
#include <math.h>
#include <stdint.h>
#include <string.h>

namespace specv {

__host__ __device__ inline double bits_to_double(uint64_t u) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __longlong_as_double(static_cast<long long>(u));
#else
  double d;
  memcpy(&d, &u, sizeof d);
  return d;
#endif
}

__host__ __device__ inline uint64_t double_to_bits(double d) {
#if defined(__HIP_DEVICE_COMPILE__)
  return static_cast<uint64_t>(__double_as_longlong(d));
#else
  uint64_t u;
  memcpy(&u, &d, sizeof u);
  return u;
#endif
}

// exp(a) for a <= 0 in fp64, without tables (registers only, so independent
// calls overlap freely): a = n ln2 + r with n = rint(a / ln2) and
// |r| <= ln2/2, exp(a) = 2^n exp(r). n comes from the 1.5*2^52 shifter (the
// low word of the shifted value holds it); r from a two-part ln2 (Cody and
// Waite: n * ln2_hi is exact for |n| < 2^11, the low part adds 1e-16
// relative); exp(r) from its degree-11 Taylor polynomial by Horner's rule
// (truncation below 1e-14 relative on |r| <= ln2/2; one coefficient per
// step, so the coefficients stay scalar operands); 2^n by ldexp, which also
// gives the subnormal range. Arguments below -746 (and -inf or NaN) are
// clamped to -746, where 2^n * exp(r) rounds to exactly 0. Relative error below
// 1e-13 down to a = -708.
__host__ __device__ inline double exp_nonpos(double a) {
  a = fmax(a, -746.0);
  const double kShift = 6755399441055744.0;         // 1.5 * 2^52
  const double kInvLn2 = 1.4426950408889634;        // 1 / ln 2
  const double kLn2Hi = 6.93147180369123816490e-01;  // ln 2, upper bits (low 32 bits zero)
  const double kLn2Lo = 1.90821492927058770002e-10;  // ln 2 - kLn2Hi
  const double t = fma(a, kInvLn2, kShift);
  const double kd = t - kShift;
  const int32_t n = static_cast<int32_t>(static_cast<uint32_t>(double_to_bits(t)));
  double r = fma(kd, -kLn2Hi, a);
  r = fma(kd, -kLn2Lo, r);
  double p = fma(r, 1.0 / 39916800.0, 1.0 / 3628800.0);  // 1/11!, 1/10!
  p = fma(p, r, 1.0 / 362880.0);
  p = fma(p, r, 1.0 / 40320.0);
  p = fma(p, r, 1.0 / 5040.0);
  p = fma(p, r, 1.0 / 720.0);
  p = fma(p, r, 1.0 / 120.0);
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(p, n);
}

}  // namespace specv
