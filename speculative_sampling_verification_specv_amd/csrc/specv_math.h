// fp64 exponential shared by the kernels; also compiled by a plain host
// compiler for its unit test.
#pragma once

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#else
#define __host__
#define __device__
#endif
#include <stdint.h>
#include <string.h>

namespace specv {

// 2^(j/256), j = 0..255, rounded to double (filled by the host).
constexpr int kExpTableSize = 256;

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

// exp(a) for a <= 0 in fp64, table-driven (Tang's method): a = (256n + j) ln2/256 + r
// with |r| <= ln2/512, exp(a) = 2^n * 2^(j/256) * exp(r), and exp(r) - 1 by its
// degree-3 Taylor polynomial (truncation below 1.5e-13 relative). Rounding
// a*256/ln2 to an integer uses the 1.5*2^52 shifter, whose low word then holds
// it; one fma reduces with ln2/256 rounded to double (error below 1e-13 for
// a >= -708). The power of two is applied by adding n to the exponent field,
// valid because results stay normal for a >= -708; below that (including
// -inf) the result is 0, which only drops terms under 3.3e-308 of the row
// maximum. NaN gives 0. Relative error below 3e-13.
__host__ __device__ inline double exp_nonpos(double a, const double* __restrict__ table) {
  const double kShift = 6755399441055744.0;      // 1.5 * 2^52
  const double kInvStep = 369.3299304675746;     // 256 / ln 2
  const double kStep = 0x1.62e42fefa39efp-9;     // ln2 / 256
  const double t = fma(a, kInvStep, kShift);
  const double kd = t - kShift;
  const int32_t k = static_cast<int32_t>(static_cast<uint32_t>(double_to_bits(t)));
  const double r = fma(kd, -kStep, a);
  const double q = fma(fma(r, 1.0 / 6.0, 0.5), r, 1.0) * r;  // exp(r) - 1
  const double base = table[k & (kExpTableSize - 1)];
  const double res = fma(base, q, base);
  const uint64_t scaled = double_to_bits(res) + (static_cast<uint64_t>(static_cast<int64_t>(k >> 8)) << 52);
  return (a >= -708.0) ? bits_to_double(scaled) : 0.0;
}

}  // namespace specv
