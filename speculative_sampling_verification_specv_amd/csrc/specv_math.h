// Device math shared by the kernels (and compiled on the host by its unit test).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

namespace specv {

// 2^(j/64), j = 0..63, rounded to double, filled by fill_exp_table().
constexpr int kExpTableSize = 64;

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

// exp(a) for a <= 0 in fp64, table-driven (Tang's method): a = (64n + j) ln2/64 + r
// with |r| <= ln2/128, exp(a) = 2^n * 2^(j/64) * exp(r), exp(r) - 1 by its degree-5
// Taylor polynomial (truncation < 4e-17 relative). The rounding-to-nearest of
// a*64/ln2 uses the 1.5*2^52 shifter, whose low word then holds the integer k.
// The power of two is applied by adding n to the exponent field, valid because
// results stay normal for a >= -708; below that (including -inf) the result is 0,
// which only drops terms under 3.3e-308 of the row maximum. NaN gives 0.
// Relative error: a few ulp.
__host__ __device__ inline double exp_nonpos(double a, const double* __restrict__ table) {
  const double kShift = 6755399441055744.0;                   // 1.5 * 2^52
  const double kInvStep = 92.332482616893658;                 // 64 / ln 2
  const double kStepHi = 0x1.62e42fefa0000p-7;                // ln2/64, 36 significant bits
  const double kStepLo = 0x1.cf79abc9e3b3ap-46;               // ln2/64 - kStepHi
  const double t = fma(a, kInvStep, kShift);
  const double kd = t - kShift;
  const int32_t k = static_cast<int32_t>(static_cast<uint32_t>(double_to_bits(t)));
  double r = fma(kd, -kStepHi, a);
  r = fma(kd, -kStepLo, r);
  double p = fma(r, 1.0 / 120.0, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = p * r;
  const double base = table[k & (kExpTableSize - 1)];
  const double res = fma(base, p, base);
  const uint64_t scaled = double_to_bits(res) + (static_cast<uint64_t>(static_cast<int64_t>(k >> 6)) << 52);
  return (a >= -708.0) ? bits_to_double(scaled) : 0.0;
}

}  // namespace specv
