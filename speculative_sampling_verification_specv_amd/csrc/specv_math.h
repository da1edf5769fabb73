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

// 2^(j/64), j = 0..63, each correctly rounded (printed by gen_exp2_table.py).
constexpr double kExp2Table[64] = {
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0,
    0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0,
    0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0,
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0,
    0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0,
    0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0,
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0,
    0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0,
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0,
    0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0,
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0,
    0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0,
    0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0,
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0,
};

// exp(a) for a <= 0 in fp64 from a 64-entry table: a = (64 m + j) ln2/64 + r
// with 64 m + j = rint(64 a / ln2) (the 1.5*2^52 shifter) and |r| <= ln2/128
// (two-part ln2/64: the high part times |64 m + j| < 2^17 is exact);
// exp(a) = 2^m * 2^(j/64) * (1 + expm1(r)) with expm1(r) from its degree-5
// Taylor polynomial (truncation below 4e-17 on |r| <= ln2/128), 2^(j/64) from
// `tab` (kExp2Table, wherever the caller keeps it), one fma joining them
// and ldexp for 2^m (which also gives the subnormal range). About 1 ulp; the
// same clamp at -746 as exp_nonpos.
__host__ __device__ inline double exp_nonpos_tab(double a, const double* tab) {
  a = fmax(a, -746.0);
  const double kShift = 6755399441055744.0;             // 1.5 * 2^52
  const double kInvLn2x64 = 92.33248261689366;          // 64 / ln 2
  const double kLn2Hi64 = 6.93147180369123816490e-01 / 64.0;  // ln 2 / 64, upper bits
  const double kLn2Lo64 = 1.90821492927058770002e-10 / 64.0;  // the rest
  const double t = fma(a, kInvLn2x64, kShift);
  const double kd = t - kShift;
  const int32_t n = static_cast<int32_t>(static_cast<uint32_t>(double_to_bits(t)));
  double r = fma(kd, -kLn2Hi64, a);
  r = fma(kd, -kLn2Lo64, r);
  double p = fma(r, 1.0 / 120.0, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = p * r;  // expm1(r)
  const double s = tab[n & 63];
  return ldexp(fma(s, p, s), n >> 6);
}

}  // namespace specv
