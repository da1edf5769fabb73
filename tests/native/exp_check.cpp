// Host check of specv::exp_nonpos against long-double exp: prints the largest
// relative error over a dense grid of [-708, 0] and a few special values.
#include <math.h>
#include <stdio.h>

#include "specv_math.h"

int main() {
  double worst = 0.0, worst_at = 0.0;
  const int n = 4000000;
  for (int i = 0; i <= n; ++i) {
    // Dense near 0 (where most residual exponents sit) and uniform over the range.
    const double a = (i % 2) ? -708.0 * (double(i) / n) : -40.0 * (double(i) / n) * (double(i) / n);
    const long double ref = expl(static_cast<long double>(a));
    const double got = specv::exp_nonpos(a);
    const double rel = static_cast<double>(fabsl((static_cast<long double>(got) - ref) / ref));
    if (rel > worst) {
      worst = rel;
      worst_at = a;
    }
  }
  printf("max_rel_err %.3e at %.17g\n", worst, worst_at);
  printf("exp0 %.17g\n", specv::exp_nonpos(0.0));
  printf("exp_minus_inf %.17g\n", specv::exp_nonpos(-INFINITY));
  printf("exp_nan %.17g\n", specv::exp_nonpos(NAN));
  printf("exp_below %.17g\n", specv::exp_nonpos(-746.0));
  printf("exp_far_below %.17g\n", specv::exp_nonpos(-1.0e300));
  // Subnormal range: within one unit of the smallest subnormal of expl.
  double sub_err = 0.0;
  for (double a = -708.5; a > -745.5; a -= 0.37)
    sub_err = fmax(sub_err, fabs(specv::exp_nonpos(a) - static_cast<double>(expl(static_cast<long double>(a)))));
  printf("subnormal_abs_err %.3e\n", sub_err);
  return 0;
}
