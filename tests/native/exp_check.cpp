// Host check of the kernels' fp64 exponentials (specv::exp_nonpos and the
// table form specv::exp_nonpos_tab) against long-double exp: prints, for each,
// the largest relative error over a dense grid of [-708, 0], a few special
// values and the error in the subnormal range; and the table's largest error
// in ulps against long-double 2^(j/256).
#include <math.h>
#include <stdio.h>

#include "specv_math.h"

template <typename F>
static void report(const char* prefix, F f) {
  double worst = 0.0, worst_at = 0.0;
  const int n = 4000000;
  for (int i = 0; i <= n; ++i) {
    // Dense near 0 (where most residual exponents sit) and uniform over the range.
    const double a = (i % 2) ? -708.0 * (double(i) / n) : -40.0 * (double(i) / n) * (double(i) / n);
    const long double ref = expl(static_cast<long double>(a));
    const double got = f(a);
    const double rel = static_cast<double>(fabsl((static_cast<long double>(got) - ref) / ref));
    if (rel > worst) {
      worst = rel;
      worst_at = a;
    }
  }
  printf("%smax_rel_err %.3e at %.17g\n", prefix, worst, worst_at);
  printf("%sexp0 %.17g\n", prefix, f(0.0));
  printf("%sexp_minus_inf %.17g\n", prefix, f(-INFINITY));
  printf("%sexp_nan %.17g\n", prefix, f(NAN));
  printf("%sexp_below %.17g\n", prefix, f(-746.0));
  printf("%sexp_far_below %.17g\n", prefix, f(-1.0e300));
  // Subnormal range: within a few units of the smallest subnormal of expl.
  double sub_err = 0.0;
  for (double a = -708.5; a > -745.5; a -= 0.37)
    sub_err = fmax(sub_err, fabs(f(a) - static_cast<double>(expl(static_cast<long double>(a)))));
  printf("%ssubnormal_abs_err %.3e\n", prefix, sub_err);
}

int main() {
  report("", [](double a) { return specv::exp_nonpos(a); });
  report("tab_", [](double a) { return specv::exp_nonpos_tab(a, specv::kExp2Table); });
  double worst_ulp = 0.0;
  constexpr int n = sizeof(specv::kExp2Table) / sizeof(specv::kExp2Table[0]);
  for (int j = 0; j < n; ++j) {
    const long double ref = powl(2.0L, static_cast<long double>(j) / n);
    const double v = specv::kExp2Table[j];
    const double ulp = nextafter(v, 2.0 * v) - v;
    worst_ulp = fmax(worst_ulp, static_cast<double>(fabsl(static_cast<long double>(v) - ref)) / ulp);
  }
  printf("table_max_ulp %.3f\n", worst_ulp);
  return 0;
}
