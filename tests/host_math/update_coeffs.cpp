// CPU check of the update coefficients the finalise kernel computes
// (csrc/update_math.h), built with the host compiler alone.  The Hyperball
// step of Eq. (1) ("Puro-2B", arXiv HTML §3.3) moves W by eta R u^ and
// projects back to radius R; with ||W|| = R and c = <W,u^>/R the norm
// before projection is R sqrt(1 - 2 eta c + eta^2) exactly.  The closed form
// the kernel evaluates from (||W||^2, <W,u>, ||u||^2) must agree with that to
// rounding, never produce a NaN from its square root (eta near 1 and c near
// 1 cancel), and reach exactly the degenerate point eta = c = 1, where
// W~ = 0 and W' is undefined.
#include <cmath>
#include <cstdio>
#include <cstdlib>

#include "update_math.h"

static int failures = 0;
#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
      std::printf(__VA_ARGS__);                  \
      std::printf("\n");                         \
      ++failures;                                \
    }                                            \
  } while (0)

int main() {
  using muonh::update_coeffs;
  const double R = 37.5, U = 3.25;   // ||W|| = R, ||u|| = U (any positive scale)
  const double etas[] = {1e-6, 1e-3, 0.0104, 0.3, 0.9, 0.999999, 1.0 - 1e-9, 1.0};
  const double cs[] = {-1.0, -0.7, 0.0, 0.01, 0.5, 0.999, 1.0 - 1e-12, 1.0};
  for (double eta : etas)
    for (double c : cs) {
      const double ww = R * R, uu = U * U, wu = c * R * U;
      const auto o = update_coeffs(MUONH_MODE_HYPERBALL, ww, wu, uu, R, eta, 0.0);
      const long double exact =
          (long double)R * sqrtl(fmaxl(0.0L, 1.0L - 2.0L * eta * c + (long double)eta * eta));
      CHECK(!std::isnan(o.wt_norm), "eta %.17g c %.17g: NaN norm", eta, c);
      // rounding of the three-term sum: a few ulp of R^2, i.e. about 1e-8 R
      // after the square root at worst
      CHECK(std::fabs(o.wt_norm - (double)exact) <= 1e-7 * R, "eta %.17g c %.17g: %.17g vs %.17Lg",
            eta, c, o.wt_norm, exact);
      CHECK(std::fabs(o.elr - eta) <= 1e-15 * (1.0 + eta), "eta %.17g: elr %.17g", eta, o.elr);
      CHECK(std::fabs(o.inner - c * R) <= 1e-13 * R, "c %.17g: inner %.17g", c, o.inner);
      // the angle of the closed form, from the c the kernel recovers (c
      // itself comes back to rounding: near c = 1 the angle is steep in c)
      const double cr = std::fmin(1.0, std::fmax(-1.0, o.inner / R));
      const double ang = std::atan2(eta * std::sqrt(std::fmax(0.0, 1.0 - cr * cr)), 1.0 - eta * cr);
      CHECK(std::fabs(o.angle - ang) <= 1e-15, "eta %.17g c %.17g: angle", eta, c);
      // Away from W~ = 0 the projection lands on the sphere to rounding; as
      // ||W~|| -> 0 its relative accuracy degrades like 1e-16 R^2/||W~||^2
      // (the cancellation above), which the absolute check covers.
      if (exact > 1e-3L * R) {
        // W' = k1 W - k2 u lands on the sphere: ||W'||^2 = k1^2 R^2 - 2 k1 k2 <W,u> + k2^2 U^2
        const double n2 = o.k1 * o.k1 * ww - 2.0 * o.k1 * o.k2 * wu + o.k2 * o.k2 * uu;
        CHECK(std::fabs(std::sqrt(n2) / R - 1.0) <= 1e-9, "eta %.17g c %.17g: |W'|/R %.17g", eta, c,
              std::sqrt(n2) / R);
      }
    }
  // eta = 1 with u parallel to W: W~ = W - R u^ = 0 exactly.
  {
    const auto o = update_coeffs(MUONH_MODE_HYPERBALL, R * R, R * U, U * U, R, 1.0, 0.0);
    CHECK(o.wt_norm == 0.0, "eta = c = 1: norm %.17g", o.wt_norm);
    CHECK(std::isinf(o.k1), "eta = c = 1: W' is undefined (k1 = R / 0)");
  }
  // a zero update: projection only (k2 = 0, k1 = R/||W||)
  {
    const auto o = update_coeffs(MUONH_MODE_HYPERBALL, 4.0 * R * R, 0.0, 0.0, R, 0.02, 0.0);
    CHECK(o.k2 == 0.0 && std::fabs(o.k1 - 0.5) <= 1e-15 && o.inner == 0.0, "zero update");
  }
  // a NaN sum propagates
  {
    const auto o = update_coeffs(MUONH_MODE_HYPERBALL, R * R, NAN, U * U, R, 0.02, 0.0);
    CHECK(std::isnan(o.k1) && std::isnan(o.k2) && std::isnan(o.wt_norm), "NaN propagates");
  }
  // Eq. (3): k1 = 1 - lambda eta, k2 = eta; Eq. (5): displacement eta ||W||
  {
    const auto a = update_coeffs(MUONH_MODE_MUON_WD, R * R, 0.3 * R * U, U * U, R, 0.02, 0.1);
    CHECK(a.k1 == 1.0 - 0.1 * 0.02 && a.k2 == 0.02, "Eq. (3) coefficients");
    const auto b = update_coeffs(MUONH_MODE_ELR_ALIGNED, R * R, 0.3 * R * U, U * U, R, 0.02, 0.0);
    CHECK(b.k1 == 1.0 && std::fabs(b.k2 * U - 0.02 * R) <= 1e-15 * R, "Eq. (5) step");
    CHECK(std::fabs(b.elr - 0.02) <= 1e-15, "Eq. (5) effective LR");
    const auto z = update_coeffs(MUONH_MODE_ELR_ALIGNED, R * R, 0.0, 0.0, R, 0.02, 0.0);
    CHECK(z.k2 == 0.0 && z.k1 == 1.0, "Eq. (5) with u = 0 leaves W unchanged");
  }
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("update coefficients: all checks passed\n");
  return 0;
}
