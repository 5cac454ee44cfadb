// Per-matrix update coefficients of the MuonH step, from the three sums the
// last Newton-Schulz product reduces: ww = ||W||^2, wu = <W,u>, uu = ||u||^2.
// Host and device code (the finalise kernel runs it per matrix; a CPU test
// drives it directly).
//
// Hyperball step, Eq. (1) of "Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX
// 5090 within $5090" (arXiv HTML §3.3): u^ = u/||u||, W~ = W - eta R u^,
// W' = R W~/||W~||.  With k = eta R/||u||, W~ = W - k u, and
//   ||W~||^2 = ||W||^2 - 2 k <W,u> + k^2 ||u||^2
// so W' = k1 W - k2 u with k1 = R/||W~||, k2 = k R/||W~|| (W~ is never
// formed).  Ordinary Muon with decoupled weight decay (Eq. (3)):
// k1 = 1 - lambda eta, k2 = eta.  Effective-LR-aligned Muon (Eq. (5)):
// k1 = 1, k2 = eta_t = eta ||W||/||u||.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "../../include/muonh.h"

namespace muonh {

struct UpdateCoeffs {
  double k1, k2;     // W' = k1 W - k2 u
  double wt_norm;    // ||W~|| (Hyperball) / ||W'|| (other modes)
  double elr;        // ||W~ - W|| / ||W||
  double inner;      // <W, u^>
  double angle;      // Hyperball: atan2(eta sqrt(1 - c^2), 1 - eta c), c = <W,u^>/R
};

__host__ __device__ inline UpdateCoeffs update_coeffs(int mode, double ww, double wu, double uu,
                                                      double R, double eta, double weight_decay) {
  UpdateCoeffs o;
  const double un = sqrt(uu), wn = sqrt(ww);
  o.angle = 0.0;
  // u^ = u / ||u||; an all-zero u gives u^ = 0 (NaN still propagates: NaN != 0).
  o.inner = (un != 0.0) ? wu / un : 0.0;
  if (mode == MUONH_MODE_HYPERBALL) {
    const double k = (un != 0.0) ? eta * R / un : 0.0;   // W~ = W - k u
    // The closed form cancels when eta is near 1 and <W,u^> near R; rounding
    // can then leave it slightly below zero, so it is clamped at zero (||W~||
    // is 0 there, and W' is undefined, as in exact arithmetic).  The clamp
    // keeps a NaN (fmax would replace it by 0).
    const double wt2 = ww - 2.0 * k * wu + k * k * uu;
    o.wt_norm = sqrt(wt2 < 0.0 ? 0.0 : wt2);
    o.k1 = R / o.wt_norm;
    o.k2 = R * k / o.wt_norm;
    o.elr = k * un / wn;
    const double c = o.inner / R;
    const double cl = fmin(1.0, fmax(-1.0, c));
    o.angle = atan2(eta * sqrt(fmax(0.0, 1.0 - cl * cl)), 1.0 - eta * cl);
  } else if (mode == MUONH_MODE_MUON_WD) {
    o.k1 = 1.0 - weight_decay * eta;
    o.k2 = eta;
    const double n2 = o.k1 * o.k1 * ww - 2.0 * o.k1 * o.k2 * wu + o.k2 * o.k2 * uu;
    o.wt_norm = sqrt(n2 < 0.0 ? 0.0 : n2);
    o.elr = eta * un / wn;
  } else {
    const double eta_t = (un != 0.0) ? eta * wn / un : 0.0;
    o.k1 = 1.0;
    o.k2 = eta_t;
    const double n2 = ww - 2.0 * o.k2 * wu + o.k2 * o.k2 * uu;
    o.wt_norm = sqrt(n2 < 0.0 ? 0.0 : n2);
    o.elr = eta_t * un / wn;
  }
  return o;
}

}  // namespace muonh
