// Row finalize shared by the VALU and MFMA half-steps: from a row's merged
// (max, sum) in log2 units, write the potential, the next column term of the
// row side and the residual term.
#pragma once

#include <cfloat>
#include <cmath>

#include "internal.h"

namespace sk {

struct RowFinal {
  int64_t np;            // rows
  const float* w;        // row weights [np]
  float* out;            // new potentials [np]
  const float* prev;     // previous potentials for the residual, or null
  const float* norm2;    // MFMA path: squared norms of the centred rows, else null
  double row_scale;      // s: potential += s * norm2 (MFMA path)
  float* Hnext;          // next column term of the row side, or null
  int64_t hstride;       // element stride of Hnext
  double lam_next;       // log2(e) / eps_next
  double hmul;           // Hnext = (log2 w + lam_next pot) * hmul - hnorm * norm2
  double hnorm;
  double neg_eps_ln2;    // -eps ln 2
  double inv_eps;        // 1 / eps
  double* red_part;      // residual partials
  Ctl* ctl;
};

// potential_i = -eps ln2 (mx + log2 sum) [+ s ||p_i||^2]; returns the residual
// term w_i |exp((prev_i - potential_i)/eps) - 1| (0 without prev).
__device__ __forceinline__ double finalize_row(const RowFinal& F, int64_t i, double mx, double sum,
                                               int* bad) {
  double v = F.neg_eps_ln2 * (mx + log2(sum));  // sum == 0 -> +inf
  if (F.norm2) v += F.row_scale * (double)F.norm2[i];
  const float v32 = (float)v;
  F.out[i] = v32;
  if (!isfinite(v32)) ++*bad;
  const double wi = (double)F.w[i];
  if (F.Hnext) {
    double h = (log2(wi) + (double)v32 * F.lam_next) * F.hmul;
    if (F.norm2) h -= F.hnorm * (double)F.norm2[i];
    F.Hnext[i * F.hstride] = (float)h;
  }
  if (F.prev && wi > 0.0) return wi * fabs(expm1(((double)F.prev[i] - v) * F.inv_eps));
  return 0.0;
}

// fixed-order sum of red_part[0, count) into ctl->residual
void launch_reduce(sinkhorn_problem* p, int64_t count);
// finalize description of a half-step (VALU conventions; the MFMA path adjusts it)
RowFinal make_rowfinal(sinkhorn_problem* p, const HalfStep& hs);

}  // namespace sk
