// The fp64 pair loop of the dense half-step for d <= 3, and the workgroup
// merge and finalize around it.
//
// FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport, §2.1: a half-step
// is a tiled streaming log-sum-exp over pairs that never stores the cost; §A.1
// reports how the precision of the arithmetic moves the potentials. Here, in
// log2 units, z_ij = h_j - kappa ||x_i - y_j||^2 with kappa = s log2(e) / eps
// and h_j = log2 w_j + g_j log2(e) / eps the column term. Every row carries a
// shift c_i (its estimated LSE minus a small headroom), and a pair costs, in
// fp64,
//   q = (x0 - y0)^2 + c/kappa, then + (x1 - y1)^2, + (x2 - y2)^2   3 add, 3 fma
//   z' = h_j - kappa q = z_ij - c_i                                 1 fma
// and then, in fp32, S += exp2(z'): 1 cvt, 1 exp2, 1 add. z' is small for the
// pairs that carry the sum, so rounding it to fp32 for the exp2 costs little;
// the large terms h_j and c_i (hundreds of log2 units when |potential| >> eps)
// cancel in fp64. Coordinates and column terms are read as fp64 (the fp32
// inputs widened exactly), 8 columns per scalar-loaded chunk. A chunk whose
// sum passes 2^64 is redone with the shift moved up to its largest exponent;
// a row whose sum stays below 2^-40 (shift far too high) is recomputed by
// the caller in two passes: the exact row maximum, then the shifted sum.
#pragma once

#include <cfloat>
#include <cmath>

#include "pairloop.h"

namespace sk {

constexpr int kChunk64 = 8;           // columns per scalar-loaded chunk
constexpr double kHeadroom64 = 2.0;   // shift = estimated LSE - headroom (log2 units)

__device__ __forceinline__ double in_vgpr64(double s) {
  return __shfl(s, (int)(threadIdx.x & 63), 64);
}

// Row sums of kR rows relative to their shifts.
struct RowAcc64 {
  float S[kR];
  double c[kR];  // shift (log2 units)
  double u[kR];  // c / kappa (cost units)
};

__device__ __forceinline__ void init_shift64(RowAcc64& R, const double (&c)[kR], double inv_kappa) {
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    R.S[r] = 0.0f;
    R.c[r] = c[r];
    R.u[r] = c[r] * inv_kappa;
  }
}

// One wave's pass over the column chunks c0, c0 + step, ... < c1 (chunks of
// kChunk64 columns) for the lane's kR rows x: Q is the column side's fp64 SoA
// [D][qs], H its fp64 column term; both stay unwritten during the kernel
// (scalar loads).
template <int D>
__device__ __forceinline__ void pair_pass64(RowAcc64& R, const double* __restrict__ Q,
                                            const double* __restrict__ H, int64_t qs, double nk,
                                            double inv_kappa, const double (&x)[kR][D], int64_t c0,
                                            int64_t c1, int64_t step) {
  const double nkv = in_vgpr64(nk);
  const int32_t niter = c1 > c0 ? (int32_t)((c1 - c0 + step - 1) / step) : 0;
  const double* qc = Q + c0 * kChunk64;
  const double* hc = H + c0 * kChunk64;
  const int64_t adv = step * kChunk64;
  for (int32_t it = 0; it < niter; ++it, qc += adv, hc += adv) {
    double yv[D][kChunk64];
    double hv[kChunk64];
#pragma unroll
    for (int k = 0; k < D; ++k)
#pragma unroll
      for (int jj = 0; jj < kChunk64; ++jj) yv[k][jj] = qc[k * qs + jj];
#pragma unroll
    for (int jj = 0; jj < kChunk64; ++jj) hv[jj] = hc[jj];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      float z[kChunk64];
#pragma unroll
      for (int jj = 0; jj < kChunk64; ++jj) {
        double dd = x[r][0] - yv[0][jj];
        double q = __builtin_fma(dd, dd, R.u[r]);
#pragma unroll
        for (int k = 1; k < D; ++k) {
          dd = x[r][k] - yv[k][jj];
          q = __builtin_fma(dd, dd, q);
        }
        z[jj] = (float)__builtin_fma(q, nkv, hv[jj]);
      }
      float acc = ex2(z[0]);
#pragma unroll
      for (int jj = 1; jj < kChunk64; ++jj) acc += ex2(z[jj]);
      const bool big = !(acc <= kBig);
      if (__builtin_amdgcn_ballot_w64(big) != 0) {
        // redo of this chunk for the lanes whose sum ran away: the shift
        // moves up to the chunk's largest exponent
        float cm = z[0];
#pragma unroll
        for (int jj = 1; jj < kChunk64; ++jj) cm = fmaxf(cm, z[jj]);
        float delta = 0.0f;
        if (big) {
          delta = cm;
          R.c[r] += (double)cm;
          R.u[r] = R.c[r] * inv_kappa;
        }
        float acc2 = 0.0f;
#pragma unroll
        for (int jj = 0; jj < kChunk64; ++jj) acc2 += ex2(z[jj] - delta);
        R.S[r] = big ? __builtin_fmaf(R.S[r], ex2(-delta), acc2) : R.S[r] + acc;
      } else {
        R.S[r] += acc;
      }
    }
  }
}

// The shifted pass in split form: the same sum as pair_pass64 with fp32
// arithmetic whose only iterate-dependent roundings are small. The column
// term is split as h_j = Hhi_j + log2 Wlo_j with Hhi_j an integer (beyond
// 2^22 in magnitude, the fp32 rounding of h_j), and each row's shift c_i is
// an fp32 integer. Then t = Hhi_j - c_i is exact: below 2^24 in magnitude
// both are integers, and beyond, for the pairs that carry the sum, they are
// within a factor 2 of each other (Sterbenz); and
//   z_ij = RN(t - kappa32 q_ij),  q_ij = ||x_i - y_j||^2 in fp32,
//   S_i += Wlo_j exp2(z_ij).
// q and kappa32 (kappa rounded to fp32 once) depend on the clouds and eps
// only, a fixed perturbation of the cost; what depends on the iterate is
// rounded once, at the magnitude of z itself (small for the pairs that carry
// the sum) or of Wlo (near 1). Per pair: d sub, 1 mul + (d - 1) fma, 1 sub,
// 1 fma, the exp2 and 1 fma. A chunk whose sum passes 2^64 is redone with the
// shift raised by the integer part of its largest exponent.
// 16 columns per chunk. The chunk's D + 2 floats per column take 80 scalar
// registers, which caps the kernel at 3 workgroups per CU; 8-column chunks
// reach 4, but their per-chunk overhead makes the pass 3-7% slower on MI355X
constexpr int kChunkS = 16;

struct RowAccS {
  float S[kR];
  float c[kR];  // integer shift (log2 units), exact in fp32
};

template <int D>
__device__ __forceinline__ void pair_pass_split(RowAccS& R, const float* __restrict__ Q,
                                                const float* __restrict__ Hhi,
                                                const float* __restrict__ Wlo, int64_t qs, float nk,
                                                const float (&x)[kR][D], int64_t c0, int64_t c1,
                                                int64_t step) {
  const float nkv = in_vgpr(nk);
  const int32_t niter = c1 > c0 ? (int32_t)((c1 - c0 + step - 1) / step) : 0;
  const float* qc = Q + c0 * kChunkS;
  const float* hc = Hhi + c0 * kChunkS;
  const float* wc = Wlo + c0 * kChunkS;
  const int64_t adv = step * kChunkS;
  for (int32_t it = 0; it < niter; ++it, qc += adv, hc += adv, wc += adv) {
    float yv[D][kChunkS];
    float hv[kChunkS];
    float wv[kChunkS];
#pragma unroll
    for (int k = 0; k < D; ++k)
#pragma unroll
      for (int jj = 0; jj < kChunkS; ++jj) yv[k][jj] = qc[k * qs + jj];
#pragma unroll
    for (int jj = 0; jj < kChunkS; ++jj) {
      hv[jj] = hc[jj];
      wv[jj] = wc[jj];
    }
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      float z[kChunkS];
#pragma unroll
      for (int jj = 0; jj < kChunkS; ++jj) {
        float dd = x[r][0] - yv[0][jj];
        float q = dd * dd;
#pragma unroll
        for (int k = 1; k < D; ++k) {
          dd = x[r][k] - yv[k][jj];
          q = __builtin_fmaf(dd, dd, q);
        }
        z[jj] = __builtin_fmaf(q, nkv, hv[jj] - R.c[r]);
      }
      float acc = wv[0] * ex2(z[0]);
#pragma unroll
      for (int jj = 1; jj < kChunkS; ++jj) acc = __builtin_fmaf(wv[jj], ex2(z[jj]), acc);
      const bool big = !(acc <= kBig);
      if (__builtin_amdgcn_ballot_w64(big) != 0) {
        float cm = z[0];
#pragma unroll
        for (int jj = 1; jj < kChunkS; ++jj) cm = fmaxf(cm, z[jj]);
        float delta = 0.0f;
        if (big) {
          delta = floorf(cm);  // an integer: c stays exact
          R.c[r] += delta;
        }
        float acc2 = 0.0f;
#pragma unroll
        for (int jj = 0; jj < kChunkS; ++jj) acc2 = __builtin_fmaf(wv[jj], ex2(z[jj] - delta), acc2);
        R.S[r] = big ? __builtin_fmaf(R.S[r], ex2(-delta), acc2) : R.S[r] + acc;
      } else {
        R.S[r] += acc;
      }
    }
  }
}

// Row maxima of z_ij = h_j - kappa ||x_i - y_j||^2 over the chunks c0, c0 +
// step, ... < c1 (fp64), folded into mx.
template <int D>
__device__ __forceinline__ void rowmax_pass64(double (&mx)[kR], const double* __restrict__ Q,
                                              const double* __restrict__ H, int64_t qs, double nk,
                                              const double (&x)[kR][D], int64_t c0, int64_t c1,
                                              int64_t step) {
  const double nkv = in_vgpr64(nk);
  const int32_t niter = c1 > c0 ? (int32_t)((c1 - c0 + step - 1) / step) : 0;
  const double* qc = Q + c0 * kChunk64;
  const double* hc = H + c0 * kChunk64;
  const int64_t adv = step * kChunk64;
  for (int32_t it = 0; it < niter; ++it, qc += adv, hc += adv) {
    double yv[D][kChunk64];
    double hv[kChunk64];
#pragma unroll
    for (int k = 0; k < D; ++k)
#pragma unroll
      for (int jj = 0; jj < kChunk64; ++jj) yv[k][jj] = qc[k * qs + jj];
#pragma unroll
    for (int jj = 0; jj < kChunk64; ++jj) hv[jj] = hc[jj];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
#pragma unroll
      for (int jj = 0; jj < kChunk64; ++jj) {
        double dd = x[r][0] - yv[0][jj];
        double q = dd * dd;
#pragma unroll
        for (int k = 1; k < D; ++k) {
          dd = x[r][k] - yv[k][jj];
          q = __builtin_fma(dd, dd, q);
        }
        mx[r] = fmax(mx[r], __builtin_fma(q, nkv, hv[jj]));
      }
    }
  }
}

// Loads the lane's kR rows of tile `tile` from the fp64 SoA [D][ps].
template <int D>
__device__ __forceinline__ void load_rows64(const double* __restrict__ P, int64_t ps, int64_t tile,
                                            int lane, double (&x)[kR][D]) {
  const int64_t row0 = tile * kRowsPerTile + lane;
#pragma unroll
  for (int r = 0; r < kR; ++r)
#pragma unroll
    for (int k = 0; k < D; ++k) x[r][k] = P[k * ps + row0 + 64 * r];
}

// Merge of the kW waves' (shift, sum) through LDS in wave order; thread
// t < 128 gets row t of the tile (fp64 shift and sum).
__device__ __forceinline__ void merge_waves64(TileLds& L, int wave, int lane, const RowAcc64& R,
                                              double& mx, double& sum) {
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    L.M[wave][lane + 64 * r] = R.c[r];
    L.S[wave][lane + 64 * r] = R.S[r];
  }
  __syncthreads();
  mx = -DBL_MAX;
  sum = 0.0;
  const int t = threadIdx.x;
  if (t < kRowsPerTile) {
#pragma unroll
    for (int v = 0; v < kW; ++v) mx = fmax(mx, L.M[v][t]);
#pragma unroll
    for (int v = 0; v < kW; ++v) sum += (double)L.S[v][t] * (double)ex2((float)(L.M[v][t] - mx));
  }
}

// Finalize of the fp64 half-step: the potential in fp64 (and/or fp32), the
// next fp64 column term of the row side and the residual term.
struct RowFinal64 {
  int64_t np;            // rows
  const float* w;        // row weights [np]
  float* out32;          // new potentials, fp32 (nullable)
  double* out64;         // new potentials, fp64 (nullable)
  const float* prev32;   // previous potentials for the residual (nullable) ...
  const double* prev64;  // ... or these (nullable)
  double* Hnext;         // next fp64 column term of the row side (nullable)
  double lam_next;       // log2(e) / eps_next
  double neg_eps_ln2;    // -eps ln 2
  double inv_eps;        // 1 / eps
  double* red_part;      // residual partials (per tile)
  Ctl* ctl;
};

// potential_i = -eps ln2 (mx + log2 sum); returns the residual term
// w_i |exp((prev_i - potential_i)/eps) - 1| (0 without a previous potential).
__device__ __forceinline__ double finalize_row64(const RowFinal64& F, int64_t i, double mx,
                                                 double sum, int* bad) {
  const double v = F.neg_eps_ln2 * (mx + log2(sum));  // sum == 0 -> +inf
  if (F.out64) F.out64[i] = v;
  if (F.out32) F.out32[i] = (float)v;
  if (!isfinite((float)v)) ++*bad;
  const double wi = (double)F.w[i];
  if (F.Hnext) F.Hnext[i] = log2(wi) + v * F.lam_next;
  const bool has_prev = F.prev64 || F.prev32;
  if (has_prev && wi > 0.0) {
    const double pv = F.prev64 ? F.prev64[i] : (double)F.prev32[i];
    return wi * fabs(expm1((pv - v) * F.inv_eps));
  }
  return 0.0;
}

// Writes the potentials of a tile's rows (threads t < 128) and its residual
// partial (the same fixed-order tree as finish_tile).
__device__ __forceinline__ void finish_tile64(const RowFinal64& F, TileLds& L, int64_t tile,
                                              double mx, double sum) {
  const int t = threadIdx.x;
  const int64_t i = tile * kRowsPerTile + t;
  const bool own = t < kRowsPerTile && i < F.np;
  double term = 0.0;
  int bad = 0;
  if (own) term = finalize_row64(F, i, mx, sum, &bad);
  if (t >= 64 && t < kRowsPerTile) L.red[t - 64] = term;
  const int nbad = __syncthreads_count(bad);
  if (t == 0 && nbad) atomicAdd(&F.ctl->nonfinite, nbad);
  if ((F.prev64 || F.prev32) && t < 64) {
    double v = term + L.red[t];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (t == 0) F.red_part[tile] = v;
  }
}

}  // namespace sk
