// The streaming pair loop shared by the dense and the sparse half-steps, and
// the workgroup-level merge and finalize around it.
//
// FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport, §2.1: a half-step
// is a tiled streaming log-sum-exp over pairs that never stores the cost.
// Here, in log2 units, z_ij = h_j - kappa q_ij with q_ij = ||x_i - y_j||^2,
// kappa = s log2(e) / eps and h_j the column term; a row's (max, sum) pair
// gives its potential -eps ln2 (max + log2 sum).
//
// Layout: a lane owns kR = 2 rows (row side SoA, coalesced loads); the column
// tile (coordinates and column term of kChunk points) is wave-uniform and
// arrives through scalar loads, so the pair loop has no vector loads. A
// workgroup holds kW = 8 waves on the same 128-row tile.
//
// Two loops, the same sum:
//   exact   per 16-column chunk the running max M is raised to the chunk max
//           and S rescaled: per pair d sub, 1 mul + (d-1) fma, 1 fma, 1/2
//           max3, 1 sub, 1 add on the VALU + 1 exp2;
//   shifted every row carries a fixed shift c = kappa u (log2 units) chosen
//           from its previous potential (c ~ LSE - 16), folded into the first
//           squared term: q' = (x - y)^2 + u, z' = h_j - kappa q' = z - c, and
//           S += exp2(z'): per pair d sub, d fma, 1 fma, 1 add + 1 exp2. A
//           chunk whose sum exceeds 2^64 (or overflows) is redone exactly for
//           the lanes concerned (the shift moves up to the chunk max); a row
//           whose final sum is below 2^-40 (shift too high: terms may have
//           underflowed) must be recomputed in exact mode by the caller. The
//           shift is kept in fp64 as the exact product kappa * u of the two
//           fp32 values the loop uses.
#pragma once

#include <cfloat>
#include <cmath>

#include "rowfinal.h"

namespace sk {

// Base-2 exponential of the hardware (v_exp_f32): about 1 ulp; -inf gives +0.
__device__ __forceinline__ float ex2(float v) { return __builtin_amdgcn_exp2f(v); }

constexpr int kR = 2;                // rows per lane
constexpr int kW = 8;                // waves per workgroup
constexpr int kRowsPerTile = 64 * kR;
constexpr int kThreads = 64 * kW;
constexpr int kMaxSplit = 64;                       // column splits per row tile, at most
constexpr int kSplitsPerWave = kMaxSplit / kW;      // splits one merge wave folds, at most
constexpr float kBig = 0x1p64f;      // shifted mode: redo a chunk whose sum exceeds this
constexpr double kTiny = 0x1p-40;    // shifted mode: a row sum below this is redone exactly
constexpr float kHeadroom = 16.0f;   // shift = estimated LSE - headroom (log2 units)

// Keeps a wave-uniform value in a VGPR (a lane shuffle is divergent to the
// compiler), so that a VOP3 with an SGPR operand (the scalar-loaded column
// term) can use it without a copy per pair. Unlike inline asm it leaves the
// scalar loads of the column tile provably unclobbered.
__device__ __forceinline__ float in_vgpr(float s) { return __shfl(s, (int)(threadIdx.x & 63), 64); }

// Per-lane running sums of kR rows; with NA > 0 also the weighted sums
// sum_j exp2(z_ij - shift) y_jk of the first NA coordinates of the columns
// (barycentric projection), on the same scale as S.
template <bool SHIFT, int NA = 0>
struct RowAcc {
  float S[kR];    // sum, relative to the max (exact) or to the shift (shifted)
  float M[kR];    // exact: running max (log2 units)
  float u[kR];    // shifted: shift / kappa
  double Md[kR];  // shifted: shift = kappa u, exact in fp64
  float A[kR][NA > 0 ? NA : 1];

  // Exact mode: empty sums.
  __device__ __forceinline__ void init_exact() {
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      S[r] = 0.0f;
      M[r] = -FLT_MAX;
#pragma unroll
      for (int k = 0; k < NA; ++k) A[r][k] = 0.0f;
    }
  }
  // Shifted mode: shift c = -pot * lam - kHeadroom from the previous potential.
  __device__ __forceinline__ void init_shift(const float (&pot)[kR], float lam, float inv_kappa,
                                             float nkappa) {
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      S[r] = 0.0f;
#pragma unroll
      for (int k = 0; k < NA; ++k) A[r][k] = 0.0f;
      const float c = -pot[r] * lam - kHeadroom;
      u[r] = c * inv_kappa;
      Md[r] = -(double)nkappa * (double)u[r];
    }
  }
  // The row's max (exact) or shift (shifted), in log2 units.
  __device__ __forceinline__ double max_or_shift(int r) const {
    return SHIFT ? Md[r] : (double)M[r];
  }
};

// One wave's pass over column chunks c0, c0 + step, ... < c1 for the lane's
// kR rows x, accumulated into R. Q is the column side's SoA [D][qs], H its
// column term; both must stay unwritten during the kernel (scalar loads).
template <int D, bool SHIFT, int NA = 0>
__device__ __forceinline__ void pair_pass(RowAcc<SHIFT, NA>& R, const float* __restrict__ Q,
                                          const float* __restrict__ H, int64_t qs, float nk,
                                          const float (&x)[kR][D], int64_t c0, int64_t c1,
                                          int64_t step) {
  const float nkv = in_vgpr(nk);
  const double kd = -(double)nk;
  // chunk pointers advanced by a uniform stride: the addresses stay scalar
  const int32_t niter = c1 > c0 ? (int32_t)((c1 - c0 + step - 1) / step) : 0;
  const float* qc = Q + c0 * kChunk;
  const float* hc = H + c0 * kChunk;
  const int64_t adv = step * kChunk;
  for (int32_t it = 0; it < niter; ++it, qc += adv, hc += adv) {
    float yv[D][kChunk];
    float hv[kChunk];
#pragma unroll
    for (int k = 0; k < D; ++k)
#pragma unroll
      for (int jj = 0; jj < kChunk; ++jj) yv[k][jj] = qc[k * qs + jj];
#pragma unroll
    for (int jj = 0; jj < kChunk; ++jj) hv[jj] = hc[jj];

#pragma unroll
    for (int r = 0; r < kR; ++r) {
      float z[kChunk];
      if (SHIFT) {
#pragma unroll
        for (int jj = 0; jj < kChunk; ++jj) {
          float dd = x[r][0] - yv[0][jj];
          float q = __builtin_fmaf(dd, dd, R.u[r]);
#pragma unroll
          for (int k = 1; k < D; ++k) {
            dd = x[r][k] - yv[k][jj];
            q = __builtin_fmaf(dd, dd, q);
          }
          z[jj] = __builtin_fmaf(q, nkv, hv[jj]);
        }
        if constexpr (NA == 0) {
          float acc = ex2(z[0]);
#pragma unroll
          for (int jj = 1; jj < kChunk; ++jj) acc += ex2(z[jj]);
          const bool big = !(acc <= kBig);
          if (__builtin_amdgcn_ballot_w64(big) != 0) {
            // exact redo of this chunk for the lanes whose sum ran away
            float cm = z[0];
#pragma unroll
            for (int jj = 1; jj < kChunk; ++jj) cm = fmaxf(cm, z[jj]);
            float delta = 0.0f;
            if (big) {
              const float un = (float)((R.Md[r] + (double)cm) / kd);
              const double Mn = kd * (double)un;
              delta = (float)(Mn - R.Md[r]);
              R.u[r] = un;
              R.Md[r] = Mn;
            }
            float acc2 = 0.0f;
#pragma unroll
            for (int jj = 0; jj < kChunk; ++jj) acc2 += ex2(z[jj] - delta);
            R.S[r] = big ? __builtin_fmaf(R.S[r], ex2(-delta), acc2) : R.S[r] + acc;
          } else {
            R.S[r] += acc;
          }
        } else {
          // the same, keeping every term for the weighted coordinate sums
          float e[kChunk];
#pragma unroll
          for (int jj = 0; jj < kChunk; ++jj) e[jj] = ex2(z[jj]);
          float acc = e[0];
#pragma unroll
          for (int jj = 1; jj < kChunk; ++jj) acc += e[jj];
          const bool big = !(acc <= kBig);
          if (__builtin_amdgcn_ballot_w64(big) != 0) {
            float cm = z[0];
#pragma unroll
            for (int jj = 1; jj < kChunk; ++jj) cm = fmaxf(cm, z[jj]);
            float delta = 0.0f;
            if (big) {
              const float un = (float)((R.Md[r] + (double)cm) / kd);
              const double Mn = kd * (double)un;
              delta = (float)(Mn - R.Md[r]);
              R.u[r] = un;
              R.Md[r] = Mn;
              acc = 0.0f;
#pragma unroll
              for (int jj = 0; jj < kChunk; ++jj) {
                e[jj] = ex2(z[jj] - delta);
                acc += e[jj];
              }
              const float sc = ex2(-delta);
              R.S[r] *= sc;
#pragma unroll
              for (int k = 0; k < NA; ++k) R.A[r][k] *= sc;
            }
          }
          R.S[r] += acc;
#pragma unroll
          for (int k = 0; k < NA; ++k)
#pragma unroll
            for (int jj = 0; jj < kChunk; ++jj) R.A[r][k] = __builtin_fmaf(e[jj], yv[k][jj], R.A[r][k]);
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < kChunk; ++jj) {
          float dd = x[r][0] - yv[0][jj];
          float q = dd * dd;
#pragma unroll
          for (int k = 1; k < D; ++k) {
            dd = x[r][k] - yv[k][jj];
            q = __builtin_fmaf(dd, dd, q);
          }
          z[jj] = __builtin_fmaf(q, nkv, hv[jj]);
        }
        float cm = z[0];
#pragma unroll
        for (int jj = 1; jj < kChunk; ++jj) cm = fmaxf(cm, z[jj]);
        const float Mn = fmaxf(R.M[r], cm);
        if constexpr (NA == 0) {
          float acc = 0.0f;
#pragma unroll
          for (int jj = 0; jj < kChunk; ++jj) acc += ex2(z[jj] - Mn);
          R.S[r] = __builtin_fmaf(R.S[r], ex2(R.M[r] - Mn), acc);
        } else {
          const float sc = ex2(R.M[r] - Mn);
          float acc = 0.0f;
          float t[NA];
#pragma unroll
          for (int k = 0; k < NA; ++k) t[k] = R.A[r][k] * sc;
#pragma unroll
          for (int jj = 0; jj < kChunk; ++jj) {
            const float e = ex2(z[jj] - Mn);
            acc += e;
#pragma unroll
            for (int k = 0; k < NA; ++k) t[k] = __builtin_fmaf(e, yv[k][jj], t[k]);
          }
          R.S[r] = __builtin_fmaf(R.S[r], sc, acc);
#pragma unroll
          for (int k = 0; k < NA; ++k) R.A[r][k] = t[k];
        }
        R.M[r] = Mn;
      }
    }
  }
}

// Loads the lane's kR rows of tile `tile` from the row side SoA [D][ps].
template <int D>
__device__ __forceinline__ void load_rows(const float* __restrict__ P, int64_t ps, int64_t tile,
                                          int lane, float (&x)[kR][D]) {
  const int64_t row0 = tile * kRowsPerTile + lane;
#pragma unroll
  for (int r = 0; r < kR; ++r)
#pragma unroll
    for (int k = 0; k < D; ++k) x[r][k] = P[k * ps + row0 + 64 * r];
}

// Previous potentials of the lane's rows (0 past the end), for the shifts.
__device__ __forceinline__ void load_shift_pot(const float* __restrict__ pot, int64_t np,
                                               int64_t tile, int lane, float (&p)[kR]) {
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int64_t i = tile * kRowsPerTile + lane + 64 * r;
    p[r] = i < np ? pot[i] : 0.0f;
  }
}

struct TileLds {
  double M[kW][kRowsPerTile];
  float S[kW][kRowsPerTile];
  double red[kThreads];
};

// Merge of the kW waves' (max, sum) through LDS in wave order; thread t < 128
// gets row t of the tile (fp64 max and sum).
template <bool SHIFT, int NA>
__device__ __forceinline__ void merge_waves(TileLds& L, int wave, int lane, const RowAcc<SHIFT, NA>& R,
                                            double& mx, double& sum) {
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    L.M[wave][lane + 64 * r] = R.max_or_shift(r);
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

// True (workgroup-uniform) when some row of the tile has a sum below kTiny:
// its shift was too high and terms may have underflowed.
__device__ __forceinline__ bool needs_exact(int64_t np, int64_t tile, double sum) {
  const int64_t i = tile * kRowsPerTile + threadIdx.x;
  const bool own = threadIdx.x < kRowsPerTile && i < np;
  return __syncthreads_or(own && !(sum >= kTiny));
}

// Writes the potentials of a tile's rows (threads t < 128) and its residual
// partial: a fixed-order pairwise tree over the 128 row terms (rows 64..127
// fold onto 0..63 through LDS, then wave 0 halves by shuffles); the tile's
// non-finite count goes out in one atomic.
__device__ __forceinline__ void finish_tile(const RowFinal& F, TileLds& L, int64_t tile, double mx,
                                            double sum) {
  const int t = threadIdx.x;
  const int64_t i = tile * kRowsPerTile + t;
  const bool own = t < kRowsPerTile && i < F.np;
  double term = 0.0;
  int bad = 0;
  if (own) term = finalize_row(F, i, mx, sum, &bad);
  if (t >= 64 && t < kRowsPerTile) L.red[t - 64] = term;
  const int nbad = __syncthreads_count(bad);
  if (t == 0 && nbad) atomicAdd(&F.ctl->nonfinite, nbad);
  if (F.prev && t < 64) {
    double v = term + L.red[t];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (t == 0) F.red_part[tile] = v;
  }
}

}  // namespace sk
