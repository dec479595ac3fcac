// Block summaries, the block-pair screen and sparse half-steps on its mask.
//
// FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport, §3.2 and §B.3:
// fine updates screen block pairs with block-level potential maxima and
// bounding boxes, keep admitted tiles in CSR form and stream them through the
// log-sum-exp; a block with no admitted tile takes a dense update; both sparse
// half-steps run on the same mask (the g-step on its transpose). §A.3: a tile
// whose mass bound is at most its threshold omits at most delta_rel a_i per
// row and delta_rel b_j per column.
//
// Blocks are B consecutive points of a side in its stored order. A tile
// (I, J) is omitted iff, in fp64 with this exact operation order and no fused
// multiply-adds,
//   gap_k = max(max(lo_Jk - hi_Ik, lo_Ik - hi_Jk), 0),
//   D     = s * ((gap_0^2 + gap_1^2) + gap_2^2),
//   (F_I + G_J) - D  <=  eps * (log(delta_rel) - max(log W_I, log W_J)),
// F/G = block maxima of the fp32 potentials, W = points * max weight of the
// block, every log taken on the host by the C library. The test is symmetric
// in I and J, so the column-major list is the same screen with the roles
// swapped. Lists are written in increasing block order: bit-exact and
// deterministic.
#include <cfloat>
#include <cmath>
#include <vector>

#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/device/device_scan.hpp>

#include "pairloop.h"

namespace sk {
namespace {

// Frame record of a side: per 16-point chunk, d rows of 16 offsets and then
// 16 weights, so that one chunk of the tile-local loop is one contiguous
// (d + 1) x 64-byte record. Slot k of point i (k = d: its weight).
__host__ __device__ __forceinline__ int64_t rec_at(int64_t i, int k, int d) {
  return (i >> 4) * ((int64_t)(d + 1) << 4) + ((int64_t)k << 4) + (i & 15);
}

// Tile-local frame, static part: one wave per block of B points; the block
// centre o = (lo + hi) / 2 per axis (fp32), every point's offset from it and
// the block radius max |y_j - o| (rounded up by 2^-20 relative), zero offsets
// on padding up to the side's stride.
template <int D>
__global__ __launch_bounds__(64) void k_frame_build(const float* __restrict__ soa, int64_t stride,
                                                    int64_t count, int32_t B, float* __restrict__ off,
                                                    float* __restrict__ ctr) {
  // off: the frame record (rec_at); this kernel writes the offset rows
  const int64_t J = blockIdx.x;
  const int64_t s = J * B;
  const int64_t e = s + B < count ? s + B : count;
  const int64_t ep = s + B < stride ? s + B : stride;
  float l[D], h[D];
#pragma unroll
  for (int k = 0; k < D; ++k) {
    l[k] = FLT_MAX;
    h[k] = -FLT_MAX;
  }
  for (int64_t i = s + threadIdx.x; i < e; i += 64)
#pragma unroll
    for (int k = 0; k < D; ++k) {
      const float v = soa[k * stride + i];
      l[k] = fminf(l[k], v);
      h[k] = fmaxf(h[k], v);
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
#pragma unroll
    for (int k = 0; k < D; ++k) {
      l[k] = fminf(l[k], __shfl_xor(l[k], o, 64));
      h[k] = fmaxf(h[k], __shfl_xor(h[k], o, 64));
    }
  float c[D];
#pragma unroll
  for (int k = 0; k < D; ++k) c[k] = 0.5f * (l[k] + h[k]);
  float r2 = 0.0f;
  for (int64_t i = s + threadIdx.x; i < ep; i += 64) {
    float q = 0.0f;
#pragma unroll
    for (int k = 0; k < D; ++k) {
      const float v = i < e ? soa[k * stride + i] - c[k] : 0.0f;
      off[rec_at(i, k, D)] = v;
      q = __builtin_fmaf(v, v, q);
    }
    r2 = fmaxf(r2, q);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) r2 = fmaxf(r2, __shfl_xor(r2, o, 64));
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 0; k < 3; ++k) ctr[J * 4 + k] = k < D ? c[k] : 0.0f;
    ctr[J * 4 + 3] = sqrtf(r2) * (1.0f + 0x1p-20f);
  }
}

// h'_j = log2 w_j + lam pot_j - kappa ||off_j||^2 in fp64 (-inf for a
// massless point).
__device__ __forceinline__ double frame_term(const float* __restrict__ rec, int32_t d,
                                             const float* __restrict__ w,
                                             const float* __restrict__ pot, int64_t i, double lam,
                                             double kappa) {
  const double wi = (double)w[i];
  if (!(wi > 0.0)) return -INFINITY;
  double q = 0.0;
  for (int k = 0; k < d; ++k) {
    const double v = (double)rec[rec_at(i, k, d)];
    q = fma(v, v, q);
  }
  return log2(wi) + lam * (double)pot[i] - kappa * q;
}

// Largest |exponent| of a pair term in the expanded form, 2 kappa |x - o| R:
// keeps 128 weighted terms of a tile far inside the fp32 range and the
// exponent's rounding near 2^-24 of it.
constexpr float kGuard = 96.0f;

// Tile-local frame, per half-step: one wave per block; m_J = max h'_j and the
// weights 2^(h'_j - m_J) (fp64 exp2, rounded once to fp32); 0 on padding and
// for every point of a block without mass (m_J = -inf). The tile-local form
// sums w'_j 2^z with |z| <= kGuard in fp32. The column with w'_j = 1 keeps
// every row's tile sum at 2^-kGuard or more, so a term that falls below the
// normal fp32 range is below 2^-30 of it and negligible; but a weight below
// 2^-126 is itself flushed or short of bits while its term can still be the
// largest of the tile, so such a block gets m_J = NaN, which sends its tiles
// to the difference form.
__global__ __launch_bounds__(64) void k_frame_weights(float* __restrict__ rec, int64_t stride,
                                                      int32_t d, const float* __restrict__ w,
                                                      const float* __restrict__ pot, int64_t count,
                                                      int32_t B, double lam, double kappa,
                                                      double* __restrict__ mx) {
  const int64_t J = blockIdx.x;
  const int64_t s = J * B;
  const int64_t e = s + B < count ? s + B : count;
  const int64_t ep = s + B < stride ? s + B : stride;
  double m = -INFINITY;
  for (int64_t i = s + threadIdx.x; i < e; i += 64)
    m = fmax(m, frame_term(rec, d, w, pot, i, lam, kappa));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
  const bool live = m > -INFINITY;
  double lo = 0.0;
  for (int64_t i = s + threadIdx.x; i < ep; i += 64) {
    const double t = (live && i < e) ? frame_term(rec, d, w, pot, i, lam, kappa) - m : -INFINITY;
    if (t > -INFINITY) lo = fmin(lo, t);
    rec[rec_at(i, d, d)] = (float)exp2(t);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lo = fmin(lo, __shfl_xor(lo, o, 64));
  if (threadIdx.x == 0) mx[J] = lo < -126.0 ? (double)NAN : m;
}

// One wave per block: min / max of each axis and the max weight.
__global__ __launch_bounds__(64) void k_block_static(const float* __restrict__ soa, int64_t stride,
                                                     int32_t d, const float* __restrict__ w,
                                                     int64_t count, int32_t B,
                                                     double* __restrict__ lo,
                                                     double* __restrict__ hi,
                                                     double* __restrict__ Wout, int64_t nb) {
  const int64_t I = blockIdx.x;
  const int64_t s = I * B;
  const int64_t e = s + B < count ? s + B : count;
  float l[3] = {FLT_MAX, FLT_MAX, FLT_MAX}, h[3] = {-FLT_MAX, -FLT_MAX, -FLT_MAX};
  float wm = -FLT_MAX;
  for (int64_t i = s + threadIdx.x; i < e; i += 64) {
    for (int k = 0; k < d; ++k) {
      const float v = soa[k * stride + i];
      l[k] = fminf(l[k], v);
      h[k] = fmaxf(h[k], v);
    }
    wm = fmaxf(wm, w[i]);
  }
  for (int o = 32; o > 0; o >>= 1) {
    for (int k = 0; k < d; ++k) {
      l[k] = fminf(l[k], __shfl_xor(l[k], o, 64));
      h[k] = fmaxf(h[k], __shfl_xor(h[k], o, 64));
    }
    wm = fmaxf(wm, __shfl_xor(wm, o, 64));
  }
  if (threadIdx.x == 0) {
    for (int k = 0; k < d; ++k) {
      lo[k * nb + I] = (double)l[k];
      hi[k * nb + I] = (double)h[k];
    }
    Wout[I] = (double)(e - s) * (double)wm;
  }
}

// Block maxima of a potential (fp32 values widened exactly).
__global__ __launch_bounds__(64) void k_block_max(const float* __restrict__ pot, int64_t count,
                                                  int32_t B, double* __restrict__ F) {
  const int64_t I = blockIdx.x;
  const int64_t s = I * B;
  const int64_t e = s + B < count ? s + B : count;
  float v = -INFINITY;
  for (int64_t i = s + threadIdx.x; i < e; i += 64) v = fmaxf(v, pot[i]);
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if (threadIdx.x == 0) F[I] = (double)v;
}

// Groups of kGrp consecutive blocks: union box, maximum potential and
// maximum log W (min / max only, so exact).
__global__ __launch_bounds__(256) void k_group_static(const double* __restrict__ lo,
                                                      const double* __restrict__ hi,
                                                      const double* __restrict__ lw, int64_t nb,
                                                      int32_t d, int64_t ng,
                                                      double* __restrict__ glo,
                                                      double* __restrict__ ghi,
                                                      double* __restrict__ glw) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= ng) return;
  const int64_t s = g * kGrp;
  const int64_t e = s + kGrp < nb ? s + kGrp : nb;
  for (int k = 0; k < d; ++k) {
    double a = INFINITY, b = -INFINITY;
    for (int64_t J = s; J < e; ++J) {
      a = fmin(a, lo[k * nb + J]);
      b = fmax(b, hi[k * nb + J]);
    }
    glo[k * ng + g] = a;
    ghi[k * ng + g] = b;
  }
  double w = -INFINITY;
  for (int64_t J = s; J < e; ++J) w = fmax(w, lw[J]);
  glw[g] = w;
}

__global__ __launch_bounds__(256) void k_group_max(const double* __restrict__ F, int64_t nb,
                                                   int64_t ng, double* __restrict__ gF) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= ng) return;
  const int64_t s = g * kGrp;
  const int64_t e = s + kGrp < nb ? s + kGrp : nb;
  double v = -INFINITY;
  for (int64_t J = s; J < e; ++J) v = fmax(v, F[J]);
  gF[g] = v;
}

struct ScreenArgs {
  const double* rlo;  // row side summaries [d][nr]
  const double* rhi;
  const double* rF;
  const double* rlw;
  int64_t nr;
  const double* clo;  // column side summaries [d][nc]
  const double* chi;
  const double* cF;
  const double* clw;
  int64_t nc;
  const double* glo;  // column groups [d][ng]
  const double* ghi;
  const double* gF;
  const double* glw;
  int64_t ng;
  double scale;
  double eps;
  double log_delta;
  int64_t* counts;    // count pass
  const int64_t* ptr; // fill pass
  int32_t* idx;
};

// Wave = row block I (its summary comes in through scalar loads). The 64
// lanes first test 64 column groups at a time; then, for each group that may
// hold an admitted tile, lane l takes member block l of the group. Admitted
// tiles are counted (FILL = false) or written in increasing block order
// (FILL = true) from wave ballots.
//
// The group test only skips work: with the union box, the largest potential
// and the largest log W of a group, (F_I + G_K) - D_IK bounds every member's
// left side from above and the right side from below (in exact arithmetic),
// so when the group's left side stays below its right side by a margin far
// above the fp64 rounding of either evaluation (1e-12 relative to the terms),
// every member is omitted by the exact test too. Members of the other groups
// take the exact per-tile test, so the lists do not depend on the grouping.
template <int D, bool FILL>
__global__ __launch_bounds__(256) void k_screen(ScreenArgs A) {
  static_assert(kGrp == 64, "one member block per lane");
  const int64_t I = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (I >= A.nr) return;  // wave-uniform; no barriers below
  const int lane = threadIdx.x & 63;
  double lo[D], hi[D];
#pragma unroll
  for (int k = 0; k < D; ++k) {
    lo[k] = A.rlo[k * A.nr + I];
    hi[k] = A.rhi[k * A.nr + I];
  }
  const double FI = A.rF[I];
  const double lwI = A.rlw[I];
  int64_t out = FILL ? A.ptr[I] : 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes < this one
  for (int64_t K0 = 0; K0 < A.ng; K0 += 64) {
    const int64_t K = K0 + lane;
    bool cand = false;
    if (K < A.ng) {
      double gacc = 0.0;
#pragma unroll
      for (int k = 0; k < D; ++k) {
        const double gap = fmax(fmax(A.glo[k * A.ng + K] - hi[k], lo[k] - A.ghi[k * A.ng + K]), 0.0);
        gacc += gap * gap;
      }
      const double Dg = A.scale * gacc;
      const double glhs = (FI + A.gF[K]) - Dg;
      const double grhs = A.eps * (A.log_delta - fmax(lwI, A.glw[K]));
      const double margin = 1e-12 * (fabs(FI) + fabs(A.gF[K]) + Dg + fabs(grhs));
      cand = !(glhs + margin <= grhs);
    }
    uint64_t m = __builtin_amdgcn_ballot_w64(cand);
    while (m) {
      const int b = __builtin_ctzll(m);
      m &= m - 1;
      const int64_t J = (K0 + b) * kGrp + lane;
      bool adm = false;
      if (J < A.nc) {
        double acc = 0.0;
#pragma unroll
        for (int k = 0; k < D; ++k) {
          const double a = __dsub_rn(A.clo[k * A.nc + J], hi[k]);
          const double c = __dsub_rn(lo[k], A.chi[k * A.nc + J]);
          const double gap = fmax(fmax(a, c), 0.0);
          const double sq = __dmul_rn(gap, gap);
          acc = k == 0 ? sq : __dadd_rn(acc, sq);
        }
        const double Dst = __dmul_rn(A.scale, acc);
        const double lhs = __dsub_rn(__dadd_rn(FI, A.cF[J]), Dst);
        const double rhs = __dmul_rn(A.eps, __dsub_rn(A.log_delta, fmax(lwI, A.clw[J])));
        adm = lhs > rhs;
      }
      const uint64_t am = __builtin_amdgcn_ballot_w64(adm);
      if (FILL && adm) A.idx[out + __builtin_popcountll(am & below)] = (int32_t)J;
      out += __builtin_popcountll(am);
    }
  }
  if (!FILL && lane == 0) A.counts[I] = out;
}

struct SparseArgs {
  const float* P;      // row side SoA [D][pstride]
  int64_t pstride;
  const float* Q;      // column side SoA [D][qstride]
  int64_t qstride;
  const float* H;      // column term of the column side
  float nkappa;
  int64_t nchunks;     // column chunks of kChunk points (all columns)
  int32_t B;           // block size (multiple of kRowsPerTile)
  const int64_t* ptr;  // [row blocks + 1]
  const int32_t* idx;  // admitted column blocks
  const float* shift_pot;  // shifted mode: previous potential of the row side
  float lam;               // log2(e) / eps
  float inv_kappa;         // 1 / kappa
  int32_t* tile_flag;      // [tiles] tiles left for the exact recompute
  const int32_t* order;    // [tiles] tile of each workgroup (heaviest first), or null: in order
  int32_t fallback;        // 1: exact recompute of the flagged tiles only
  // shifted mode, tile-local expanded form (null rec: every tile in the
  // difference form)
  const float* rec;        // column frame records: per 16-point chunk D rows of
                           // offsets from the block centre, then the weights
                           // 2^(h'_j - m_J)
  const float* ctr;        // [column blocks][4] block centre (first D slots) and radius
  const double* mx;        // [column blocks] m_J (NaN: weights beyond the fp32 range)
  float two_kappa;         // 2 kappa
  double kappa;            // kappa (fp64)
  float guard2;            // a tile takes the expanded form when every row of the
                           // wave has |x_i - o_J|^2 R_J^2 <= guard2 = (kGuard / 2 kappa)^2
  RowFinal F;
};

// v * 2^s for an fp64 exponent s clamped to [-1000, 1000]: the fraction
// through v_exp_f32, the integer part exactly by v_ldexp.
__device__ __forceinline__ float scale2(float v, double s) {
  s = fmin(fmax(s, -1000.0), 1000.0);
  const double fl = floor(s);
  return ldexpf(v * ex2((float)(s - fl)), (int)fl);
}

typedef float v4f __attribute__((ext_vector_type(4)));

// The tile (row tile against column block J, chunks c0 .. c1) in the
// tile-local expanded form, for the lane's kR rows; false (nothing done) when
// some row of the wave fails the range guard or the block's weights do not
// fit fp32 (m_J = NaN). With a_i = x_i - o_J and the
// column offsets dy_j = y_j - o_J,
//   z_ij - c_i = log2 w'_j + 2 kappa a_i . dy_j + s_i,
//   s_i = m_J - kappa ||a_i||^2 - c_i,  w'_j = 2^(h'_j - m_J),
// and the tile sum T_i = sum_j w'_j 2^(2 kappa a_i . dy_j) is then added as
// T_i 2^(s_i) to the row sum (fp64 exponent). A tile whose contribution
// passes 2^64 raises the row's shift to it first.
//
// The cross terms 2 kappa a_i . dy_j of a 16-column chunk and 16 rows are D
// v_mfma_f32_4x4x1_16b_f32 steps, one per coordinate (on this part the
// matrix and vector pipes do not overlap, so the K = 1 blocks, which spend no
// cycles on a padded coordinate, are the cheapest shape). Block b pairs the
// column quad b / 4 with the row quad b % 4; lane l = 4 b + j then holds
// row l % 16 and columns 4 (l / 16) + v in its four results v. A pair costs
// 3/4 of an MFMA cycle per lane-group, the exp2 and 1 fma. Each lane keeps
// one partial T per 16-row block; at the end of the tile the four lane groups
// of a row add their partials (two exchange steps), which leaves each lane
// the whole T of rows l and l + 64, its two rows in RowAcc.
template <int D>
__device__ __forceinline__ bool local_tile(RowAcc<true>& R, const SparseArgs& A,
                                           const float* __restrict__ rec, const float (&x)[kR][D],
                                           int lane, int64_t J, int64_t c0, int64_t c1) {
  static_assert(kR == 2 && kRowsPerTile == 128 && kChunk == 16, "layout of the exchanges below");
  constexpr int NB = kRowsPerTile / 16;
  const double mJ = A.mx[J];
  if (isnan(mJ)) return false;  // uniform: weights beyond the fp32 range
  const float* ct = A.ctr + J * 4;
  float o[D];
#pragma unroll
  for (int k = 0; k < D; ++k) o[k] = ct[k];
  const float RJ = ct[3];
  float ap[kR][D];
  double n2[kR];
  bool ok = true;
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    float q = 0.0f;
    double qd = 0.0;
#pragma unroll
    for (int k = 0; k < D; ++k) {
      const float a = x[r][k] - o[k];
      q = __builtin_fmaf(a, a, q);
      qd = fma((double)a, (double)a, qd);
      ap[r][k] = a * A.two_kappa;
    }
    n2[r] = qd;
    ok = ok && (q * (RJ * RJ) <= A.guard2);
  }
  if (__builtin_amdgcn_ballot_w64(!ok) != 0) return false;
  // row operand of block rb: 2 kappa a of row 16 rb + l % 16, which RowAcc
  // keeps in lane 16 (rb % 4) + l % 16, slot rb / 4
  float bop[NB][D];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb)
#pragma unroll
    for (int k = 0; k < D; ++k) bop[rb][k] = __shfl(ap[rb / 4][k], 16 * (rb % 4) + (lane & 15), 64);
  float T[NB];
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) T[rb] = 0.0f;
  const int g = lane >> 4;
  // one contiguous record per chunk: a uniform base and this lane's offsets
  // within it (its column 4 g + l % 4, and the weights of columns 4 g .. + 3)
  const int32_t ao = 4 * g + (lane & 3);
  const int32_t wo = D * kChunk + 4 * g;
  const int32_t nc = (int32_t)(c1 - c0);
  const float* base = rec + c0 * (D + 1) * kChunk;
  for (int32_t c = 0; c < nc; ++c, base += (D + 1) * kChunk) {
    float av[D];
#pragma unroll
    for (int k = 0; k < D; ++k) av[k] = base[ao + k * kChunk];
    const v4f wv = *(const v4f*)(base + wo);
    v4f z[NB];
#pragma unroll
    for (int rb = 0; rb < NB; ++rb)
      z[rb] = __builtin_amdgcn_mfma_f32_4x4x1f32(av[0], bop[rb][0], (v4f){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
    for (int k = 1; k < D; ++k)
#pragma unroll
      for (int rb = 0; rb < NB; ++rb) z[rb] = __builtin_amdgcn_mfma_f32_4x4x1f32(av[k], bop[rb][k], z[rb], 0, 0, 0);
#pragma unroll
    for (int rb = 0; rb < NB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) T[rb] = __builtin_fmaf(wv[v], ex2(z[rb][v]), T[rb]);
  }
  // lane groups g and g ^ 2 (lanes l and l ^ 32): keep the blocks rb with
  // rb & 2 == g & 2 and add the partner's; then g and g ^ 1 (l ^ 16): keep
  // rb & 1 == g & 1. What is left is block g (row l) and block g + 4 (row
  // l + 64).
  const bool g2 = (g & 2) != 0;
  float keep[4], send[4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      keep[2 * h + e] = g2 ? T[4 * h + 2 + e] : T[4 * h + e];
      send[2 * h + e] = g2 ? T[4 * h + e] : T[4 * h + 2 + e];
    }
#pragma unroll
  for (int t = 0; t < 4; ++t) keep[t] += __shfl_xor(send[t], 32, 64);
  const bool g1 = (g & 1) != 0;
  float Tr[kR];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float mine = g1 ? keep[2 * h + 1] : keep[2 * h];
    const float other = g1 ? keep[2 * h] : keep[2 * h + 1];
    Tr[h] = mine + __shfl_xor(other, 16, 64);
  }
  const double kd = -(double)A.nkappa;
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const float T = Tr[r];
    const double sr = mJ - A.kappa * n2[r] - R.Md[r];
    const float cval = scale2(T, sr);
    const bool big = !(cval <= kBig);
    if (__builtin_amdgcn_ballot_w64(big) != 0) {
      if (big) {
        // the row's shift moves up to this tile's scale (the same fp32 u /
        // fp64 kappa u pair as the difference form keeps)
        const double t = sr + (double)__log2f(T);
        const float un = (float)((R.Md[r] + t) / kd);
        const double Mn = kd * (double)un;
        const double delta = Mn - R.Md[r];
        R.u[r] = un;
        R.Md[r] = Mn;
        R.S[r] = scale2(R.S[r], -delta) + scale2(T, sr - delta);
      } else {
        R.S[r] += cval;
      }
    } else {
      R.S[r] += cval;
    }
  }
  return true;
}

// Workgroup = one 128-row tile of row block I = tile * 128 / B; its waves
// share out the admitted column blocks (or, for an empty list, all column
// chunks) and merge through LDS in wave order. In shifted mode a tile with a
// too-small row sum is flagged (its residual partial zeroed) and left to the
// fallback launch, which recomputes exactly the flagged tiles only. The
// workgroups take the tiles in A.order when given (the longest lists first,
// so that no long tile starts late); every tile writes only its own rows and
// residual partial, so the order leaves the results unchanged.
template <int D, bool SHIFT>
__global__ __launch_bounds__(kThreads) void k_lse_sparse(SparseArgs A, const float* __restrict__ Q,
                                                        const float* __restrict__ H,
                                                        const float* __restrict__ rec) {
  __shared__ TileLds L;
  const int64_t tile = A.order ? (int64_t)A.order[blockIdx.x] : (int64_t)blockIdx.x;
  if (tile < 0) return;                                         // an empty slot (uniform)
  if (!SHIFT && A.fallback && A.tile_flag[tile] == 0) return;  // uniform
  const int64_t I = tile * kRowsPerTile / A.B;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float x[kR][D];
  load_rows<D>(A.P, A.pstride, tile, lane, x);
  RowAcc<SHIFT> R;
  if (SHIFT) {
    float pot[kR];
    load_shift_pot(A.shift_pot, A.F.np, tile, lane, pot);
    R.init_shift(pot, A.lam, A.inv_kappa, A.nkappa);
  } else {
    R.init_exact();
  }
  const int64_t p0 = A.ptr[I];
  const int64_t p1 = A.ptr[I + 1];
  const int64_t cpb = A.B / kChunk;  // chunks per column block
  if (p1 > p0) {
    for (int64_t q = p0 + wave; q < p1; q += kW) {
      const int64_t J = A.idx[q];
      const int64_t c0 = J * cpb;
      const int64_t c1 = c0 + cpb < A.nchunks ? c0 + cpb : A.nchunks;
      if constexpr (SHIFT) {
        if (A.rec != nullptr && local_tile<D>(R, A, rec, x, lane, J, c0, c1)) continue;
      }
      pair_pass<D, SHIFT>(R, Q, H, A.qstride, A.nkappa, x, c0, c1, 1);
    }
  } else {
    pair_pass<D, SHIFT>(R, Q, H, A.qstride, A.nkappa, x, wave, A.nchunks, kW);
  }
  double mx, sum;
  merge_waves(L, wave, lane, R, mx, sum);
  if (SHIFT && needs_exact(A.F.np, tile, sum)) {
    if (threadIdx.x == 0) {
      A.tile_flag[tile] = 1;
      if (A.F.prev) A.F.red_part[tile] = 0.0;
    }
    return;
  }
  if (!SHIFT && A.fallback && threadIdx.x == 0) A.tile_flag[tile] = 0;
  finish_tile(A.F, L, tile, mx, sum);
}

// Counts entries of idx outside [0, nc) and rows whose ptr decreases.
__global__ __launch_bounds__(256) void k_check_csr(const int64_t* __restrict__ ptr, int64_t nr,
                                                   const int32_t* __restrict__ idx, int64_t nc,
                                                   uint32_t* __restrict__ bad) {
  const int64_t I = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (I >= nr) return;
  const int64_t a = ptr[I], b = ptr[I + 1];
  if (b < a || a < 0) {
    atomicAdd(bad, 1u);
    return;
  }
  for (int64_t q = a; q < b; ++q)
    if (idx[q] < 0 || idx[q] >= nc) atomicAdd(bad, 1u);
}

// number of row blocks with an empty list
__global__ __launch_bounds__(256) void k_count_empty(const int64_t* __restrict__ ptr, int64_t nr,
                                                     uint32_t* __restrict__ out) {
  const int64_t I = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (I < nr && ptr[I + 1] == ptr[I]) atomicAdd(out, 1u);
}

template <int D>
void launch_screen(hipStream_t st, const ScreenArgs& A, bool fill) {
  const dim3 grid((uint32_t)((A.nr + 3) / 4));  // a wave per row block
  if (fill)
    hipLaunchKernelGGL((k_screen<D, true>), grid, dim3(256), 0, st, A);
  else
    hipLaunchKernelGGL((k_screen<D, false>), grid, dim3(256), 0, st, A);
  SK_LAUNCH_CHECK();
}

}  // namespace

// ---------------------------------------------------------------- summaries
void BlockSummary::release() {
  dev_free(lo);
  dev_free(hi);
  dev_free(lw);
  dev_free(F);
  dev_free(glo);
  dev_free(ghi);
  dev_free(glw);
  dev_free(gF);
  lo = hi = lw = F = glo = ghi = glw = gF = nullptr;
  nb = ng = 0;
}

void block_static(sinkhorn_problem* p, const Side& s, int32_t B, BlockSummary& out) {
  out.release();
  out.nb = (s.count + B - 1) / B;
  out.B = B;
  out.lo = (double*)dev_alloc(sizeof(double) * 3 * out.nb);
  out.hi = (double*)dev_alloc(sizeof(double) * 3 * out.nb);
  out.lw = (double*)dev_alloc(sizeof(double) * out.nb);
  out.F = (double*)dev_alloc(sizeof(double) * out.nb);
  double* W = (double*)dev_alloc(sizeof(double) * out.nb);
  hipLaunchKernelGGL(k_block_static, grid1(out.nb, 64), dim3(64), 0, p->stream, s.soa,
                     s.padded, p->d, s.w, s.count, B, out.lo, out.hi, W, out.nb);
  SK_LAUNCH_CHECK();
  std::vector<double> h((size_t)out.nb);
  SK_HIP(hipMemcpyAsync(h.data(), W, sizeof(double) * out.nb, hipMemcpyDeviceToHost, p->stream));
  SK_HIP(hipStreamSynchronize(p->stream));
  dev_free(W);
  for (auto& v : h) v = v > 0.0 ? std::log(v) : -INFINITY;  // C library log
  SK_HIP(hipMemcpyAsync(out.lw, h.data(), sizeof(double) * out.nb, hipMemcpyHostToDevice, p->stream));
  out.ng = (out.nb + kGrp - 1) / kGrp;
  out.glo = (double*)dev_alloc(sizeof(double) * 3 * out.ng);
  out.ghi = (double*)dev_alloc(sizeof(double) * 3 * out.ng);
  out.glw = (double*)dev_alloc(sizeof(double) * out.ng);
  out.gF = (double*)dev_alloc(sizeof(double) * out.ng);
  hipLaunchKernelGGL(k_group_static, grid1(((out.ng + 255) / 256), 256), dim3(256), 0,
                     p->stream, out.lo, out.hi, out.lw, out.nb, p->d, out.ng, out.glo, out.ghi,
                     out.glw);
  SK_LAUNCH_CHECK();
  SK_HIP(hipStreamSynchronize(p->stream));
}

void block_potential_max(sinkhorn_problem* p, const float* pot, int64_t count, BlockSummary& s) {
  hipLaunchKernelGGL(k_block_max, grid1(s.nb, 64), dim3(64), 0, p->stream, pot, count, s.B, s.F);
  SK_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_group_max, grid1(((s.ng + 255) / 256), 256), dim3(256), 0, p->stream, s.F,
                     s.nb, s.ng, s.gF);
  SK_LAUNCH_CHECK();
}

void LocalFrame::release() {
  dev_free(rec);
  dev_free(ctr);
  dev_free(mx);
  rec = ctr = nullptr;
  mx = nullptr;
  nb = 0;
}

void frame_build(sinkhorn_problem* p, const Side& s, int32_t B, LocalFrame& out) {
  if (p->d > 3) fail(SINKHORN_ERR_UNSUPPORTED, "tile-local frames need d <= 3");
  if (B < 1) fail(SINKHORN_ERR_INVALID_ARG, "block size must be >= 1");
  out.release();
  out.nb = (s.count + B - 1) / B;
  out.B = B;
  out.stride = s.padded;
  out.rec = (float*)dev_alloc(sizeof(float) * (p->d + 1) * s.padded);
  out.ctr = (float*)dev_alloc(sizeof(float) * 4 * out.nb);
  out.mx = (double*)dev_alloc(sizeof(double) * out.nb);
  switch (p->d) {
#define SK_FRAME(Dv)                                                                              \
  case Dv:                                                                                        \
    hipLaunchKernelGGL(k_frame_build<Dv>, grid1(out.nb, 64), dim3(64), 0, p->stream, s.soa,      \
                       s.padded, s.count, B, out.rec, out.ctr);                                   \
    break;
    SK_FRAME(1)
    SK_FRAME(2)
    SK_FRAME(3)
#undef SK_FRAME
  }
  SK_LAUNCH_CHECK();
}

void frame_weights(sinkhorn_problem* p, const Side& s, const float* pot, double eps, LocalFrame& fr) {
  const double lam = kLog2e / eps;
  const double kappa = p->scale * kLog2e / eps;
  hipLaunchKernelGGL(k_frame_weights, grid1(fr.nb, 64), dim3(64), 0, p->stream, fr.rec, fr.stride,
                     p->d, s.w, pot, s.count, fr.B, lam, kappa, fr.mx);
  SK_LAUNCH_CHECK();
}

// Row-major list of the tiles admitted between `rows` and `cols` summaries.
// ptr [rows.nb + 1] is always written; idx only when the count fits cap.
// Returns the count. counts_tmp must hold rows.nb + 1 int64.
int64_t screen_tiles(sinkhorn_problem* p, const BlockSummary& rows, const BlockSummary& cols,
                     double eps, double delta_rel, int64_t* ptr, int32_t* idx, int64_t cap,
                     int64_t* counts_tmp) {
  ScreenArgs A;
  A.rlo = rows.lo;
  A.rhi = rows.hi;
  A.rF = rows.F;
  A.rlw = rows.lw;
  A.nr = rows.nb;
  A.clo = cols.lo;
  A.chi = cols.hi;
  A.cF = cols.F;
  A.clw = cols.lw;
  A.nc = cols.nb;
  A.glo = cols.glo;
  A.ghi = cols.ghi;
  A.gF = cols.gF;
  A.glw = cols.glw;
  A.ng = cols.ng;
  A.scale = p->scale;
  A.eps = eps;
  A.log_delta = std::log(delta_rel);  // C library log
  A.counts = counts_tmp;
  A.ptr = ptr;
  A.idx = idx;
  auto screen = [&](bool fill) {
    switch (p->d) {
      case 1: launch_screen<1>(p->stream, A, fill); break;
      case 2: launch_screen<2>(p->stream, A, fill); break;
      case 3: launch_screen<3>(p->stream, A, fill); break;
      default: fail(SINKHORN_ERR_UNSUPPORTED, "block screen needs d <= 3");
    }
  };
  screen(false);
  // ptr = exclusive scan of counts (counts_tmp[nb] = 0 makes ptr[nb] the total)
  zero_i32((int32_t*)(counts_tmp + rows.nb), 2, p->stream);
  size_t tb = 0;
  SK_HIP(rocprim::exclusive_scan(nullptr, tb, counts_tmp, ptr, (int64_t)0, (size_t)(rows.nb + 1),
                                 rocprim::plus<int64_t>(), p->stream));
  void* temp = dev_alloc(tb);
  const hipError_t e = rocprim::exclusive_scan(temp, tb, counts_tmp, ptr, (int64_t)0,
                                               (size_t)(rows.nb + 1), rocprim::plus<int64_t>(),
                                               p->stream);
  int64_t nnz = 0;
  if (e == hipSuccess) {
    const hipError_t c = hipMemcpyAsync(&nnz, ptr + rows.nb, sizeof(int64_t), hipMemcpyDeviceToHost,
                                        p->stream);
    const hipError_t s = hipStreamSynchronize(p->stream);
    dev_free(temp);
    check_hip(c, "hipMemcpyAsync");
    check_hip(s, "hipStreamSynchronize");
  } else {
    dev_free(temp);
    check_hip(e, "rocprim::exclusive_scan");
  }
  if (idx && nnz <= cap) screen(true);
  return nnz;
}

int64_t count_empty_rows(sinkhorn_problem* p, const int64_t* ptr, int64_t nr) {
  uint32_t* d = (uint32_t*)dev_alloc(sizeof(uint32_t));
  zero_i32((int32_t*)d, 1, p->stream);
  hipLaunchKernelGGL(k_count_empty, grid1(((nr + 255) / 256), 256), dim3(256), 0, p->stream, ptr,
                     nr, d);
  SK_LAUNCH_CHECK();
  uint32_t h = 0;
  SK_HIP(hipMemcpyAsync(&h, d, sizeof(uint32_t), hipMemcpyDeviceToHost, p->stream));
  SK_HIP(hipStreamSynchronize(p->stream));
  dev_free(d);
  return (int64_t)h;
}

// ---------------------------------------------------------------- sparse half-step
// Work of each row tile: its row block's list length in column blocks, or
// all `dense` column blocks for an empty list (a dense pass).
__global__ __launch_bounds__(256) void k_tile_work(const int64_t* __restrict__ ptr, int64_t tiles,
                                                   int32_t B, int64_t dense,
                                                   int64_t* __restrict__ work) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= tiles) return;
  const int64_t I = t * kRowsPerTile / B;
  const int64_t c = ptr[I + 1] - ptr[I];
  work[t] = c > 0 ? c : (dense > 0 ? dense : 1);
}

// Sort key of each row tile: its XCD segment (row tiles cut, in order, into
// kXcds runs of about equal total work) above the bit length of its work
// (lists within a factor of two share a length key), so that a descending
// sort puts segment 0 first and, within a segment, the longest lists first;
// counts the tiles of each segment.
constexpr int kXcds = 8;
constexpr int kLenBits = 6;
constexpr int kKeyBits = kLenBits + 3;
__global__ __launch_bounds__(256) void k_tile_keys(const int64_t* __restrict__ work,
                                                   const int64_t* __restrict__ pre, int64_t tiles,
                                                   uint32_t* __restrict__ key,
                                                   int32_t* __restrict__ val,
                                                   uint32_t* __restrict__ seg_count) {
  __shared__ uint32_t cnt[kXcds];
  if (threadIdx.x < kXcds) cnt[threadIdx.x] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < tiles) {
    const int64_t total = pre[tiles - 1];
    const int64_t before = pre[t] - work[t];
    int64_t seg = before * kXcds / total;
    if (seg > kXcds - 1) seg = kXcds - 1;
    const uint32_t len = 64u - (uint32_t)__clzll((unsigned long long)work[t]);
    key[t] = ((uint32_t)(kXcds - 1 - seg) << kLenBits) | len;
    val[t] = (int32_t)t;
    atomicAdd(&cnt[seg], 1u);
  }
  __syncthreads();
  if (threadIdx.x < kXcds && cnt[threadIdx.x]) atomicAdd(&seg_count[threadIdx.x], cnt[threadIdx.x]);
}

// Length keys alone (the fallback order when the XCD runs are very uneven).
__global__ __launch_bounds__(256) void k_len_only(const int64_t* __restrict__ work, int64_t tiles,
                                                  uint32_t* __restrict__ key,
                                                  int32_t* __restrict__ val) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= tiles) return;
  key[t] = 64u - (uint32_t)__clzll((unsigned long long)work[t]);
  val[t] = (int32_t)t;
}

struct SegTable {
  int64_t start[kXcds];
  int64_t count[kXcds];
};

// Workgroup w runs on XCD w mod kXcds (workgroups are dealt to the XCDs in
// turn), so slot w takes the (w / kXcds)-th tile of segment w mod kXcds, or
// -1 (the workgroup exits) past the segment's end.
__global__ __launch_bounds__(256) void k_xcd_slots(const int32_t* __restrict__ sorted, SegTable S,
                                                   int64_t slots, int32_t* __restrict__ out) {
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= slots) return;
  const int seg = (int)(w % kXcds);
  const int64_t i = w / kXcds;
  out[w] = i < S.count[seg] ? sorted[S.start[seg] + i] : -1;
}

// Dispatch order of the row tiles of a sparse launch. The tiles are cut, in
// row order, into one run per XCD of about equal total work, and each XCD
// takes its own run, longest lists first by powers of two and in tile order
// within a power (a stable radix sort). Neighbouring row blocks (Morton
// order) share most of their column blocks, so a run keeps its column reads
// in its own XCD's L2; the rare lists tens of times the average start first
// instead of running alone at the end. Returns the slot table (a tile index
// or -1 per workgroup) and its length in *slots; a table more than twice the
// tile count (very uneven runs) falls back to one sequence, the longest lists
// first, with *slots = tiles. Synchronizes the stream (the segment counts).
// Measured at 2^24 before the XCD runs: 798 ms per launch in tile order,
// 778 ms with the exact lengths sorted, 765 ms by powers of two.
const int32_t* heavy_first(sinkhorn_problem* p, const int64_t* ptr, int64_t tiles, int32_t B,
                           int64_t dense_work, int64_t* slots) {
  hipStream_t st = p->stream;
  if (tiles > p->order_cap) {
    SK_HIP(hipStreamSynchronize(st));
    dev_free(p->order_key);
    dev_free(p->order_val);
    p->order_key = nullptr;
    p->order_val = nullptr;
    p->order_cap = 0;
    p->order_key = (uint32_t*)dev_alloc(sizeof(uint32_t) * 2 * tiles);
    p->order_val = (int32_t*)dev_alloc(sizeof(int32_t) * 2 * tiles);
    p->order_cap = tiles;
  }
  uint32_t* kin = p->order_key;
  uint32_t* kout = p->order_key + p->order_cap;
  int32_t* vin = p->order_val;
  int32_t* vout = p->order_val + p->order_cap;
  struct Tmp {
    int64_t* work = nullptr;
    uint32_t* cnt = nullptr;
    void* scan = nullptr;
    ~Tmp() {
      dev_free(work);
      dev_free(cnt);
      dev_free(scan);
    }
  } tmp;
  tmp.work = (int64_t*)dev_alloc(sizeof(int64_t) * 2 * tiles);
  int64_t* pre = tmp.work + tiles;
  tmp.cnt = (uint32_t*)dev_alloc(sizeof(uint32_t) * kXcds);
  zero_i32((int32_t*)tmp.cnt, kXcds, st);
  hipLaunchKernelGGL(k_tile_work, grid1(((tiles + 255) / 256), 256), dim3(256), 0, st, ptr, tiles, B,
                     dense_work, tmp.work);
  SK_LAUNCH_CHECK();
  size_t scan_bytes = 0;
  SK_HIP(rocprim::inclusive_scan(nullptr, scan_bytes, tmp.work, pre, (size_t)tiles,
                                 rocprim::plus<int64_t>(), st));
  tmp.scan = dev_alloc(scan_bytes);
  SK_HIP(rocprim::inclusive_scan(tmp.scan, scan_bytes, tmp.work, pre, (size_t)tiles,
                                 rocprim::plus<int64_t>(), st));
  hipLaunchKernelGGL(k_tile_keys, grid1(((tiles + 255) / 256), 256), dim3(256), 0, st, tmp.work, pre,
                     tiles, kin, vin, tmp.cnt);
  SK_LAUNCH_CHECK();
  size_t need = 0;
  SK_HIP(rocprim::radix_sort_pairs_desc(nullptr, need, kin, kout, vin, vout, (size_t)tiles, 0,
                                        kKeyBits, st));
  if (need > p->order_temp_bytes) {
    SK_HIP(hipStreamSynchronize(st));
    dev_free(p->order_temp);
    p->order_temp = nullptr;
    p->order_temp_bytes = 0;
    p->order_temp = dev_alloc(need);
    p->order_temp_bytes = need;
  }
  SK_HIP(rocprim::radix_sort_pairs_desc(p->order_temp, need, kin, kout, vin, vout, (size_t)tiles, 0,
                                        kKeyBits, st));
  uint32_t cnt[kXcds];
  SK_HIP(hipMemcpyAsync(cnt, tmp.cnt, sizeof(cnt), hipMemcpyDeviceToHost, st));
  SK_HIP(hipStreamSynchronize(st));
  SegTable S;
  int64_t most = 0, at = 0;
  for (int k = 0; k < kXcds; ++k) {
    S.start[k] = at;
    S.count[k] = cnt[k];
    at += cnt[k];
    most = cnt[k] > most ? cnt[k] : most;
  }
  if (at != tiles) fail(SINKHORN_ERR_HIP, "tile segments do not add up");
  const int64_t n_slots = most * kXcds;
  if (n_slots > 2 * tiles) {
    // one sequence: the length keys alone, longest first (segments ignored)
    *slots = tiles;
    hipLaunchKernelGGL(k_len_only, grid1(((tiles + 255) / 256), 256), dim3(256), 0, st, tmp.work,
                       tiles, kin, vin);
    SK_LAUNCH_CHECK();
    SK_HIP(rocprim::radix_sort_pairs_desc(p->order_temp, need, kin, kout, vin, vout, (size_t)tiles, 0,
                                          kKeyBits, st));
    return vout;
  }
  // the slot table reuses the key buffers (2 * order_cap entries >= n_slots)
  int32_t* out = (int32_t*)p->order_key;
  hipLaunchKernelGGL(k_xcd_slots, grid1(((n_slots + 255) / 256), 256), dim3(256), 0, st, vout, S,
                     n_slots, out);
  SK_LAUNCH_CHECK();
  *slots = n_slots;
  return out;
}

// `tiles` workgroups: one per entry of A.order when given, else per row tile.
template <int D>
void launch_sparse(sinkhorn_problem* p, const SparseArgs& A, int64_t tiles, bool shifted,
                   const ProfEv& pe) {
  if (shifted)
    hipExtLaunchKernelGGL((k_lse_sparse<D, true>), grid1(tiles, kThreads), dim3(kThreads), 0, p->stream,
                          pe.start, pe.stop, 0, A, A.Q, A.H, A.rec);
  else
    hipExtLaunchKernelGGL((k_lse_sparse<D, false>), grid1(tiles, kThreads), dim3(kThreads), 0,
                          p->stream, pe.start, pe.stop, 0, A, A.Q, A.H, A.rec);
  SK_LAUNCH_CHECK();
}

void sparse_halfstep(sinkhorn_problem* p, const HalfStep& hs, int32_t B, const int64_t* ptr,
                     const int32_t* idx, double pairs) {
  const Side& rows = *hs.rows;
  const Side& cols = *hs.cols;
  if (B % kRowsPerTile != 0) fail(SINKHORN_ERR_UNSUPPORTED, "sparse half-steps need B a multiple of 128");
  const int64_t tiles = (rows.count + kRowsPerTile - 1) / kRowsPerTile;
  if (tiles > p->red_cap) fail(SINKHORN_ERR_HIP, "reduction buffer too small");
  const bool shifted = hs.shift_pot != nullptr;
  SparseArgs A;
  A.P = rows.soa;
  A.pstride = rows.padded;
  A.Q = cols.soa;
  A.qstride = cols.padded;
  A.H = hs.Hcols;
  const double kappa = p->scale * kLog2e / hs.eps;
  A.nkappa = (float)(-kappa);
  A.nchunks = (cols.count + kChunk - 1) / kChunk;
  A.B = B;
  A.ptr = ptr;
  A.idx = idx;
  A.shift_pot = hs.shift_pot;
  A.lam = (float)(kLog2e / hs.eps);
  A.inv_kappa = (float)(1.0 / kappa);
  A.tile_flag = p->tile_flag;
  A.fallback = 0;
  int64_t slots = tiles;
  A.order = heavy_first(p, ptr, tiles, B, (cols.count + B - 1) / B, &slots);
  A.rec = nullptr;
  A.ctr = nullptr;
  A.mx = nullptr;
  A.two_kappa = (float)(2.0 * kappa);
  A.kappa = kappa;
  {
    const double g = (double)kGuard / (2.0 * kappa);
    A.guard2 = (float)(g * g);
  }
  if (shifted && hs.frame && hs.cols_pot) {
    LocalFrame& fr = *hs.frame;
    if (fr.B != B || fr.stride != cols.padded || fr.nb != (cols.count + B - 1) / B)
      fail(SINKHORN_ERR_INVALID_ARG, "tile-local frame built for another side or block size");
    frame_weights(p, cols, hs.cols_pot, hs.eps, fr);
    A.rec = fr.rec;
    A.ctr = fr.ctr;
    A.mx = fr.mx;
  }
  A.F = make_rowfinal(p, hs);
  auto launch = [&](const SparseArgs& a, bool sh, const ProfEv& pe) {
    const int64_t wg = a.order ? slots : tiles;
    switch (p->d) {
      case 1: launch_sparse<1>(p, a, wg, sh, pe); break;
      case 2: launch_sparse<2>(p, a, wg, sh, pe); break;
      case 3: launch_sparse<3>(p, a, wg, sh, pe); break;
      default: fail(SINKHORN_ERR_UNSUPPORTED, "sparse half-steps need d <= 3");
    }
  };
  launch(A, shifted, prof_events(p, SINKHORN_PROF_SPARSE));
  prof_done(p, SINKHORN_PROF_SPARSE, pairs);
  if (shifted) {  // exact recompute of flagged tiles (the other workgroups exit at once)
    SparseArgs E = A;
    E.fallback = 1;
    E.order = nullptr;
    launch(E, false, ProfEv{});
  }
  if (A.F.prev) launch_reduce(p, tiles);
}

void check_csr(sinkhorn_problem* p, const int64_t* ptr, int64_t nr, const int32_t* idx, int64_t nc) {
  uint32_t* d = (uint32_t*)dev_alloc(sizeof(uint32_t));
  zero_i32((int32_t*)d, 1, p->stream);
  hipLaunchKernelGGL(k_check_csr, grid1(((nr + 255) / 256), 256), dim3(256), 0, p->stream, ptr,
                     nr, idx, nc, d);
  SK_LAUNCH_CHECK();
  uint32_t h = 0;
  SK_HIP(hipMemcpyAsync(&h, d, sizeof(uint32_t), hipMemcpyDeviceToHost, p->stream));
  SK_HIP(hipStreamSynchronize(p->stream));
  dev_free(d);
  if (h) fail(SINKHORN_ERR_INVALID_ARG, "tile list has out-of-range entries");
}

}  // namespace sk

using namespace sk;

namespace {

// A tile-local frame released when the call returns or throws.
struct FrameHold {
  LocalFrame f;
  ~FrameHold() { f.release(); }
};

template <class F>
int guarded(F&& body) {
  try {
    return body();
  } catch (const Failure& e) {
    set_last_error(e.msg);
    return e.code;
  } catch (...) {
    set_last_error("unexpected exception");
    return SINKHORN_ERR_HIP;
  }
}

void require(bool ok, const char* what) {
  if (!ok) fail(SINKHORN_ERR_INVALID_ARG, what);
}

}  // namespace

extern "C" {

int sinkhorn_block_screen(sinkhorn_problem* p, double eps, const float* f, const float* g,
                          int32_t B, double delta_rel, int32_t transpose, int64_t* ptr,
                          int32_t* idx, int64_t cap, int64_t* nnz_out) {
  return guarded([&] {
    require(p && f && g && ptr && nnz_out, "null pointer");
    require(std::isfinite(eps) && eps > 0.0, "eps must be finite and > 0");
    require(B >= 1 && B <= 1024, "B must be in [1, 1024]");
    require(delta_rel > 0.0 && std::isfinite(delta_rel), "delta_rel must be finite and > 0");
    require(cap >= 0, "cap must be >= 0");
    if (p->d > 3) fail(SINKHORN_ERR_UNSUPPORTED, "block screen needs d <= 3");
    BlockSummary sx, sy;
    try {
      block_static(p, p->X, B, sx);
      block_static(p, p->Y, B, sy);
      block_potential_max(p, f, p->n, sx);
      block_potential_max(p, g, p->m, sy);
      const BlockSummary& R = transpose ? sy : sx;
      const BlockSummary& C = transpose ? sx : sy;
      int64_t* tmp = (int64_t*)dev_alloc(sizeof(int64_t) * (R.nb + 1));
      int64_t nnz = 0;
      try {
        nnz = screen_tiles(p, R, C, eps, delta_rel, ptr, idx, cap, tmp);
        SK_HIP(hipStreamSynchronize(p->stream));
      } catch (...) {
        dev_free(tmp);
        throw;
      }
      dev_free(tmp);
      *nnz_out = nnz;
      sx.release();
      sy.release();
      if (!idx || nnz > cap) return nnz == 0 ? SINKHORN_OK : SINKHORN_ERR_CAPACITY;
      return SINKHORN_OK;
    } catch (...) {
      sx.release();
      sy.release();
      throw;
    }
  });
}

int sinkhorn_sparse_halfstep_f(sinkhorn_problem* p, double eps, const float* g, int32_t B,
                               const int64_t* ptr, const int32_t* idx, float* f_out,
                               const float* f_prev, double* row_l1) {
  return guarded([&] {
    require(p && g && ptr && f_out, "null pointer");
    require(std::isfinite(eps) && eps > 0.0, "eps must be finite and > 0");
    require(B >= 1 && B <= 1024, "B must be in [1, 1024]");
    if (p->d > 3) fail(SINKHORN_ERR_UNSUPPORTED, "sparse half-steps need d <= 3");
    const int64_t nr = (p->n + B - 1) / B, nc = (p->m + B - 1) / B;
    check_csr(p, ptr, nr, idx, nc);
    prep_column_term(p, p->Y, g, eps, p->Y.H);
    reset_nonfinite(p);
    HalfStep hs{&p->X, &p->Y, p->Y.H, f_out, f_prev, nullptr, eps, eps, f_prev && row_l1};
    hs.shift_pot = f_prev;  // the previous potential estimates the row shifts
    FrameHold fr;
    if (f_prev) {  // shifted mode: the tile-local frame of the columns for this call
      frame_build(p, p->Y, B, fr.f);
      hs.frame = &fr.f;
      hs.cols_pot = g;
    }
    sparse_halfstep(p, hs, B, ptr, idx, 0.0);
    double v = 0.0;
    int32_t bad = 0;
    read_reduction(p, &v, &bad);
    if (row_l1) *row_l1 = hs.residual ? v : NAN;
    if (bad) fail(SINKHORN_ERR_NONFINITE, "non-finite potential in sparse half-step");
    return SINKHORN_OK;
  });
}

int sinkhorn_sparse_halfstep_g(sinkhorn_problem* p, double eps, const float* f, int32_t B,
                               const int64_t* ptr, const int32_t* idx, float* g_out,
                               const float* g_prev, double* col_l1) {
  return guarded([&] {
    require(p && f && ptr && g_out, "null pointer");
    require(std::isfinite(eps) && eps > 0.0, "eps must be finite and > 0");
    require(B >= 1 && B <= 1024, "B must be in [1, 1024]");
    if (p->d > 3) fail(SINKHORN_ERR_UNSUPPORTED, "sparse half-steps need d <= 3");
    const int64_t nr = (p->m + B - 1) / B, nc = (p->n + B - 1) / B;
    check_csr(p, ptr, nr, idx, nc);
    prep_column_term(p, p->X, f, eps, p->X.H);
    reset_nonfinite(p);
    HalfStep hs{&p->Y, &p->X, p->X.H, g_out, g_prev, nullptr, eps, eps, g_prev && col_l1};
    hs.shift_pot = g_prev;
    FrameHold fr;
    if (g_prev) {
      frame_build(p, p->X, B, fr.f);
      hs.frame = &fr.f;
      hs.cols_pot = f;
    }
    sparse_halfstep(p, hs, B, ptr, idx, 0.0);
    double v = 0.0;
    int32_t bad = 0;
    read_reduction(p, &v, &bad);
    if (col_l1) *col_l1 = hs.residual ? v : NAN;
    if (bad) fail(SINKHORN_ERR_NONFINITE, "non-finite potential in sparse half-step");
    return SINKHORN_OK;
  });
}

}  // extern "C"
