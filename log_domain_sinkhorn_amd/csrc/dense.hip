// Dense online half-step for small d: difference-form pair loop on the VALU.
//
// FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport, §2.1: a half-step
// is a tiled streaming log-sum-exp over all pairs that never stores the cost.
//
// Layout and mapping:
//   * a lane owns R = 2 rows (row side SoA, coalesced loads); the column tile
//     (coordinates and column term of kChunk points) is wave-uniform and
//     arrives through scalar loads, so the pair loop has no vector loads;
//   * a workgroup holds W = 8 waves on the SAME 128-row tile, each wave a
//     contiguous slice of the workgroup's columns; the W partials are merged
//     through LDS in wave order;
//   * when the rows alone give too few workgroups, G workgroups per tile split
//     the columns further and a merge kernel (one workgroup per tile) combines
//     their partials in split order; otherwise the workgroup finalizes in place.
//
// Two pair loops, the same sum:
//   exact   z = h_j - kappa q_ij; per 16-column chunk the running max M is
//           raised to the chunk max and S rescaled: per pair d sub, 1 mul +
//           (d-1) fma, 1 fma, 1/2 max3, 1 sub, 1 add on the VALU + 1 exp2;
//   shifted every row carries a fixed shift c = kappa u (log2 units) chosen
//           from its previous potential (c ~ LSE - 16), folded into the first
//           squared term: q' = (x - y)^2 + u, z' = h_j - kappa q' = z - c, and
//           S += exp2(z'): per pair d sub, d fma, 1 fma, 1 add + 1 exp2. A
//           chunk whose sum exceeds 2^64 (or overflows) is redone exactly for
//           the lanes concerned (the shift moves up to the chunk max); a row
//           whose final sum is below 2^-40 (shift too high: terms may have
//           underflowed) marks its tile, and the whole tile is recomputed in
//           exact mode by a second launch. The shift is kept in fp64 as the
//           exact product kappa * u of the two fp32 values the loop uses.
// Finalizing writes the potential, optionally the next column term of the row
// side and the residual terms, summed per tile and then, on request, in tile
// order by a one-block kernel. Results are bit-reproducible.
#include <cfloat>
#include <cmath>
#include <cstring>

#include "rowfinal.h"

namespace sk {
namespace {

// Base-2 exponential of the hardware (v_exp_f32): about 1 ulp; -inf gives +0.
__device__ __forceinline__ float ex2(float v) { return __builtin_amdgcn_exp2f(v); }

constexpr int kR = 2;                // rows per lane
constexpr int kW = 8;                // waves per workgroup
constexpr int kRowsPerTile = 64 * kR;
constexpr int kThreads = 64 * kW;
constexpr float kBig = 0x1p64f;      // shifted mode: redo a chunk whose sum exceeds this
constexpr double kTiny = 0x1p-40;    // shifted mode: a row sum below this is redone exactly
constexpr float kHeadroom = 16.0f;   // shift = estimated LSE - headroom (log2 units)

struct LseArgs {
  const float* P;       // row side SoA [D][pstride]
  int64_t pstride;
  const float* Q;       // column side SoA [D][qstride]
  int64_t qstride;
  const float* H;       // column term of the column side, log2 units, -inf padding
  float nkappa;         // -s log2(e) / eps
  int32_t G;            // workgroups per tile (global column splits)
  int64_t nchunks;      // column chunks of kChunk points
  int64_t cps;          // chunks per global split
  double* Mp;           // [G][np] partial shift / max (G > 1)
  float* Sp;            // [G][np] partial sum (G > 1)
  const float* shift_pot;  // shifted mode: previous potential of the row side
  float lam;               // log2(e) / eps
  float inv_kappa;         // 1 / kappa
  int32_t* tile_flag;      // [tiles] tiles to recompute exactly
  int32_t fallback;        // 1: exact recompute of the flagged tiles only (G = 1)
  RowFinal F;
};

// Keeps a wave-uniform value in a VGPR (a lane shuffle is divergent to the
// compiler), so that a VOP3 with an SGPR operand (the scalar-loaded column
// term) can use it without a copy per pair. Unlike inline asm it leaves the
// scalar loads of the column tile provably unclobbered.
__device__ __forceinline__ float in_vgpr(float s) { return __shfl(s, (int)(threadIdx.x & 63), 64); }

template <int D, bool SHIFT>
__global__ __launch_bounds__(kThreads) void k_lse_valu(LseArgs A) {
  const bool fb = A.fallback != 0;
  const int32_t G = fb ? 1 : A.G;
  const int32_t gs = (int32_t)(blockIdx.x % (uint32_t)G);
  const int64_t tile = blockIdx.x / (uint32_t)G;
  if (fb && A.tile_flag[tile] == 0) return;  // uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int lane = threadIdx.x & 63;
  const int64_t row0 = tile * kRowsPerTile + lane;
  const float nk = A.nkappa;
  const float nkv = in_vgpr(nk);
  const double kd = -(double)nk;

  float x[kR][D];
  float S[kR];
  float Mf[kR];   // exact mode: running max
  float u[kR];    // shifted mode: shift / kappa
  double Md[kR];  // shifted mode: shift = kappa * u
#pragma unroll
  for (int r = 0; r < kR; ++r) {
#pragma unroll
    for (int k = 0; k < D; ++k) x[r][k] = A.P[k * A.pstride + row0 + 64 * r];
    S[r] = 0.0f;
    Mf[r] = -FLT_MAX;
    if (SHIFT) {
      const int64_t i = row0 + 64 * r;
      const float p = i < A.F.np ? A.shift_pot[i] : 0.0f;
      const float c = -p * A.lam - kHeadroom;
      u[r] = c * A.inv_kappa;
      Md[r] = kd * (double)u[r];
    }
  }
  const float* __restrict__ Q = A.Q;
  const float* __restrict__ H = A.H;
  const int64_t qs = A.qstride;

  // this wave's slice of this workgroup's column range
  const int64_t cps = fb ? A.nchunks : A.cps;
  const int64_t g0 = (int64_t)gs * cps;
  const int64_t g1 = g0 + cps < A.nchunks ? g0 + cps : A.nchunks;
  const int64_t per = (g1 - g0 + kW - 1) / kW;
  const int64_t c0 = g0 + wave * per;
  const int64_t c1 = c0 + per < g1 ? c0 + per : g1;
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t j0 = c * kChunk;
    float yv[D][kChunk];
    float hv[kChunk];
#pragma unroll
    for (int k = 0; k < D; ++k)
#pragma unroll
      for (int jj = 0; jj < kChunk; ++jj) yv[k][jj] = Q[k * qs + j0 + jj];
#pragma unroll
    for (int jj = 0; jj < kChunk; ++jj) hv[jj] = H[j0 + jj];

#pragma unroll
    for (int r = 0; r < kR; ++r) {
      float z[kChunk];
      if (SHIFT) {
#pragma unroll
        for (int jj = 0; jj < kChunk; ++jj) {
          float dd = x[r][0] - yv[0][jj];
          float q = __builtin_fmaf(dd, dd, u[r]);
#pragma unroll
          for (int k = 1; k < D; ++k) {
            dd = x[r][k] - yv[k][jj];
            q = __builtin_fmaf(dd, dd, q);
          }
          z[jj] = __builtin_fmaf(q, nkv, hv[jj]);
        }
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
            const float un = (float)((Md[r] + (double)cm) / kd);
            const double Mn = kd * (double)un;
            delta = (float)(Mn - Md[r]);
            u[r] = un;
            Md[r] = Mn;
          }
          float acc2 = 0.0f;
#pragma unroll
          for (int jj = 0; jj < kChunk; ++jj) acc2 += ex2(z[jj] - delta);
          S[r] = big ? __builtin_fmaf(S[r], ex2(-delta), acc2) : S[r] + acc;
        } else {
          S[r] += acc;
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
        const float Mn = fmaxf(Mf[r], cm);
        float acc = 0.0f;
#pragma unroll
        for (int jj = 0; jj < kChunk; ++jj) acc += ex2(z[jj] - Mn);
        S[r] = __builtin_fmaf(S[r], ex2(Mf[r] - Mn), acc);
        Mf[r] = Mn;
      }
    }
  }
  if (!SHIFT) {
#pragma unroll
    for (int r = 0; r < kR; ++r) Md[r] = (double)Mf[r];
  }

  // ---- merge the W waves through LDS (wave order)
  __shared__ double sM[kW][kRowsPerTile];
  __shared__ float sS[kW][kRowsPerTile];
  __shared__ double sRed[kThreads];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    sM[wave][lane + 64 * r] = Md[r];
    sS[wave][lane + 64 * r] = S[r];
  }
  __syncthreads();
  double mx = -DBL_MAX, sum = 0.0;
  const int t = threadIdx.x;
  const int64_t i = tile * kRowsPerTile + t;
  const bool own = t < kRowsPerTile && i < A.F.np;
  if (t < kRowsPerTile) {
#pragma unroll
    for (int v = 0; v < kW; ++v) mx = fmax(mx, sM[v][t]);
#pragma unroll
    for (int v = 0; v < kW; ++v) sum += (double)sS[v][t] * (double)ex2((float)(sM[v][t] - mx));
  }
  if (A.G > 1 && !fb) {
    if (own) {
      A.Mp[(int64_t)gs * A.F.np + i] = mx;
      A.Sp[(int64_t)gs * A.F.np + i] = (float)sum;
    }
    return;
  }
  if (SHIFT) {
    const bool redo = __syncthreads_or(own && !(sum >= kTiny));
    if (redo) {
      if (threadIdx.x == 0) {
        A.tile_flag[tile] = 1;
        if (A.F.prev) A.F.red_part[tile] = 0.0;
      }
      return;
    }
  }
  double term = 0.0;
  int bad = 0;
  if (own) term = finalize_row(A.F, i, mx, sum, &bad);
  if (bad) atomicAdd(&A.F.ctl->nonfinite, bad);
  if (fb && threadIdx.x == 0) A.tile_flag[tile] = 0;
  if (A.F.prev) {
    sRed[threadIdx.x] = term;
    __syncthreads();
#pragma unroll
    for (int w = kThreads / 2; w > 0; w >>= 1) {
      if (threadIdx.x < w) sRed[threadIdx.x] += sRed[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) A.F.red_part[tile] = sRed[0];
  }
}

// Merge of the G global splits of each row of a 128-row tile (split order),
// then finalize; in shifted mode a tile with a too-small row sum is flagged
// for the exact recompute instead.
__global__ __launch_bounds__(kRowsPerTile) void k_merge(LseArgs A, int32_t shifted) {
  __shared__ double sRed[kRowsPerTile];
  const int64_t tile = blockIdx.x;
  const int64_t i = tile * kRowsPerTile + threadIdx.x;
  const bool own = i < A.F.np;
  double mx = -DBL_MAX, sum = 0.0;
  if (own) {
    for (int32_t t = 0; t < A.G; ++t) mx = fmax(mx, A.Mp[(int64_t)t * A.F.np + i]);
    for (int32_t t = 0; t < A.G; ++t) {
      const int64_t o = (int64_t)t * A.F.np + i;
      sum += (double)A.Sp[o] * (double)ex2((float)(A.Mp[o] - mx));
    }
  }
  if (shifted) {
    const bool redo = __syncthreads_or(own && !(sum >= kTiny));
    if (redo) {
      if (threadIdx.x == 0) {
        A.tile_flag[tile] = 1;
        if (A.F.prev) A.F.red_part[tile] = 0.0;
      }
      return;
    }
  }
  double term = 0.0;
  int bad = 0;
  if (own) term = finalize_row(A.F, i, mx, sum, &bad);
  if (bad) atomicAdd(&A.F.ctl->nonfinite, bad);
  if (A.F.prev) {
    sRed[threadIdx.x] = term;
    __syncthreads();
#pragma unroll
    for (int w = kRowsPerTile / 2; w > 0; w >>= 1) {
      if (threadIdx.x < w) sRed[threadIdx.x] += sRed[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) A.F.red_part[tile] = sRed[0];
  }
}

// Merge of G split partials for the shared merge entry point (fp32 maxima).
__global__ __launch_bounds__(256) void k_merge_f32(RowFinal F, int32_t G, const float* __restrict__ Mp,
                                                   const float* __restrict__ Sp) {
  __shared__ double sRed[256];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  double term = 0.0;
  int bad = 0;
  if (i < F.np) {
    float mx = -FLT_MAX;
    for (int32_t t = 0; t < G; ++t) mx = fmaxf(mx, Mp[(int64_t)t * F.np + i]);
    double sum = 0.0;
    for (int32_t t = 0; t < G; ++t) {
      const int64_t o = (int64_t)t * F.np + i;
      sum += (double)Sp[o] * (double)ex2(Mp[o] - mx);
    }
    term = finalize_row(F, i, (double)mx, sum, &bad);
  }
  if (bad) atomicAdd(&F.ctl->nonfinite, bad);
  if (F.prev) {
    sRed[threadIdx.x] = term;
    __syncthreads();
#pragma unroll
    for (int w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) sRed[threadIdx.x] += sRed[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) F.red_part[blockIdx.x] = sRed[0];
  }
}

// Sum of count doubles in a fixed order into ctl->residual (one block).
__global__ __launch_bounds__(256) void k_reduce(const double* __restrict__ part, int64_t count,
                                                Ctl* ctl) {
  __shared__ double sh[256];
  double acc = 0.0;
  for (int64_t k = threadIdx.x; k < count; k += 256) acc += part[k];
  sh[threadIdx.x] = acc;
  __syncthreads();
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) ctl->residual = sh[0];
}

// Column term H_j = log2 w_j + pot_j * log2(e) / eps, rounded once to fp32.
__global__ __launch_bounds__(256) void k_column_term(const float* __restrict__ w,
                                                     const float* __restrict__ pot,
                                                     int64_t count, double lam,
                                                     float* __restrict__ H) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j < count) H[j] = (float)(log2((double)w[j]) + (double)pot[j] * lam);
}

__global__ void k_reset_ctl(Ctl* ctl) {
  if (threadIdx.x == 0) {
    ctl->residual = 0.0;
    ctl->nonfinite = 0;
  }
}

struct SplitPlan {
  int32_t G;
  int64_t cps;
  int64_t nchunks;
  int64_t tiles;
};

SplitPlan plan_split(int64_t nrows, int64_t ncols) {
  SplitPlan sp;
  sp.nchunks = (ncols + kChunk - 1) / kChunk;
  sp.tiles = (nrows + kRowsPerTile - 1) / kRowsPerTile;
  // aim at >= 2048 workgroups (8 per CU, so the last round is short) with at
  // least 4 chunks per wave
  int64_t want = (2048 + sp.tiles - 1) / sp.tiles;
  const int64_t maxsplit = sp.nchunks / (4 * kW) > 1 ? sp.nchunks / (4 * kW) : 1;
  if (want > 64) want = 64;
  if (want > maxsplit) want = maxsplit;
  if (want < 1) want = 1;
  sp.cps = (sp.nchunks + want - 1) / want;
  sp.G = (int32_t)((sp.nchunks + sp.cps - 1) / sp.cps);
  return sp;
}

template <int D>
void launch_lse(sinkhorn_problem* p, const LseArgs& A, int64_t blocks, bool shifted, double pairs,
                bool timed) {
  if (timed) prof_begin(p);
  if (shifted)
    hipLaunchKernelGGL((k_lse_valu<D, true>), dim3((uint32_t)blocks), dim3(kThreads), 0, p->stream, A);
  else
    hipLaunchKernelGGL((k_lse_valu<D, false>), dim3((uint32_t)blocks), dim3(kThreads), 0, p->stream, A);
  SK_LAUNCH_CHECK();
  if (timed) prof_end(p, pairs);
}

template <int D>
void run_halfstep(sinkhorn_problem* p, LseArgs& A, const SplitPlan& sp, bool shifted, double pairs) {
  launch_lse<D>(p, A, sp.tiles * sp.G, shifted, pairs, true);
  if (sp.G > 1) {
    hipLaunchKernelGGL(k_merge, dim3((uint32_t)sp.tiles), dim3(kRowsPerTile), 0, p->stream, A,
                       (int32_t)shifted);
    SK_LAUNCH_CHECK();
  }
  if (shifted) {  // exact recompute of flagged tiles (most workgroups exit at once)
    LseArgs B = A;
    B.fallback = 1;
    launch_lse<D>(p, B, sp.tiles, false, 0.0, false);
  }
}

}  // namespace

RowFinal make_rowfinal(sinkhorn_problem* p, const HalfStep& hs) {
  RowFinal F;
  F.np = hs.rows->count;
  F.w = hs.rows->w;
  F.out = hs.pot_out;
  F.prev = hs.residual ? hs.pot_prev : nullptr;
  F.norm2 = nullptr;
  F.row_scale = 0.0;
  F.Hnext = hs.H_next;
  F.hstride = 1;
  F.lam_next = kLog2e / hs.eps_next;
  F.hmul = 1.0;
  F.hnorm = 0.0;
  F.neg_eps_ln2 = -hs.eps * kLn2;
  F.inv_eps = 1.0 / hs.eps;
  F.red_part = p->red_part;
  F.ctl = p->ctl;
  return F;
}

void launch_merge(sinkhorn_problem* p, const RowFinal& F, int32_t G, const float* Mp,
                  const float* Sp) {
  const int64_t nblocks = (F.np + 255) / 256;
  hipLaunchKernelGGL(k_merge_f32, dim3((uint32_t)nblocks), dim3(256), 0, p->stream, F, G, Mp, Sp);
  SK_LAUNCH_CHECK();
  if (F.prev) launch_reduce(p, nblocks);
}

void launch_reduce(sinkhorn_problem* p, int64_t count) {
  hipLaunchKernelGGL(k_reduce, dim3(1), dim3(256), 0, p->stream, p->red_part, count, p->ctl);
  SK_LAUNCH_CHECK();
}

int64_t row_groups(int64_t rows) {
  const int64_t tiles = (rows + kRowsPerTile - 1) / kRowsPerTile;
  const int64_t merge_blocks = (rows + 255) / 256;
  return tiles > merge_blocks ? tiles : merge_blocks;
}

int64_t partial_floats_needed(const sinkhorn_problem* p, int64_t nrows, int64_t rows_padded,
                              int64_t ncols) {
  (void)rows_padded;
  if (p->d > kMaxValuD) return mfma_partial_floats(nrows, ncols);
  const SplitPlan sp = plan_split(nrows, ncols);
  return sp.G > 1 ? 2 * (int64_t)sp.G * nrows : 1;  // fp64 maxima take two slots
}

void prep_column_term(sinkhorn_problem* p, const Side& side, const float* pot, double eps,
                      float* H) {
  if (p->d > kMaxValuD) {
    mfma_column_term(p, side, pot, eps);
    return;
  }
  const int64_t blocks = (side.count + 255) / 256;
  hipLaunchKernelGGL(k_column_term, dim3((uint32_t)blocks), dim3(256), 0, p->stream, side.w, pot,
                     side.count, kLog2e / eps, H);
  SK_LAUNCH_CHECK();
}

void dense_halfstep(sinkhorn_problem* p, const HalfStep& hs) {
  if (p->d > kMaxValuD) {
    mfma_halfstep(p, hs);
    return;
  }
  const Side& rows = *hs.rows;
  const Side& cols = *hs.cols;
  const SplitPlan sp = plan_split(rows.count, cols.count);
  // fp64 maxima: two float slots per partial
  if (sp.G > 1 && 2 * (int64_t)sp.G * rows.count > p->part_cap)
    fail(SINKHORN_ERR_HIP, "partial buffer too small");
  if (row_groups(rows.count) > p->red_cap) fail(SINKHORN_ERR_HIP, "reduction buffer too small");
  const bool shifted = hs.shift_pot != nullptr;
  LseArgs A;
  A.P = rows.soa;
  A.pstride = rows.padded;
  A.Q = cols.soa;
  A.qstride = cols.padded;
  A.H = hs.Hcols;
  const double kappa = p->scale * kLog2e / hs.eps;
  A.nkappa = (float)(-kappa);
  A.G = sp.G;
  A.nchunks = sp.nchunks;
  A.cps = sp.cps;
  A.Mp = reinterpret_cast<double*>(p->Mpart);
  A.Sp = p->Spart;
  A.shift_pot = hs.shift_pot;
  A.lam = (float)(kLog2e / hs.eps);
  A.inv_kappa = (float)(1.0 / kappa);
  A.tile_flag = p->tile_flag;
  A.fallback = 0;
  A.F = make_rowfinal(p, hs);
  const double pairs = (double)rows.count * (double)cols.count;
  switch (p->d) {
    case 1: run_halfstep<1>(p, A, sp, shifted, pairs); break;
    case 2: run_halfstep<2>(p, A, sp, shifted, pairs); break;
    case 3: run_halfstep<3>(p, A, sp, shifted, pairs); break;
    case 4: run_halfstep<4>(p, A, sp, shifted, pairs); break;
    case 5: run_halfstep<5>(p, A, sp, shifted, pairs); break;
    case 6: run_halfstep<6>(p, A, sp, shifted, pairs); break;
    case 7: run_halfstep<7>(p, A, sp, shifted, pairs); break;
    case 8: run_halfstep<8>(p, A, sp, shifted, pairs); break;
    default: fail(SINKHORN_ERR_UNSUPPORTED, "VALU half-step supports d <= 8");
  }
  if (A.F.prev) launch_reduce(p, sp.tiles);
}

void reset_nonfinite(sinkhorn_problem* p) {
  hipLaunchKernelGGL(k_reset_ctl, dim3(1), dim3(64), 0, p->stream, p->ctl);
  SK_LAUNCH_CHECK();
}

void copy_ctl(sinkhorn_problem* p) {
  SK_HIP(hipMemcpyAsync(p->host_ctl, p->ctl, sizeof(Ctl), hipMemcpyDeviceToHost, p->stream));
}

void read_reduction(sinkhorn_problem* p, double* value, int32_t* nonfinite) {
  copy_ctl(p);
  SK_HIP(hipStreamSynchronize(p->stream));
  if (value) *value = p->host_ctl->residual;
  if (nonfinite) *nonfinite = p->host_ctl->nonfinite;
}

}  // namespace sk
