// Dense online half-step for small d: difference-form pair loop on the VALU.
//
// FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport, §2.1: a half-step
// is a tiled streaming log-sum-exp over all pairs that never stores the cost.
//
// Layout and mapping:
//   * a lane owns R = 2 rows (row side SoA, coalesced loads); the column tile
//     (coordinates and column term of kChunk points) is wave-uniform and
//     arrives through scalar loads, so the pair loop has no vector loads;
//   * a workgroup holds W = 8 waves on the SAME 128-row tile, the waves taking
//     the chunks of its column range in turn; their partials are merged
//     through LDS in wave order;
//   * G workgroups per tile split the columns (G a multiple of 8 when the
//     columns outgrow an XCD's L2: workgroups are dealt to the 8 XCDs in turn,
//     so each XCD then streams only its own splits), and a merge kernel (one
//     workgroup per tile) combines their partials in split order and
//     finalizes.
//
// The pair loop itself (exact and shifted) is in pairloop.h.
// Finalizing writes the potential, optionally the next column term of the row
// side and the residual terms, summed per tile and then, on request, in tile
// order by a one-block kernel. Results are bit-reproducible.
#include <cfloat>
#include <cmath>
#include <cstring>

#include "pairloop.h"

namespace sk {
namespace {

struct LseArgs {
  const float* P;       // row side SoA [D][pstride]
  int64_t pstride;
  const float* Q;       // column side SoA [D][qstride]
  int64_t qstride;
  const float* H;       // column term of the column side, log2 units, -inf padding
  float nkappa;         // -s log2(e) / eps
  int64_t nchunks;      // column chunks of kChunk points
  int64_t tiles;        // row tiles of kRowsPerTile rows
  int32_t G;            // column splits (a power of two): workgroup w works on tile w / G, split w % G
  int32_t glog;         // log2 G
  int64_t cps;          // chunks per split
  double* Mp;           // [G][np] partial shift / max
  float* Sp;            // [G][np] partial sum
  const float* shift_pot;  // shifted mode: previous potential of the row side
  float lam;               // log2(e) / eps
  float inv_kappa;         // 1 / kappa
  RowFinal F;
};


// Exact recompute of a whole tile (all columns) by the kW waves of the
// workgroup: the fallback of shifted mode when a row's shift was too high.
template <int D>
__device__ void exact_tile(const LseArgs& A, TileLds& L, int64_t tile, double& mx, double& sum) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float x[kR][D];
  load_rows<D>(A.P, A.pstride, tile, lane, x);
  RowAcc<false> R;
  R.init_exact();
  pair_pass<D, false>(R, A.Q, A.H, A.qstride, A.nkappa, x, wave, A.nchunks, kW);
  __syncthreads();  // LDS reuse
  merge_waves(L, wave, lane, R, mx, sum);
}

// Q, H, Mp and Sp come as separate no-alias arguments, so the column data
// provably stays unclobbered by the partial stores and arrives through scalar
// loads.
template <int D, bool SHIFT>
__global__ __launch_bounds__(kThreads) void k_lse_valu(LseArgs A, const float* __restrict__ Q,
                                                      const float* __restrict__ H,
                                                      double* __restrict__ Mp,
                                                      float* __restrict__ Sp) {
  __shared__ TileLds L;
  const int32_t gs = (int32_t)(blockIdx.x & (uint32_t)(A.G - 1));
  const int64_t tile = blockIdx.x >> A.glog;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
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
  const int64_t g0 = (int64_t)gs * A.cps;
  const int64_t g1 = g0 + A.cps < A.nchunks ? g0 + A.cps : A.nchunks;
  pair_pass<D, SHIFT>(R, Q, H, A.qstride, A.nkappa, x, g0 + wave, g1, kW);
  double mx, sum;
  merge_waves(L, wave, lane, R, mx, sum);
  const int64_t i = tile * kRowsPerTile + threadIdx.x;
  if (threadIdx.x < kRowsPerTile && i < A.F.np) {
    Mp[(int64_t)gs * A.F.np + i] = mx;
    Sp[(int64_t)gs * A.F.np + i] = (float)sum;
  }
}

// Merge of the G splits of each row of a 128-row tile, then finalize: wave w
// combines splits w, w + 8, ... of the lane's rows (fp64), and the 8 wave
// results are combined through LDS in wave order. In shifted mode a tile with
// a too-small row sum is recomputed exactly by the whole workgroup first.
template <int D>
__global__ __launch_bounds__(kThreads) void k_merge(LseArgs A, int32_t shifted) {
  __shared__ TileLds L;
  __shared__ double sS[kW][kRowsPerTile];
  const int64_t tile = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t np = A.F.np;
  // all of the lane's partials in one round of loads (G <= kMaxSplit)
  double mv[kR][kSplitsPerWave];
  float sv[kR][kSplitsPerWave];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int64_t i = tile * kRowsPerTile + lane + 64 * r;
#pragma unroll
    for (int q = 0; q < kSplitsPerWave; ++q) {
      const int32_t t = wave + kW * q;
      mv[r][q] = -DBL_MAX;
      sv[r][q] = 0.0f;
      if (i < np && t < A.G) {
        const int64_t o = (int64_t)t * np + i;
        mv[r][q] = A.Mp[o];
        sv[r][q] = A.Sp[o];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    double m = -DBL_MAX, acc = 0.0;
#pragma unroll
    for (int q = 0; q < kSplitsPerWave; ++q) m = fmax(m, mv[r][q]);
#pragma unroll
    for (int q = 0; q < kSplitsPerWave; ++q)
      if (wave + kW * q < A.G) acc += (double)sv[r][q] * (double)ex2((float)(mv[r][q] - m));
    L.M[wave][lane + 64 * r] = m;
    sS[wave][lane + 64 * r] = acc;
  }
  __syncthreads();
  double mx = -DBL_MAX, sum = 0.0;
  const int t = threadIdx.x;
  if (t < kRowsPerTile) {
#pragma unroll
    for (int v = 0; v < kW; ++v) mx = fmax(mx, L.M[v][t]);
#pragma unroll
    for (int v = 0; v < kW; ++v) sum += sS[v][t] * (double)ex2((float)(L.M[v][t] - mx));
  }
  if (shifted && needs_exact(A.F.np, tile, sum)) exact_tile<D>(A, L, tile, mx, sum);
  finish_tile(A.F, L, tile, mx, sum);
}

// Sum of count doubles in a fixed order into ctl->residual (one block):
// thread t adds part[t], part[t + 256], ...; the 256 sums are then halved
// pairwise (t + 128 onto t, ..., 1 onto 0; the last six steps by shuffles
// within wave 0). The result and the non-finite count also go to the
// host-mapped mirror, so the host reads them after an event without a copy.
__global__ __launch_bounds__(256) void k_reduce(const double* __restrict__ part, int64_t count,
                                                Ctl* ctl, Ctl* host) {
  __shared__ double sh[256];
  const int t = threadIdx.x;
  double acc = 0.0;
  for (int64_t k = t; k < count; k += 256) acc += part[k];
  sh[t] = acc;
  __syncthreads();
  if (t < 128) sh[t] += sh[t + 128];
  __syncthreads();
  if (t < 64) {
    double v = sh[t] + sh[t + 64];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (t == 0) {
      ctl->residual = v;
      __hip_atomic_store(&host->residual, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(&host->nonfinite, ctl->nonfinite, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
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

// Workgroups of the pair kernel resident on the whole chip at once. The
// per-CU figure is queried once per instantiation (a static initialised
// under the language's once-only guarantee, so handles on other host
// threads may ask concurrently; a failed query leaves it to the next call).
template <int D>
int64_t resident_slots(sinkhorn_problem* p) {
  static const int per_cu = [] {
    int nb = 0;
    SK_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_lse_valu<D, true>, kThreads, 0));
    return nb > 0 ? nb : 1;
  }();
  return (int64_t)per_cu * p->num_cu;
}

constexpr int64_t kXcds = 8;
constexpr int64_t kL2Slice = 2 << 20;  // column bytes an XCD's L2 keeps comfortably

// Column splits G per row tile (plan_dense_split: a power of two, at least 4
// chunks per wave, about three rounds of the resident workgroups, a multiple
// of the 8 XCDs when the columns outgrow an XCD's L2, and a grid that fits
// one dispatch). Trailing splits may be empty; they leave an empty partial.
int64_t plan_split(LseArgs& A, int64_t nrows, int64_t ncols, int64_t slots, int d) {
  const DenseSplit s = plan_dense_split(nrows, ncols, slots, d, kChunk, kRowsPerTile, kW, kThreads,
                                        kMaxSplit, kXcds, kL2Slice);
  if (!s.ok) fail(SINKHORN_ERR_UNSUPPORTED, "too many row tiles for one dispatch");
  A.nchunks = s.nchunks;
  A.tiles = s.tiles;
  A.G = s.G;
  A.glog = s.glog;
  A.cps = s.cps;
  return A.tiles * A.G;
}

template <int D>
void launch_lse(sinkhorn_problem* p, const LseArgs& A, int64_t blocks, bool shifted, double pairs) {
  const int32_t kind = shifted ? SINKHORN_PROF_DENSE : SINKHORN_PROF_DENSE_EXACT;
  const ProfEv pe = prof_events(p, kind);
  if (shifted)
    hipExtLaunchKernelGGL((k_lse_valu<D, true>), grid1(blocks, kThreads), dim3(kThreads), 0, p->stream,
                          pe.start, pe.stop, 0, A, A.Q, A.H, A.Mp, A.Sp);
  else
    hipExtLaunchKernelGGL((k_lse_valu<D, false>), grid1(blocks, kThreads), dim3(kThreads), 0, p->stream,
                          pe.start, pe.stop, 0, A, A.Q, A.H, A.Mp, A.Sp);
  SK_LAUNCH_CHECK();
  prof_done(p, kind, pairs);
}

template <int D>
void run_halfstep(sinkhorn_problem* p, const HalfStep& hs, LseArgs& A, bool shifted, double pairs) {
  const int64_t blocks = plan_split(A, hs.rows->count, hs.cols->count, resident_slots<D>(p), D);
  // fp64 maxima: two float slots per partial
  if (2 * (int64_t)A.G * hs.rows->count > p->part_cap)
    fail(SINKHORN_ERR_HIP, "partial buffer too small");
  if (row_groups(hs.rows->count) > p->red_cap) fail(SINKHORN_ERR_HIP, "reduction buffer too small");
  launch_lse<D>(p, A, blocks, shifted, pairs);
  hipLaunchKernelGGL(k_merge<D>, grid1(A.tiles, kThreads), dim3(kThreads), 0, p->stream, A,
                     (int32_t)shifted);
  SK_LAUNCH_CHECK();
  if (A.F.prev) launch_reduce(p, A.tiles);
}

template <int D>
int64_t split_floats(sinkhorn_problem* p, int64_t nrows, int64_t ncols) {
  LseArgs A;
  plan_split(A, nrows, ncols, resident_slots<D>(p), D);
  return 2 * (int64_t)A.G * nrows;  // fp64 maxima take two slots
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


void launch_reduce(sinkhorn_problem* p, int64_t count) {
  hipLaunchKernelGGL(k_reduce, dim3(1), dim3(256), 0, p->stream, p->red_part, count, p->ctl,
                     p->host_ctl_dev);
  SK_LAUNCH_CHECK();
}

SplitInfo dense_split(sinkhorn_problem* p, int64_t nrows, int64_t ncols) {
  LseArgs A;
  switch (p->d) {
    case 1: plan_split(A, nrows, ncols, resident_slots<1>(p), 1); break;
    case 2: plan_split(A, nrows, ncols, resident_slots<2>(p), 2); break;
    case 3: plan_split(A, nrows, ncols, resident_slots<3>(p), 3); break;
    case 4: plan_split(A, nrows, ncols, resident_slots<4>(p), 4); break;
    case 5: plan_split(A, nrows, ncols, resident_slots<5>(p), 5); break;
    case 6: plan_split(A, nrows, ncols, resident_slots<6>(p), 6); break;
    case 7: plan_split(A, nrows, ncols, resident_slots<7>(p), 7); break;
    case 8: plan_split(A, nrows, ncols, resident_slots<8>(p), 8); break;
    default: fail(SINKHORN_ERR_UNSUPPORTED, "VALU kernels support d <= 8");
  }
  return SplitInfo{A.G, A.glog, A.cps, A.nchunks, A.tiles};
}

int64_t row_groups(int64_t rows) {
  const int64_t tiles = (rows + kRowsPerTile - 1) / kRowsPerTile;
  const int64_t merge_blocks = (rows + 255) / 256;
  return tiles > merge_blocks ? tiles : merge_blocks;
}

int64_t partial_floats_needed(sinkhorn_problem* p, int64_t nrows, int64_t rows_padded,
                              int64_t ncols) {
  (void)rows_padded;
  switch (p->d) {
    case 1: return split_floats<1>(p, nrows, ncols);
    case 2: return split_floats<2>(p, nrows, ncols);
    case 3: return split_floats<3>(p, nrows, ncols);
    case 4: return split_floats<4>(p, nrows, ncols);
    case 5: return split_floats<5>(p, nrows, ncols);
    case 6: return split_floats<6>(p, nrows, ncols);
    case 7: return split_floats<7>(p, nrows, ncols);
    case 8: return split_floats<8>(p, nrows, ncols);
    default: return mfma_partial_floats(p, nrows, ncols);
  }
}

void prep_column_term(sinkhorn_problem* p, const Side& side, const float* pot, double eps,
                      float* H) {
  if (p->d > kMaxValuD) {
    mfma_column_term(p, side, pot, eps);
    return;
  }
  const int64_t blocks = (side.count + 255) / 256;
  hipLaunchKernelGGL(k_column_term, grid1(blocks, 256), dim3(256), 0, p->stream, side.w, pot,
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
  const bool shifted = hs.shift_pot != nullptr;
  LseArgs A;
  A.P = rows.soa;
  A.pstride = rows.padded;
  A.Q = cols.soa;
  A.qstride = cols.padded;
  A.H = hs.Hcols;
  const double kappa = p->scale * kLog2e / hs.eps;
  A.nkappa = (float)(-kappa);
  A.Mp = reinterpret_cast<double*>(p->Mpart);
  A.Sp = p->Spart;
  A.shift_pot = hs.shift_pot;
  A.lam = (float)(kLog2e / hs.eps);
  A.inv_kappa = (float)(1.0 / kappa);
  A.F = make_rowfinal(p, hs);
  const double pairs = (double)rows.count * (double)cols.count;
  switch (p->d) {
    case 1: run_halfstep<1>(p, hs, A, shifted, pairs); break;
    case 2: run_halfstep<2>(p, hs, A, shifted, pairs); break;
    case 3: run_halfstep<3>(p, hs, A, shifted, pairs); break;
    case 4: run_halfstep<4>(p, hs, A, shifted, pairs); break;
    case 5: run_halfstep<5>(p, hs, A, shifted, pairs); break;
    case 6: run_halfstep<6>(p, hs, A, shifted, pairs); break;
    case 7: run_halfstep<7>(p, hs, A, shifted, pairs); break;
    case 8: run_halfstep<8>(p, hs, A, shifted, pairs); break;
    default: fail(SINKHORN_ERR_UNSUPPORTED, "VALU half-step supports d <= 8");
  }
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
