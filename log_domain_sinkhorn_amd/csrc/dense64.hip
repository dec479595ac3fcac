// Dense online half-step for d <= 3 with fp64 solve state (pairloop64.h).
//
// FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport, §2.1: the
// streaming tiled log-sum-exp over all pairs; §A.1 on how the precision of
// the arithmetic moves the potentials. When |potential| >> eps (eps = 1e-4
// with potentials of a few hundredths), the column term h_j and the row shift
// are hundreds of log2 units, and an fp32 rounding of either, or of the
// potentials themselves, moves each half-step by ~1e-5 eps in a way that
// depends on the iterate; Sinkhorn's slow modes integrate that over thousands
// of iterations. Here the potentials, the column terms and the row shifts are
// fp64. The shifted pass (pair_pass_split) keeps them exact in fp32 as an
// integer plus a small remainder, so its pair arithmetic is fp32 with only
// small iterate-dependent roundings; the exact two-pass recompute is fp64
// throughout.
//
// Mapping as the fp32 kernels (dense.hip): a lane owns 2 rows, a workgroup of
// 8 waves shares a 128-row tile, G workgroups per tile split the columns
// (a power of two, XCD-aligned when the columns outgrow an XCD's L2), and a
// merge kernel folds the split partials (fp64 shift, fp32 sum) in split order
// and finalizes. Calls without a previous potential, and tiles whose shift
// was far too high, run the exact two-pass form (row maxima, then the
// shifted sum) in one workgroup per tile. Results are bit-reproducible.
#include <cfloat>
#include <cmath>

#include "pairloop64.h"

namespace sk {
namespace {

struct LseArgs64 {
  const double* P;      // row side fp64 SoA [D][pstride]
  int64_t pstride;
  const double* Q;      // column side fp64 SoA [D][qstride]
  int64_t qstride;
  const double* H;      // fp64 column term of the column side, -inf padding
  double nkappa;        // -s log2(e) / eps
  double inv_kappa;     // 1 / kappa
  int64_t nchunks;      // column chunks of kChunk64 points
  int64_t tiles;        // row tiles of kRowsPerTile rows
  int32_t G;            // column splits (a power of two)
  int32_t glog;
  int64_t cps;          // chunks per split
  double* Mp;           // [G][np] partial shift
  float* Sp;            // [G][np] partial sum
  const double* shift_pot;  // previous potential of the row side (shifted mode)
  double shift_mul;         // shift c = pot * shift_mul + shift_add (log2 units)
  double shift_add;
  // split form of the shifted pass: fp32 coordinates and the column term
  // split into an integer and a weight (see pair_pass_split)
  const float* P32;         // row side fp32 SoA [D][pstride]
  const float* Q32;         // column side fp32 SoA [D][qstride]
  const float* Hhi;
  const float* Wlo;
  float nkappa32;           // -kappa rounded to fp32
  int64_t nchunks32;        // column chunks of kChunkS points
  int64_t cps32;            // chunks of kChunkS per split
  RowFinal64 F;
};

// Exact two-pass recompute of a whole tile (all columns) by the kW waves of
// the workgroup: the row maxima of z (fp64), then the sum shifted to
// max - kHeadroom64.
template <int D>
__device__ void exact_tile64(const LseArgs64& A, TileLds& L, int64_t tile, double& mx,
                             double& sum) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  double x[kR][D];
  load_rows64<D>(A.P, A.pstride, tile, lane, x);
  double m[kR] = {-INFINITY, -INFINITY};
  rowmax_pass64<D>(m, A.Q, A.H, A.qstride, A.nkappa, x, wave, A.nchunks, kW);
  __syncthreads();  // LDS reuse
#pragma unroll
  for (int r = 0; r < kR; ++r) L.M[wave][lane + 64 * r] = m[r];
  __syncthreads();
  const int t = threadIdx.x;
  if (t < kRowsPerTile) {
    double v = L.M[0][t];
#pragma unroll
    for (int w = 1; w < kW; ++w) v = fmax(v, L.M[w][t]);
    L.red[t] = v;
  }
  __syncthreads();
  double c[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const double v = L.red[lane + 64 * r];
    c[r] = isfinite(v) ? v - kHeadroom64 : 0.0;  // an all -inf row sums to 0
  }
  __syncthreads();  // L.red is read before merge_waves64 and finish_tile64 reuse LDS
  RowAcc64 R;
  init_shift64(R, c, A.inv_kappa);
  pair_pass64<D>(R, A.Q, A.H, A.qstride, A.nkappa, A.inv_kappa, x, wave, A.nchunks, kW);
  merge_waves64(L, wave, lane, R, mx, sum);
}

// Shifted pair kernel in split form (pair_pass_split): workgroup w works on
// tile w / G, column split w % G, and writes the split's partials (fp64
// shift, fp32 sum) for k_merge64. Q, Hhi, Wlo, Mp and Sp come as separate
// no-alias arguments (scalar column loads). A row's shift is its estimated
// LSE less the headroom, rounded down to an integer and then to fp32 (exact
// below 2^24 in magnitude; beyond, the fp32 value is the shift, and the merge
// takes that same value).
template <int D>
__global__ __launch_bounds__(kThreads) void k_lse_split(LseArgs64 A, const float* __restrict__ Q,
                                                       const float* __restrict__ Hhi,
                                                       const float* __restrict__ Wlo,
                                                       double* __restrict__ Mp,
                                                       float* __restrict__ Sp) {
  __shared__ TileLds L;
  const int32_t gs = (int32_t)(blockIdx.x & (uint32_t)(A.G - 1));
  const int64_t tile = blockIdx.x >> A.glog;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float x[kR][D];
  load_rows<D>(A.P32, A.pstride, tile, lane, x);
  RowAccS R;
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int64_t i = tile * kRowsPerTile + lane + 64 * r;
    const double c = (i < A.F.np ? A.shift_pot[i] : 0.0) * A.shift_mul + A.shift_add;
    R.c[r] = isfinite(c) ? (float)floor(c) : 0.0f;
    R.S[r] = 0.0f;
  }
  const int64_t g0 = (int64_t)gs * A.cps32;
  const int64_t g1 = g0 + A.cps32 < A.nchunks32 ? g0 + A.cps32 : A.nchunks32;
  pair_pass_split<D>(R, Q, Hhi, Wlo, A.qstride, A.nkappa32, x, g0 + wave, g1, kW);
  // merge the waves' (shift, sum) through LDS in wave order (as merge_waves64)
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    L.M[wave][lane + 64 * r] = (double)R.c[r];
    L.S[wave][lane + 64 * r] = R.S[r];
  }
  __syncthreads();
  const int t = threadIdx.x;
  const int64_t i = tile * kRowsPerTile + t;
  if (t < kRowsPerTile && i < A.F.np) {
    double mx = -DBL_MAX, sum = 0.0;
#pragma unroll
    for (int v = 0; v < kW; ++v) mx = fmax(mx, L.M[v][t]);
#pragma unroll
    for (int v = 0; v < kW; ++v) sum += (double)L.S[v][t] * (double)ex2((float)(L.M[v][t] - mx));
    Mp[(int64_t)gs * A.F.np + i] = mx;
    Sp[(int64_t)gs * A.F.np + i] = (float)sum;
  }
}

// Split of the fp64 column term for the split form: Hhi = the integer below
// H, Wlo = 2^(H - Hhi) (fp64 exp2, one rounding); |H| >= 2^22: Hhi = H rounded
// to fp32 (a multiple of its ulp) and Wlo = 2^(H - Hhi), so the split is as
// exact there; padding and massless points: -inf and 0.
__global__ __launch_bounds__(256) void k_split_terms(const double* __restrict__ H, int64_t n,
                                                     float* __restrict__ Hhi,
                                                     float* __restrict__ Wlo) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  const double h = H[j];
  if (!isfinite(h)) {
    Hhi[j] = (float)h;
    Wlo[j] = 0.0f;
    return;
  }
  const double hi = fabs(h) < 0x1p22 ? floor(h) : (double)(float)h;
  Hhi[j] = (float)hi;
  Wlo[j] = (float)exp2(h - hi);
}

// Merge of the G splits of each row of a tile (as k_merge in dense.hip), the
// exact recompute of a tile with a too-small row sum, then finalize.
template <int D>
__global__ __launch_bounds__(kThreads) void k_merge64(LseArgs64 A) {
  __shared__ TileLds L;
  __shared__ double sS[kW][kRowsPerTile];
  const int64_t tile = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t np = A.F.np;
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
  if (needs_exact(np, tile, sum)) exact_tile64<D>(A, L, tile, mx, sum);
  finish_tile64(A.F, L, tile, mx, sum);
}

// Exact mode (no previous potential): one workgroup per tile, two passes.
template <int D>
__global__ __launch_bounds__(kThreads) void k_exact64(LseArgs64 A) {
  __shared__ TileLds L;
  const int64_t tile = blockIdx.x;
  double mx, sum;
  exact_tile64<D>(A, L, tile, mx, sum);
  finish_tile64(A.F, L, tile, mx, sum);
}

// fp64 column term H_j = log2 w_j + pot_j log2(e) / eps from an fp32 or an
// fp64 potential (exactly one non-null).
__global__ __launch_bounds__(256) void k_column_term64(const float* __restrict__ w,
                                                       const float* __restrict__ pot32,
                                                       const double* __restrict__ pot64,
                                                       int64_t count, double lam,
                                                       double* __restrict__ H) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j < count) H[j] = log2((double)w[j]) + (pot64 ? pot64[j] : (double)pot32[j]) * lam;
}

template <int D>
int64_t resident_slots64(sinkhorn_problem* p) {
  static const int per_cu = [] {
    int nb = 0;
    SK_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_lse_split<D>, kThreads, 0));
    return nb > 0 ? nb : 1;
  }();
  return (int64_t)per_cu * p->num_cu;
}

constexpr int64_t kXcds64 = 8;
constexpr int64_t kL2Slice64 = 2 << 20;

// The fp32 kernels' split rule (launch_plan.h) for 8-column chunks of fp64
// columns ((d + 1) * 8 bytes per column).
DenseSplit split64(int64_t nrows, int64_t ncols, int64_t slots, int d) {
  return plan_dense_split(nrows, ncols, slots, 2 * d + 1, kChunk64, kRowsPerTile, kW, kThreads,
                          kMaxSplit, kXcds64, kL2Slice64);
}

template <int D>
void run64(sinkhorn_problem* p, const HalfStep64& hs, LseArgs64& A, double pairs) {
  const bool shifted = hs.shift_pot != nullptr;
  const DenseSplit s = split64(hs.rows->count, hs.cols->count, resident_slots64<D>(p), D);
  if (!s.ok) fail(SINKHORN_ERR_UNSUPPORTED, "too many row tiles for one dispatch");
  A.nchunks = s.nchunks;
  A.tiles = s.tiles;
  A.G = s.G;
  A.glog = s.glog;
  A.cps = s.cps;
  if (row_groups(hs.rows->count) > p->red_cap) fail(SINKHORN_ERR_HIP, "reduction buffer too small");
  if (shifted) {
    if (2 * (int64_t)A.G * hs.rows->count > p->part_cap)
      fail(SINKHORN_ERR_HIP, "partial buffer too small");
    const Side& cols = *hs.cols;
    // the column term's split for this half-step, then the split-form pass
    // over the same G column splits, cut in chunks of kChunkS columns
    hipLaunchKernelGGL(k_split_terms, grid1((cols.padded + 255) / 256, 256), dim3(256), 0, p->stream,
                       A.H, cols.padded, cols.Hhi, cols.Wlo);
    SK_LAUNCH_CHECK();
    A.P32 = hs.rows->soa;
    A.Q32 = cols.soa;
    A.Hhi = cols.Hhi;
    A.Wlo = cols.Wlo;
    A.nkappa32 = (float)A.nkappa;
    A.nchunks32 = (cols.count + kChunkS - 1) / kChunkS;
    A.cps32 = (A.nchunks32 + A.G - 1) / A.G;
    const ProfEv pe = prof_events(p, SINKHORN_PROF_DENSE);
    hipExtLaunchKernelGGL((k_lse_split<D>), grid1(A.tiles * A.G, kThreads), dim3(kThreads), 0,
                          p->stream, pe.start, pe.stop, 0, A, A.Q32, A.Hhi, A.Wlo, A.Mp, A.Sp);
    SK_LAUNCH_CHECK();
    prof_done(p, SINKHORN_PROF_DENSE, pairs);
    hipLaunchKernelGGL(k_merge64<D>, grid1(A.tiles, kThreads), dim3(kThreads), 0, p->stream, A);
    SK_LAUNCH_CHECK();
  } else {
    const ProfEv pe = prof_events(p, SINKHORN_PROF_DENSE_EXACT);
    hipExtLaunchKernelGGL((k_exact64<D>), grid1(A.tiles, kThreads), dim3(kThreads), 0, p->stream,
                          pe.start, pe.stop, 0, A);
    SK_LAUNCH_CHECK();
    prof_done(p, SINKHORN_PROF_DENSE_EXACT, pairs);  // the half-step's pairs (each visited twice)
  }
  if (hs.residual) launch_reduce(p, A.tiles);
}

}  // namespace

int64_t dense64_partial_floats(sinkhorn_problem* p, int64_t nrows, int64_t ncols) {
  DenseSplit s;
  switch (p->d) {
    case 1: s = split64(nrows, ncols, resident_slots64<1>(p), 1); break;
    case 2: s = split64(nrows, ncols, resident_slots64<2>(p), 2); break;
    case 3: s = split64(nrows, ncols, resident_slots64<3>(p), 3); break;
    default: return 0;
  }
  return 2 * (int64_t)s.G * nrows;  // fp64 shifts take two float slots
}

void prep_column_term64(sinkhorn_problem* p, const Side& side, const float* pot32,
                        const double* pot64, double eps, double* H) {
  hipLaunchKernelGGL(k_column_term64, grid1((side.count + 255) / 256, 256), dim3(256), 0, p->stream,
                     side.w, pot32, pot64, side.count, kLog2e / eps, H);
  SK_LAUNCH_CHECK();
}

void dense_halfstep64(sinkhorn_problem* p, const HalfStep64& hs) {
  const Side& rows = *hs.rows;
  const Side& cols = *hs.cols;
  if (!rows.soa64 || !cols.soa64) fail(SINKHORN_ERR_HIP, "fp64 half-step without fp64 coordinates");
  LseArgs64 A;
  A.P = rows.soa64;
  A.pstride = rows.padded;
  A.Q = cols.soa64;
  A.qstride = cols.padded;
  A.H = hs.Hcols;
  const double kappa = p->scale * kLog2e / hs.eps;
  A.nkappa = -kappa;
  A.inv_kappa = 1.0 / kappa;
  A.Mp = reinterpret_cast<double*>(p->Mpart);
  A.Sp = p->Spart;
  A.shift_pot = hs.shift_pot;
  A.shift_mul = -kLog2e / hs.eps;
  A.shift_add = -kHeadroom64;
  RowFinal64& F = A.F;
  F.np = rows.count;
  F.w = rows.w;
  F.out32 = hs.out32;
  F.out64 = hs.out64;
  F.prev32 = hs.residual ? hs.prev32 : nullptr;
  F.prev64 = hs.residual ? hs.prev64 : nullptr;
  F.Hnext = hs.Hnext;
  F.lam_next = kLog2e / hs.eps_next;
  F.neg_eps_ln2 = -hs.eps * kLn2;
  F.inv_eps = 1.0 / hs.eps;
  F.red_part = p->red_part;
  F.ctl = p->ctl;
  const double pairs = (double)rows.count * (double)cols.count;
  switch (p->d) {
    case 1: run64<1>(p, hs, A, pairs); break;
    case 2: run64<2>(p, hs, A, pairs); break;
    case 3: run64<3>(p, hs, A, pairs); break;
    default: fail(SINKHORN_ERR_UNSUPPORTED, "fp64 half-step supports d <= 3");
  }
}

}  // namespace sk
