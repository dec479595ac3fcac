// Barycentric projection of plan rows and the source-coordinate gradient.
//
// FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport, §A.2: holding the
// target side and its potentials fixed, the gradient of the objective with
// respect to source point x_i is 2 s a_i (x_i - T_i), where T_i, the
// barycentric projection of row i, is the mean of the targets under the row's
// conditional plan weights; §A.4: the masked gradient restricts the plan to
// the admitted tiles. With pi_ij = a_i b_j exp((f_i + g_j - C_ij)/eps) the row
// factor cancels: T_i = sum_j w_ij y_j / sum_j w_ij, w_ij = b_j exp((g_j - C_ij)/eps),
// which is the f-step's streaming sum with d extra accumulators.
//
// Dense: the column split of the dense half-step (G workgroups per 128-row
// tile, partials (max, sum, d weighted sums) per split), then a merge kernel
// per tile in fixed order that writes T and the gradient. Sparse: one
// workgroup per 128-row tile over its row block's admitted tiles. With the row
// potentials given, the loops run shifted (pairloop.h); a tile with a row whose
// sum came out below 2^-40 is recomputed exactly. Results are
// bit-reproducible. d <= 8.
#include <cfloat>
#include <cmath>

#include "pairloop.h"

namespace sk {
namespace {

struct BaryArgs {
  const float* P;   // row side SoA [D][pstride]
  int64_t pstride;
  const float* Q;   // column side SoA [D][qstride]
  int64_t qstride;
  const float* H;   // column term of the column side (log2 units)
  float nkappa;     // -s log2(e) / eps
  int64_t nchunks;  // column chunks
  int64_t tiles;    // row tiles
  int32_t G;        // dense: column splits (a power of two)
  int32_t glog;     // dense: log2 G
  int64_t cps;      // dense: chunks per split
  double* Mp;       // dense: [G][np] partial max / shift
  float* Sp;        // dense: [G][np] partial sum
  float* Ap;        // dense: [G][D][np] partial weighted coordinate sums
  const float* shift_pot;  // row potentials for the shifts, or null (exact loop)
  float lam;               // log2(e) / eps
  float inv_kappa;         // 1 / kappa
  const float* w;          // row weights [np]
  int64_t np;              // rows
  double gscale;           // 2 s
  float* T;                // [np][D] row-major, or null
  float* grad;             // [np][D] row-major, or null
  int32_t B;               // sparse: block size
  const int64_t* ptr;      // sparse: [row blocks + 1]
  const int32_t* idx;      // sparse: admitted column blocks
  int32_t* tile_flag;      // sparse: tiles left for the exact recompute
  int32_t fallback;        // sparse: 1 = exact recompute of flagged tiles only
  const int32_t* order;    // sparse: tile of each workgroup (longest lists first), or null
};

template <int D>
struct BaryLds {
  double M[kW][kRowsPerTile];
  double S[kW][kRowsPerTile];
  double A[kW][D][kRowsPerTile];
};

// Per-wave (max, sum, weighted sums) of the lane's rows into LDS; thread
// t < 128 then combines row t over the waves in wave order (fp64).
template <int D>
__device__ __forceinline__ void bary_merge_waves(BaryLds<D>& L, int wave, int lane,
                                                 const double (&m)[kR], const double (&s)[kR],
                                                 const double (&a)[kR][D], double& mx, double& sum,
                                                 double (&acc)[D]) {
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    L.M[wave][lane + 64 * r] = m[r];
    L.S[wave][lane + 64 * r] = s[r];
#pragma unroll
    for (int k = 0; k < D; ++k) L.A[wave][k][lane + 64 * r] = a[r][k];
  }
  __syncthreads();
  mx = -DBL_MAX;
  sum = 0.0;
#pragma unroll
  for (int k = 0; k < D; ++k) acc[k] = 0.0;
  const int t = threadIdx.x;
  if (t < kRowsPerTile) {
#pragma unroll
    for (int v = 0; v < kW; ++v) mx = fmax(mx, L.M[v][t]);
#pragma unroll
    for (int v = 0; v < kW; ++v) {
      const double sc = (double)ex2((float)(L.M[v][t] - mx));
      sum += L.S[v][t] * sc;
#pragma unroll
      for (int k = 0; k < D; ++k) acc[k] += L.A[v][k][t] * sc;
    }
  }
}

template <int D, bool SHIFT>
__device__ __forceinline__ void acc_to_double(const RowAcc<SHIFT, D>& R, double (&m)[kR],
                                              double (&s)[kR], double (&a)[kR][D]) {
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    m[r] = R.max_or_shift(r);
    s[r] = (double)R.S[r];
#pragma unroll
    for (int k = 0; k < D; ++k) a[r][k] = (double)R.A[r][k];
  }
}

template <int D, bool SHIFT>
__device__ __forceinline__ void init_rows(const BaryArgs& A, int64_t tile, int lane,
                                          RowAcc<SHIFT, D>& R) {
  if (SHIFT) {
    float pot[kR];
    load_shift_pot(A.shift_pot, A.np, tile, lane, pot);
    R.init_shift(pot, A.lam, A.inv_kappa, A.nkappa);
  } else {
    R.init_exact();
  }
}

// T_i = acc / sum, grad_i = 2 s a_i (x_i - T_i) for row t < 128 of the tile.
template <int D>
__device__ __forceinline__ void bary_write(const BaryArgs& A, int64_t tile, double sum,
                                           const double (&acc)[D]) {
  const int64_t i = tile * kRowsPerTile + threadIdx.x;
  if (threadIdx.x >= kRowsPerTile || i >= A.np) return;
  const double wi = (double)A.w[i];
#pragma unroll
  for (int k = 0; k < D; ++k) {
    const double Tk = acc[k] / sum;
    if (A.T) A.T[i * D + k] = (float)Tk;
    if (A.grad) A.grad[i * D + k] = (float)(A.gscale * wi * ((double)A.P[k * A.pstride + i] - Tk));
  }
}

// Exact recompute of a whole dense tile (all columns) by the workgroup.
template <int D>
__device__ void bary_exact_tile(const BaryArgs& A, BaryLds<D>& L, int64_t tile, double& mx,
                                double& sum, double (&acc)[D]) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float x[kR][D];
  load_rows<D>(A.P, A.pstride, tile, lane, x);
  RowAcc<false, D> R;
  R.init_exact();
  pair_pass<D, false, D>(R, A.Q, A.H, A.qstride, A.nkappa, x, wave, A.nchunks, kW);
  double m[kR], s[kR], a[kR][D];
  acc_to_double(R, m, s, a);
  __syncthreads();  // LDS reuse
  bary_merge_waves(L, wave, lane, m, s, a, mx, sum, acc);
}

// Dense: workgroup = (tile, split); writes the split's partials.
template <int D, bool SHIFT>
__global__ __launch_bounds__(kThreads) void k_bary_valu(BaryArgs A, const float* __restrict__ Q,
                                                       const float* __restrict__ H,
                                                       double* __restrict__ Mp,
                                                       float* __restrict__ Sp,
                                                       float* __restrict__ Ap) {
  __shared__ BaryLds<D> L;
  const int32_t gs = (int32_t)(blockIdx.x & (uint32_t)(A.G - 1));
  const int64_t tile = blockIdx.x >> A.glog;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float x[kR][D];
  load_rows<D>(A.P, A.pstride, tile, lane, x);
  RowAcc<SHIFT, D> R;
  init_rows<D, SHIFT>(A, tile, lane, R);
  const int64_t g0 = (int64_t)gs * A.cps;
  const int64_t g1 = g0 + A.cps < A.nchunks ? g0 + A.cps : A.nchunks;
  pair_pass<D, SHIFT, D>(R, Q, H, A.qstride, A.nkappa, x, g0 + wave, g1, kW);
  double m[kR], s[kR], a[kR][D], mx, sum, acc[D];
  acc_to_double(R, m, s, a);
  bary_merge_waves(L, wave, lane, m, s, a, mx, sum, acc);
  const int64_t i = tile * kRowsPerTile + threadIdx.x;
  if (threadIdx.x < kRowsPerTile && i < A.np) {
    Mp[(int64_t)gs * A.np + i] = mx;
    Sp[(int64_t)gs * A.np + i] = (float)sum;
#pragma unroll
    for (int k = 0; k < D; ++k) Ap[((int64_t)gs * D + k) * A.np + i] = (float)acc[k];
  }
}

// Dense: merge of a tile's G splits (wave w takes splits w, w + 8, ...; the
// waves then combine in wave order), exact recompute if needed, outputs.
template <int D>
__global__ __launch_bounds__(kThreads) void k_bary_merge(BaryArgs A, int32_t shifted) {
  __shared__ BaryLds<D> L;
  const int64_t tile = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  double m[kR], s[kR], a[kR][D];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int64_t i = tile * kRowsPerTile + lane + 64 * r;
    m[r] = -DBL_MAX;
    s[r] = 0.0;
#pragma unroll
    for (int k = 0; k < D; ++k) a[r][k] = 0.0;
    if (i < A.np) {
      for (int32_t t = wave; t < A.G; t += kW) m[r] = fmax(m[r], A.Mp[(int64_t)t * A.np + i]);
      for (int32_t t = wave; t < A.G; t += kW) {
        const int64_t o = (int64_t)t * A.np + i;
        const double sc = (double)ex2((float)(A.Mp[o] - m[r]));
        s[r] += (double)A.Sp[o] * sc;
#pragma unroll
        for (int k = 0; k < D; ++k) a[r][k] += (double)A.Ap[((int64_t)t * D + k) * A.np + i] * sc;
      }
    }
  }
  double mx, sum, acc[D];
  bary_merge_waves(L, wave, lane, m, s, a, mx, sum, acc);
  if (shifted && needs_exact(A.np, tile, sum)) bary_exact_tile<D>(A, L, tile, mx, sum, acc);
  bary_write<D>(A, tile, sum, acc);
}

// Sparse: workgroup = 128-row tile of row block I over its admitted tiles
// (all columns when it has none); writes the outputs directly. In shifted mode
// a tile with a too-small row sum is flagged for the fallback launch. Tiles
// are taken in A.order when given (longest lists first; results unchanged).
template <int D, bool SHIFT>
__global__ __launch_bounds__(kThreads) void k_bary_sparse(BaryArgs A, const float* __restrict__ Q,
                                                         const float* __restrict__ H) {
  __shared__ BaryLds<D> L;
  const int64_t tile = A.order ? (int64_t)A.order[blockIdx.x] : (int64_t)blockIdx.x;
  if (tile < 0) return;                                         // an empty slot (uniform)
  if (!SHIFT && A.fallback && A.tile_flag[tile] == 0) return;  // uniform
  const int64_t I = tile * kRowsPerTile / A.B;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float x[kR][D];
  load_rows<D>(A.P, A.pstride, tile, lane, x);
  RowAcc<SHIFT, D> R;
  init_rows<D, SHIFT>(A, tile, lane, R);
  const int64_t p0 = A.ptr[I];
  const int64_t p1 = A.ptr[I + 1];
  const int64_t cpb = A.B / kChunk;
  if (p1 > p0) {
    for (int64_t q = p0 + wave; q < p1; q += kW) {
      const int64_t c0 = (int64_t)A.idx[q] * cpb;
      const int64_t c1 = c0 + cpb < A.nchunks ? c0 + cpb : A.nchunks;
      pair_pass<D, SHIFT, D>(R, Q, H, A.qstride, A.nkappa, x, c0, c1, 1);
    }
  } else {
    pair_pass<D, SHIFT, D>(R, Q, H, A.qstride, A.nkappa, x, wave, A.nchunks, kW);
  }
  double m[kR], s[kR], a[kR][D], mx, sum, acc[D];
  acc_to_double(R, m, s, a);
  bary_merge_waves(L, wave, lane, m, s, a, mx, sum, acc);
  if (SHIFT && needs_exact(A.np, tile, sum)) {
    if (threadIdx.x == 0) A.tile_flag[tile] = 1;
    return;
  }
  if (!SHIFT && A.fallback && threadIdx.x == 0) A.tile_flag[tile] = 0;
  bary_write<D>(A, tile, sum, acc);
}

BaryArgs make_args(sinkhorn_problem* p, double eps, const float* f_hint, float* T, float* grad) {
  BaryArgs A{};
  A.P = p->X.soa;
  A.pstride = p->X.padded;
  A.Q = p->Y.soa;
  A.qstride = p->Y.padded;
  A.H = p->Y.H;
  const double kappa = p->scale * kLog2e / eps;
  A.nkappa = (float)(-kappa);
  A.nchunks = (p->m + kChunk - 1) / kChunk;
  A.tiles = (p->n + kRowsPerTile - 1) / kRowsPerTile;
  A.shift_pot = f_hint;
  A.lam = (float)(kLog2e / eps);
  A.inv_kappa = (float)(1.0 / kappa);
  A.w = p->X.w;
  A.np = p->n;
  A.gscale = 2.0 * p->scale;
  A.T = T;
  A.grad = grad;
  A.tile_flag = p->tile_flag;
  return A;
}

template <int D>
void dense_bary(sinkhorn_problem* p, BaryArgs& A) {
  const SplitInfo sp = dense_split(p, p->n, p->m);
  A.G = sp.G;
  A.glog = sp.glog;
  A.cps = sp.cps;
  A.nchunks = sp.nchunks;
  A.tiles = sp.tiles;
  const int64_t np = p->n;
  // the split partials of the half-step (same plan, so they fit) and a
  // grown-on-demand buffer for the weighted sums: no allocation per call
  if (2 * (int64_t)A.G * np > p->part_cap) fail(SINKHORN_ERR_HIP, "partial buffer too small");
  A.Mp = reinterpret_cast<double*>(p->Mpart);
  A.Sp = p->Spart;
  const int64_t need = (int64_t)A.G * D * np;
  if (need > p->bary_cap) {
    SK_HIP(hipStreamSynchronize(p->stream));
    dev_free(p->bary_part);
    p->bary_part = nullptr;
    p->bary_cap = 0;
    p->bary_part = (float*)dev_alloc(sizeof(float) * (size_t)need);
    p->bary_cap = need;
  }
  A.Ap = p->bary_part;
  const bool shifted = A.shift_pot != nullptr;
  {
    const dim3 grid((uint32_t)(A.tiles * A.G));
    const ProfEv pe = prof_events(p, SINKHORN_PROF_BARY);
    if (shifted)
      hipExtLaunchKernelGGL((k_bary_valu<D, true>), grid, dim3(kThreads), 0, p->stream, pe.start,
                            pe.stop, 0, A, A.Q, A.H, A.Mp, A.Sp, A.Ap);
    else
      hipExtLaunchKernelGGL((k_bary_valu<D, false>), grid, dim3(kThreads), 0, p->stream, pe.start,
                            pe.stop, 0, A, A.Q, A.H, A.Mp, A.Sp, A.Ap);
    SK_LAUNCH_CHECK();
    prof_done(p, SINKHORN_PROF_BARY, (double)p->n * (double)p->m);
    hipLaunchKernelGGL(k_bary_merge<D>, grid1(A.tiles, kThreads), dim3(kThreads), 0, p->stream, A,
                       (int32_t)shifted);
    SK_LAUNCH_CHECK();
  }
}

template <int D>
void sparse_bary(sinkhorn_problem* p, BaryArgs& A) {
  int64_t slots = A.tiles;
  A.order = heavy_first(p, A.ptr, A.tiles, A.B, (p->m + A.B - 1) / A.B, &slots);
  const dim3 grid = grid1(slots, kThreads);
  if (A.shift_pot) {
    hipLaunchKernelGGL((k_bary_sparse<D, true>), grid, dim3(kThreads), 0, p->stream, A, A.Q, A.H);
    SK_LAUNCH_CHECK();
    BaryArgs E = A;
    E.fallback = 1;
    E.order = nullptr;
    hipLaunchKernelGGL((k_bary_sparse<D, false>), grid1(A.tiles, kThreads), dim3(kThreads), 0,
                       p->stream, E, E.Q, E.H);
  } else {
    hipLaunchKernelGGL((k_bary_sparse<D, false>), grid, dim3(kThreads), 0, p->stream, A, A.Q, A.H);
  }
  SK_LAUNCH_CHECK();
}

void check_args(sinkhorn_problem* p, double eps, const float* g, float* T, float* grad) {
  if (!p || !g) fail(SINKHORN_ERR_INVALID_ARG, "null pointer");
  if (!T && !grad) fail(SINKHORN_ERR_INVALID_ARG, "T and grad are both null");
  if (!(std::isfinite(eps) && eps > 0.0)) fail(SINKHORN_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (p->d > kMaxValuD) fail(SINKHORN_ERR_UNSUPPORTED, "barycentric projection supports d <= 8");
}

template <typename Fn>
int guarded(Fn&& fn) {
  try {
    return fn();
  } catch (const Failure& e) {
    set_last_error(e.msg);
    return e.code;
  } catch (const std::bad_alloc&) {
    set_last_error("host allocation failed");
    return SINKHORN_ERR_OOM;
  } catch (...) {
    set_last_error("unexpected exception");
    return SINKHORN_ERR_HIP;
  }
}

}  // namespace
}  // namespace sk

using namespace sk;

extern "C" {

int sinkhorn_barycentric(sinkhorn_problem* p, double eps, const float* g, const float* f_hint,
                         float* T, float* grad) {
  return guarded([&] {
    check_args(p, eps, g, T, grad);
    prep_column_term(p, p->Y, g, eps, p->Y.H);
    BaryArgs A = make_args(p, eps, f_hint, T, grad);
    switch (p->d) {
      case 1: dense_bary<1>(p, A); break;
      case 2: dense_bary<2>(p, A); break;
      case 3: dense_bary<3>(p, A); break;
      case 4: dense_bary<4>(p, A); break;
      case 5: dense_bary<5>(p, A); break;
      case 6: dense_bary<6>(p, A); break;
      case 7: dense_bary<7>(p, A); break;
      case 8: dense_bary<8>(p, A); break;
    }
    return SINKHORN_OK;
  });
}

int sinkhorn_sparse_barycentric(sinkhorn_problem* p, double eps, const float* g, const float* f_hint,
                                int32_t B, const int64_t* ptr, const int32_t* idx, float* T,
                                float* grad) {
  return guarded([&] {
    check_args(p, eps, g, T, grad);
    if (!ptr) fail(SINKHORN_ERR_INVALID_ARG, "null pointer");
    if (p->d > 3) fail(SINKHORN_ERR_UNSUPPORTED, "sparse barycentric projection needs d <= 3");
    if (B < kRowsPerTile || B % kRowsPerTile != 0 || B > 1024)
      fail(SINKHORN_ERR_UNSUPPORTED, "B must be a multiple of 128, at most 1024");
    const int64_t nr = (p->n + B - 1) / B, nc = (p->m + B - 1) / B;
    check_csr(p, ptr, nr, idx, nc);
    prep_column_term(p, p->Y, g, eps, p->Y.H);
    BaryArgs A = make_args(p, eps, f_hint, T, grad);
    A.B = B;
    A.ptr = ptr;
    A.idx = idx;
    switch (p->d) {
      case 1: sparse_bary<1>(p, A); break;
      case 2: sparse_bary<2>(p, A); break;
      case 3: sparse_bary<3>(p, A); break;
    }
    return SINKHORN_OK;
  });
}

}  // extern "C"
