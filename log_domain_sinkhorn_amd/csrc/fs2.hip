// Block-sparse multiscale solve (d <= 3).
//
// FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport:
//   §3, §B.1   Morton order; blocks of B consecutive sorted points; cells are
//              Morton-prefix groups, at most about twice as many as blocks
//              (prefix of p = floor(log2(2 max(NB, MB))) bits by default);
//   §3.1, §B.2 annealed dense Sinkhorn on cell records (mass-weighted
//              centroid, mass), continued at the target eps until the coarse
//              residual is small, stalls, or hits its cap;
//   §1, §A.1   the coarse potentials are lifted to the points by one
//              log-sum-exp against the other side's centroids;
//   §3.2       every fine update rebuilds the mask at the current potentials
//              and runs the sparse f- and g-steps on it (g on the transpose);
//   §C.4       the stop certificate is the admitted-plan residual plus a bound
//              on the omitted mass: max(R_A,row, R_A,col) + Omega <= tol with
//              Omega = max(NB, MB) delta_rel, the a-priori total omitted mass
//              of the threshold rule (§3.2).
// The admitted-plan residual of the state (f, g) is the fused residual of the
// sparse f-step built at (f, g); the column residual is a sparse g pass at
// (f, g), run only when the row test already passes.
#include <chrono>
#include <cmath>
#include <vector>

#include <rocprim/device/device_scan.hpp>

#include "internal.h"
#include "verify.h"

namespace sk {
namespace {

__global__ __launch_bounds__(256) void k_gather(const float* __restrict__ soa, int64_t istride,
                                                const float* __restrict__ w,
                                                const int32_t* __restrict__ perm, int64_t count,
                                                int32_t d, float* __restrict__ out,
                                                int64_t ostride, float* __restrict__ wout) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  const int64_t s = perm[i];
  for (int k = 0; k < d; ++k) out[k * ostride + i] = soa[k * istride + s];
  wout[i] = w[s];
}

__global__ __launch_bounds__(256) void k_scatter(const float* __restrict__ in,
                                                 const int32_t* __restrict__ perm, int64_t count,
                                                 float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) out[perm[i]] = in[i];
}

__global__ __launch_bounds__(256) void k_gather_pot(const float* __restrict__ in,
                                                    const int32_t* __restrict__ perm, int64_t count,
                                                    float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) out[i] = in[perm[i]];
}

__global__ __launch_bounds__(256) void k_cell_flags(const uint64_t* __restrict__ codes,
                                                    int64_t count, int32_t shift,
                                                    int32_t* __restrict__ flags) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  flags[i] = (i == 0 || (codes[i] >> shift) != (codes[i - 1] >> shift)) ? 1 : 0;
}

// incl = inclusive scan of flags; a cell c starts where flags[i] = 1 and incl[i] = c + 1.
__global__ __launch_bounds__(256) void k_cell_offsets(const int32_t* __restrict__ flags,
                                                      const int32_t* __restrict__ incl,
                                                      int64_t count, int64_t* __restrict__ off) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  if (flags[i]) off[incl[i] - 1] = i;
  if (i == count - 1) off[incl[i]] = count;
}

// One thread per cell: mass and mass-weighted centroid, accumulated in fp64.
__global__ __launch_bounds__(256) void k_cell_records(const float* __restrict__ soa,
                                                      int64_t stride, const float* __restrict__ w,
                                                      const int64_t* __restrict__ off,
                                                      int64_t ncells, int32_t d,
                                                      float* __restrict__ cent, int64_t cstride,
                                                      float* __restrict__ mass) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= ncells) return;
  const int64_t s = off[c], e = off[c + 1];
  double m = 0.0, acc[3] = {0.0, 0.0, 0.0}, plain[3] = {0.0, 0.0, 0.0};
  for (int64_t i = s; i < e; ++i) {
    const double wi = (double)w[i];
    m += wi;
    for (int k = 0; k < d; ++k) {
      const double v = (double)soa[k * stride + i];
      acc[k] += wi * v;
      plain[k] += v;
    }
  }
  for (int k = 0; k < d; ++k)
    cent[k * cstride + c] = (float)(m > 0.0 ? acc[k] / m : plain[k] / (double)(e - s));
  mass[c] = (float)m;
}

void free_side(Side& s) {
  dev_free(s.soa);
  dev_free(s.w);
  dev_free(s.H);
  s = Side();
}

void alloc_side(Side& s, int64_t count, int32_t d, hipStream_t st) {
  s.count = count;
  s.padded = round_up(count, kPad);
  s.soa = (float*)dev_alloc(sizeof(float) * d * s.padded);
  s.w = (float*)dev_alloc(sizeof(float) * count);
  s.H = (float*)dev_alloc(sizeof(float) * s.padded);
  fill_f32(s.soa, d * s.padded, 0.0f, st);
  fill_f32(s.H, s.padded, -INFINITY, st);
}

// Morton-prefix cells of a sorted side: centroids and masses as a new side.
void build_cells(sinkhorn_problem* p, const Side& sorted, const uint64_t* codes, int32_t p_bits,
                 Side& cells) {
  hipStream_t st = p->stream;
  const int64_t n = sorted.count;
  const int32_t shift = 21 * p->d - p_bits;
  int32_t* flags = (int32_t*)dev_alloc(sizeof(int32_t) * n);
  int32_t* incl = (int32_t*)dev_alloc(sizeof(int32_t) * n);
  int64_t* off = nullptr;
  void* temp = nullptr;
  try {
    hipLaunchKernelGGL(k_cell_flags, grid1(((n + 255) / 256), 256), dim3(256), 0, st, codes, n,
                       shift, flags);
    SK_LAUNCH_CHECK();
    size_t tb = 0;
    SK_HIP(rocprim::inclusive_scan(nullptr, tb, flags, incl, (size_t)n, rocprim::plus<int32_t>(), st));
    temp = dev_alloc(tb);
    SK_HIP(rocprim::inclusive_scan(temp, tb, flags, incl, (size_t)n, rocprim::plus<int32_t>(), st));
    int32_t ncell = 0;
    SK_HIP(hipMemcpyAsync(&ncell, incl + n - 1, sizeof(int32_t), hipMemcpyDeviceToHost, st));
    SK_HIP(hipStreamSynchronize(st));
    off = (int64_t*)dev_alloc(sizeof(int64_t) * (ncell + 1));
    hipLaunchKernelGGL(k_cell_offsets, grid1(((n + 255) / 256), 256), dim3(256), 0, st, flags,
                       incl, n, off);
    SK_LAUNCH_CHECK();
    alloc_side(cells, ncell, p->d, st);
    hipLaunchKernelGGL(k_cell_records, grid1(((ncell + 255) / 256), 256), dim3(256), 0, st,
                       sorted.soa, sorted.padded, sorted.w, off, (int64_t)ncell, p->d, cells.soa,
                       cells.padded, cells.w);
    SK_LAUNCH_CHECK();
    SK_HIP(hipStreamSynchronize(st));
  } catch (...) {
    dev_free(flags);
    dev_free(incl);
    dev_free(off);
    dev_free(temp);
    throw;
  }
  dev_free(flags);
  dev_free(incl);
  dev_free(off);
  dev_free(temp);
}

// Grow the split partial buffers to hold `floats` entries each.
void ensure_partials(sinkhorn_problem* p, int64_t floats) {
  if (floats <= p->part_cap) return;
  SK_HIP(hipStreamSynchronize(p->stream));
  dev_free(p->Mpart);
  dev_free(p->Spart);
  p->Mpart = p->Spart = nullptr;
  p->part_cap = 0;
  p->Mpart = (float*)dev_alloc(sizeof(float) * floats);
  p->Spart = (float*)dev_alloc(sizeof(float) * floats);
  p->part_cap = floats;
}

double now_s() {
  return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

// Device buffers of one tile list that grows on demand.
struct TileList {
  int64_t* ptr = nullptr;
  int64_t* tmp = nullptr;
  int32_t* idx = nullptr;
  int64_t cap = 0;
  int64_t nnz = 0;
  ~TileList() {
    dev_free(ptr);
    dev_free(tmp);
    dev_free(idx);
  }
  void build(sinkhorn_problem* p, const BlockSummary& r, const BlockSummary& c, double eps,
             double delta) {
    if (!ptr) {
      ptr = (int64_t*)dev_alloc(sizeof(int64_t) * (r.nb + 1));
      tmp = (int64_t*)dev_alloc(sizeof(int64_t) * (r.nb + 1));
    }
    nnz = screen_tiles(p, r, c, eps, delta, ptr, idx, cap, tmp);
    if (nnz > cap) {
      dev_free(idx);
      idx = nullptr;
      cap = 0;
      const int64_t want = nnz + nnz / 4 + 1024;
      idx = (int32_t*)dev_alloc(sizeof(int32_t) * want);
      cap = want;
      nnz = screen_tiles(p, r, c, eps, delta, ptr, idx, cap, tmp);
    }
  }
};

// Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds of two 64 x 64 -> 128-bit products
// with the key bumped by the Weyl constants between rounds.
__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(kM0, c[0]), lo0 = kM0 * c[0];
    const uint64_t hi1 = __umul64hi(kM1, c[2]), lo1 = kM1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += kW0;
    k1 += kW1;
  }
}

// Sample k of a side of size count: word k % 4 of the block at counter
// (k / 4 + 1, 0, 0, 0), key (seed, stream), modulo count.
__global__ __launch_bounds__(256) void k_sample_idx(uint64_t seed, uint64_t stream, int64_t count,
                                                    int32_t K, int32_t* __restrict__ out) {
  const int32_t k = (int32_t)(blockIdx.x * 256 + threadIdx.x);
  if (k >= K) return;
  uint64_t c[4] = {(uint64_t)(k / 4) + 1ull, 0ull, 0ull, 0ull};
  philox4x64_10(c, seed, stream);
  out[k] = (int32_t)(c[k & 3] % (uint64_t)count);
}

// Drawn points of a side (coordinates, weight, potential) into a small side.
__global__ __launch_bounds__(256) void k_gather_samples(const float* __restrict__ soa, int64_t stride,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ pot,
                                                        const int32_t* __restrict__ idx, int32_t K,
                                                        int32_t d, float* __restrict__ dsoa,
                                                        int64_t dstride, float* __restrict__ dw,
                                                        float* __restrict__ dpot) {
  const int32_t k = (int32_t)(blockIdx.x * 256 + threadIdx.x);
  if (k >= K) return;
  const int64_t i = idx[k];
  for (int32_t a = 0; a < d; ++a) dsoa[a * dstride + k] = soa[a * stride + i];
  dw[k] = w[i];
  dpot[k] = pot[i];
}

// One block: t_k = w_k |exp((f_k - ft_k)/eps) - 1| (the drawn row's |row sum
// - w_k| from the half-step identity), out[0] = mean t, out[1] = sum (t -
// mean)^2, in a fixed order.
__global__ __launch_bounds__(256) void k_sample_terms(const float* __restrict__ w,
                                                      const float* __restrict__ f,
                                                      const float* __restrict__ ft, int32_t K,
                                                      double inv_eps, double* __restrict__ out) {
  __shared__ double sh[256];
  auto term = [&](int32_t k) {
    return (double)w[k] * fabs(expm1(((double)f[k] - (double)ft[k]) * inv_eps));
  };
  double s = 0.0;
  for (int32_t k = threadIdx.x; k < K; k += 256) s += term(k);
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  const double mean = sh[0] / (double)K;
  __syncthreads();
  double v = 0.0;
  for (int32_t k = threadIdx.x; k < K; k += 256) {
    const double e = term(k) - mean;
    v += e * e;
  }
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[0] = mean;
    out[1] = sh[0];
  }
}

// Device buffers of one verified tile list (row- or column-major).
struct VerifiedList {
  int64_t* ptr = nullptr;
  int32_t* idx = nullptr;
  int64_t cap = 0;
  int64_t nnz = 0;
  ~VerifiedList() {
    dev_free(ptr);
    dev_free(idx);
  }
  void reserve(sinkhorn_problem* p, int64_t nb, int64_t want) {
    if (!ptr) ptr = (int64_t*)dev_alloc(sizeof(int64_t) * (nb + 1));
    if (want > cap) {
      SK_HIP(hipStreamSynchronize(p->stream));
      dev_free(idx);
      idx = nullptr;
      cap = 0;
      const int64_t c = want + want / 4 + 1024;
      idx = (int32_t*)dev_alloc(sizeof(int32_t) * c);
      cap = c;
    }
  }
};

// Drawn points of one side for the sampled residual check.
struct SampleSide {
  Side S;
  int32_t* idx = nullptr;
  float* pot = nullptr;   // potential at the drawn points
  float* ft = nullptr;    // half-step at the drawn points
  double* sums = nullptr; // [2] mean term, sum of squared deviations
  int32_t K = 0;
  void release() {
    free_side(S);
    dev_free(idx);
    dev_free(pot);
    dev_free(ft);
    dev_free(sums);
    idx = nullptr;
    pot = ft = nullptr;
    sums = nullptr;
    K = 0;
  }
  ~SampleSide() { release(); }
};

// (estimate, standard error) of sum_i |sum_j pi_ij - w_i| over the rows of
// `rows` from K rows drawn with replacement (FlashSinkhorn 2, §3.1: sampled
// row sums cost O(md)); `cols.H` must hold the column term of the other
// side's potential at eps.
void sampled_residual(sinkhorn_problem* p, const Side& rows, const Side& cols, const float* pot,
                      double eps, uint64_t seed, uint64_t stream, int32_t K, SampleSide& S,
                      double* est, double* se) {
  hipStream_t st = p->stream;
  if (S.K != K) {
    SK_HIP(hipStreamSynchronize(st));
    S.release();
    alloc_side(S.S, K, p->d, st);
    S.idx = (int32_t*)dev_alloc(sizeof(int32_t) * K);
    S.pot = (float*)dev_alloc(sizeof(float) * K);
    S.ft = (float*)dev_alloc(sizeof(float) * K);
    S.sums = (double*)dev_alloc(sizeof(double) * 2);
    S.K = K;
  }
  const uint32_t blocks = (uint32_t)((K + 255) / 256);
  hipLaunchKernelGGL(k_sample_idx, dim3(blocks), dim3(256), 0, st, seed, stream, rows.count, K, S.idx);
  SK_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_gather_samples, dim3(blocks), dim3(256), 0, st, rows.soa, rows.padded, rows.w,
                     pot, S.idx, K, p->d, S.S.soa, S.S.padded, S.S.w, S.pot);
  SK_LAUNCH_CHECK();
  HalfStep hs{&S.S, &cols, cols.H, S.ft, nullptr, nullptr, eps, eps, false};
  hs.shift_pot = S.pot;
  dense_halfstep(p, hs);
  hipLaunchKernelGGL(k_sample_terms, dim3(1), dim3(256), 0, st, S.S.w, S.pot, S.ft, K, 1.0 / eps,
                     S.sums);
  SK_LAUNCH_CHECK();
  double h[2] = {0.0, 0.0};
  SK_HIP(hipMemcpyAsync(h, S.sums, sizeof(h), hipMemcpyDeviceToHost, st));
  SK_HIP(hipStreamSynchronize(st));
  const double c = (double)rows.count;
  *est = c * h[0];
  *se = K > 1 ? c * std::sqrt(h[1] / (double)(K - 1)) / std::sqrt((double)K) : INFINITY;
}

}  // namespace
}  // namespace sk

using namespace sk;

extern "C" int sinkhorn_solve_multiscale(sinkhorn_problem* p, const sinkhorn_multiscale_params* prm,
                                         float* f, float* g, sinkhorn_multiscale_report* rep) {
  Side Xs, Ys, Cx, Cy;
  uint64_t* codes[2] = {nullptr, nullptr};
  int32_t* perm[2] = {nullptr, nullptr};
  float* pot[10] = {};
  BlockSummary sx, sy;
  LocalFrame lx, ly;
  auto cleanup = [&]() {
    lx.release();
    ly.release();
    free_side(Xs);
    free_side(Ys);
    free_side(Cx);
    free_side(Cy);
    for (int k = 0; k < 2; ++k) {
      dev_free(codes[k]);
      dev_free(perm[k]);
    }
    for (auto& q : pot) dev_free(q);
    sx.release();
    sy.release();
  };
  try {
    if (!p || !prm || !f || !g) fail(SINKHORN_ERR_INVALID_ARG, "null pointer");
    const sinkhorn_multiscale_params P = *prm;
    if (p->d > 3) fail(SINKHORN_ERR_UNSUPPORTED, "the multiscale solve needs d <= 3");
    if (P.B < 128 || P.B % 128 != 0) fail(SINKHORN_ERR_UNSUPPORTED, "B must be a multiple of 128");
    if (!(std::isfinite(P.eps) && P.eps > 0.0)) fail(SINKHORN_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (!(P.tol > 0.0) || !(P.delta_scale > 0.0)) fail(SINKHORN_ERR_INVALID_ARG, "tol and delta_scale must be > 0");
    if (P.max_fine < 0 || P.coarse_max < 1) fail(SINKHORN_ERR_INVALID_ARG, "bad iteration caps");
    if (P.warm_start && P.adaptive) fail(SINKHORN_ERR_INVALID_ARG, "warm_start excludes the adaptive switch");
    if (P.verify && P.B != kVerifyB) fail(SINKHORN_ERR_UNSUPPORTED, "tile verification needs B = 128");
    if (P.adaptive && (P.check_every < 1 || P.check_samples < 2 || P.check_samples_max < P.check_samples ||
                       P.check_samples_max > (1 << 24)))
      fail(SINKHORN_ERR_INVALID_ARG, "adaptive switch: need check_every >= 1 and "
                                     "2 <= check_samples <= check_samples_max <= 2^24");
    hipStream_t st = p->stream;
    const int32_t d = p->d;
    const int64_t n = p->n, m = p->m;
    const double t_start = now_s();
    const int64_t NB = (n + P.B - 1) / P.B, MB = (m + P.B - 1) / P.B;
    const double delta = P.delta_scale / (double)(NB > MB ? NB : MB);
    const double omega = (double)(NB > MB ? NB : MB) * delta;
    int32_t p_bits = P.p_bits;
    if (p_bits <= 0) p_bits = (int32_t)std::floor(std::log2(2.0 * (double)(NB > MB ? NB : MB)));
    if (p_bits > 21 * d) p_bits = 21 * d;
    sinkhorn_multiscale_report R{};
    R.omega = omega;
    const int64_t bytes0 = thread_alloc_current();
    thread_alloc_mark();

    // ---- Morton order and sorted sides
    for (int k = 0; k < 2; ++k) {
      const int64_t c = k == 0 ? n : m;
      codes[k] = (uint64_t*)dev_alloc(sizeof(uint64_t) * c);
      perm[k] = (int32_t*)dev_alloc(sizeof(int32_t) * c);
    }
    morton_sort_soa(p->X.soa, p->X.padded, p->Y.soa, p->Y.padded, n, m, d, st, codes[0], perm[0],
                    codes[1], perm[1]);
    alloc_side(Xs, n, d, st);
    alloc_side(Ys, m, d, st);
    hipLaunchKernelGGL(k_gather, grid1(((n + 255) / 256), 256), dim3(256), 0, st, p->X.soa,
                       p->X.padded, p->X.w, perm[0], n, d, Xs.soa, Xs.padded, Xs.w);
    SK_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_gather, grid1(((m + 255) / 256), 256), dim3(256), 0, st, p->Y.soa,
                       p->Y.padded, p->Y.w, perm[1], m, d, Ys.soa, Ys.padded, Ys.w);
    SK_LAUNCH_CHECK();
    if (!P.warm_start) {
      build_cells(p, Xs, codes[0], p_bits, Cx);
      build_cells(p, Ys, codes[1], p_bits, Cy);
    }
    R.ncells_x = Cx.count;
    R.ncells_y = Cy.count;
    SK_HIP(hipStreamSynchronize(st));
    const double t_sorted = now_s();
    R.seconds_sort = t_sorted - t_start;
    progress("multiscale: Morton order and cells done: %d x %d cells (%.3f s)", (int)R.ncells_x,
             (int)R.ncells_y, R.seconds_sort);

    // ---- coarse annealed solve on the cells
    auto need = [&](int64_t rows, int64_t cols) {
      ensure_partials(p, partial_floats_needed(p, rows, round_up(rows, kPad), cols));
    };
    if (!P.warm_start) {
      need(Cx.count, Cy.count);
      need(Cy.count, Cx.count);
      need(n, Cy.count);
      need(m, Cx.count);
    }
    pot[0] = (float*)dev_alloc(sizeof(float) * Cx.count);  // F
    pot[1] = (float*)dev_alloc(sizeof(float) * Cy.count);  // G
    pot[2] = (float*)dev_alloc(sizeof(float) * Cx.count);
    pot[3] = (float*)dev_alloc(sizeof(float) * Cx.count);
    pot[4] = (float*)dev_alloc(sizeof(float) * Cy.count);
    pot[5] = (float*)dev_alloc(sizeof(float) * Cy.count);
    fill_f32(pot[0], Cx.count, 0.0f, st);
    fill_f32(pot[1], Cy.count, 0.0f, st);
    float* CF[2] = {pot[2], pot[3]};
    float* CG[2] = {pot[4], pot[5]};
    sinkhorn_schedule cs;
    cs.eps_start = P.coarse_eps_start > P.eps ? P.coarse_eps_start : P.eps;
    cs.eps_target = P.eps;
    cs.eps_factor = P.coarse_factor;
    cs.iters_per_stage = P.coarse_iters_per_stage;
    cs.fixed_iters = 0;
    cs.tol = P.coarse_tol;
    cs.max_iters = P.coarse_max;
    cs.check_every = 1;
    float* fs[2] = {(float*)dev_alloc(sizeof(float) * n), (float*)dev_alloc(sizeof(float) * n)};
    pot[6] = fs[0];
    pot[7] = fs[1];
    float* gs[2] = {(float*)dev_alloc(sizeof(float) * m), (float*)dev_alloc(sizeof(float) * m)};
    pot[8] = gs[0];
    pot[9] = gs[1];
    const double eps = P.eps;
    // lift: f from the y cells, g from the x cells
    auto lift = [&]() {
      reset_nonfinite(p);
      prep_column_term(p, Cy, pot[1], eps, Cy.H);
      dense_halfstep(p, HalfStep{&Xs, &Cy, Cy.H, fs[0], nullptr, nullptr, eps, eps, false});
      prep_column_term(p, Cx, pot[0], eps, Cx.H);
      dense_halfstep(p, HalfStep{&Ys, &Cx, Cx.H, gs[0], nullptr, nullptr, eps, eps, false});
      R.pairs_evaluated += (double)n * (double)Cy.count + (double)m * (double)Cx.count;
      int32_t bad = 0;
      read_reduction(p, nullptr, &bad);
      if (bad) fail(SINKHORN_ERR_NONFINITE, "non-finite lifted potential");
    };
    bool accepted = false;
    double t_coarse, t_lift;
    if (P.warm_start) {
      // the fine loop starts from the caller's potentials (in Morton order)
      hipLaunchKernelGGL(k_gather_pot, grid1((n + 255) / 256, 256), dim3(256), 0, st, f, perm[0], n,
                         fs[0]);
      SK_LAUNCH_CHECK();
      hipLaunchKernelGGL(k_gather_pot, grid1((m + 255) / 256, 256), dim3(256), 0, st, g, perm[1], m,
                         gs[0]);
      SK_LAUNCH_CHECK();
      t_coarse = t_lift = now_s();
    } else if (!P.adaptive) {
      const SolveOut co = dense_solve(p, Cx, Cy, pot[0], pot[1], CF, CG, cs, P.stall_window, P.stall_rel);
      R.coarse_iters = co.iters;
      R.pairs_evaluated += co.pairs;
      t_coarse = now_s();
      R.seconds_coarse = t_coarse - t_sorted;
      progress("multiscale: coarse solve done: %d iterations (%.3f s)", (int)R.coarse_iters,
               R.seconds_coarse);
      lift();
      t_lift = now_s();
      R.seconds_lift = t_lift - t_coarse;
    } else {
      // batches of centroid updates, each followed by a lift and the sampled check
      need(P.check_samples_max, m);
      need(P.check_samples_max, n);
      SampleSide smp[2][2];  // [side][small, large sample]
      int64_t at_eps = 0;
      double lift_s = 0.0;
      for (bool first = true;; first = false) {
        sinkhorn_schedule bs = cs;
        if (!first) bs.eps_start = P.eps;
        const int64_t left = (int64_t)P.coarse_max - at_eps;
        bs.max_iters = (int32_t)(left < P.check_every ? (left > 0 ? left : 1) : P.check_every);
        const SolveOut co = dense_solve(p, Cx, Cy, pot[0], pot[1], CF, CG, bs, P.stall_window, P.stall_rel);
        R.coarse_iters += co.iters;
        R.pairs_evaluated += co.pairs;
        at_eps += co.final_iters;
        const bool done = co.converged || co.stalled;
        const double tl = now_s();
        lift();
        lift_s += now_s() - tl;
        int32_t K = P.check_samples;
        double er = 0.0, sr = 0.0, ec = 0.0, sc = 0.0;
        while (true) {
          const int big = K == P.check_samples ? 0 : 1;
          prep_column_term(p, Ys, gs[0], eps, Ys.H);
          sampled_residual(p, Xs, Ys, fs[0], eps, P.sample_seed, 0, K, smp[0][big], &er, &sr);
          prep_column_term(p, Xs, fs[0], eps, Xs.H);
          sampled_residual(p, Ys, Xs, gs[0], eps, P.sample_seed, 1, K, smp[1][big], &ec, &sc);
          R.pairs_evaluated += (double)K * (double)(n + m);
          const double hi = std::max(er + 3.0 * sr, ec + 3.0 * sc);
          const double lo = std::max(er - 3.0 * sr, ec - 3.0 * sc);
          if (hi < P.tol) {
            accepted = true;
            break;
          }
          if (lo >= P.tol || K >= P.check_samples_max) break;
          K = P.check_samples_max;
        }
        ++R.checks;
        R.last_check_samples = K;
        R.last_check[0] = er;
        R.last_check[1] = sr;
        R.last_check[2] = ec;
        R.last_check[3] = sc;
        progress("multiscale: check %d after %d coarse updates: row %.4g +- %.3g, column %.4g +- %.3g "
                 "(%d samples) -> %s", (int)R.checks, (int)R.coarse_iters, er, sr, ec, sc, (int)K,
                 accepted ? "accepted" : (done || at_eps >= P.coarse_max ? "fine updates" : "more coarse"));
        if (accepted || done || at_eps >= P.coarse_max) break;
      }
      t_lift = now_s();
      R.seconds_lift = lift_s;
      R.seconds_coarse = t_lift - t_sorted - lift_s;
      t_coarse = t_lift - lift_s;
    }
    (void)t_coarse;
    for (int k = 2; k < 6; ++k) {
      dev_free(pot[k]);
      pot[k] = nullptr;
    }
    progress("multiscale: lift done (%.3f s)", R.seconds_lift);
    R.accepted_by_sample = accepted ? 1 : 0;

    // ---- fine loop on the block-pair mask
    block_static(p, Xs, P.B, sx);
    block_static(p, Ys, P.B, sy);
    frame_build(p, Xs, P.B, lx);
    frame_build(p, Ys, P.B, ly);
    TileList rowL, colL;
    VerifiedList rowV, colV;
    VerifyScratch vscr;
    int cf = 0, cg = 0;
    int status = accepted ? SINKHORN_OK : SINKHORN_NOT_CONVERGED;
    double Rrow = NAN, Rcol = NAN;
    const double pair_block = (double)P.B * (double)P.B;
    while (!accepted) {
      block_potential_max(p, fs[cf], n, sx);
      block_potential_max(p, gs[cg], m, sy);
      rowL.build(p, sx, sy, eps, delta);
      const int64_t *rptr = rowL.ptr, *cptr = nullptr;
      const int32_t *ridx = rowL.idx, *cidx = nullptr;
      int64_t rnnz = rowL.nnz, cnnz = 0;
      if (P.verify) {
        // the exact share check at (f, g) on the screened tiles; both lists
        // come from the survivors
        rowV.reserve(p, sx.nb, rowL.nnz);
        colV.reserve(p, sy.nb, rowL.nnz);
        const int64_t kept = verify_tiles(p, Xs, Ys, fs[cf], gs[cg], eps, delta, rowL.ptr, rowL.idx,
                                          rowL.nnz, sx.nb, sy.nb, rowV.ptr, rowV.idx, colV.ptr,
                                          colV.idx, vscr);
        rowV.nnz = colV.nnz = kept;
        rptr = rowV.ptr;
        ridx = rowV.idx;
        cptr = colV.ptr;
        cidx = colV.idx;
        rnnz = cnnz = kept;
      } else {
        colL.build(p, sy, sx, eps, delta);
        cptr = colL.ptr;
        cidx = colL.idx;
        cnnz = colL.nnz;
      }
      R.last_candidates = rowL.nnz;
      R.last_tiles = rnnz;
      const double row_pairs = (double)rnnz * pair_block +
                               (double)count_empty_rows(p, rptr, sx.nb) * P.B * (double)m;
      const double col_pairs = (double)cnnz * pair_block +
                               (double)count_empty_rows(p, cptr, sy.nb) * P.B * (double)n;
      // sparse f-step at (f, g); its fused residual is R_A,row of (f, g)
      reset_nonfinite(p);
      prep_column_term(p, Ys, gs[cg], eps, Ys.H);
      sparse_halfstep(p, HalfStep{&Xs, &Ys, Ys.H, fs[1 - cf], fs[cf], nullptr, eps, eps, true, fs[cf],
                                  &ly, gs[cg]},
                      P.B, rptr, ridx, row_pairs);
      int32_t bad = 0;
      read_reduction(p, &Rrow, &bad);
      if (bad) fail(SINKHORN_ERR_NONFINITE, "non-finite potential in the fine loop");
      R.pairs_evaluated += row_pairs;
      Rcol = NAN;
      if (Rrow + omega <= P.tol) {
        prep_column_term(p, Xs, fs[cf], eps, Xs.H);
        sparse_halfstep(p, HalfStep{&Ys, &Xs, Xs.H, gs[1 - cg], gs[cg], nullptr, eps, eps, true, gs[cg],
                                    &lx, fs[cf]},
                        P.B, cptr, cidx, col_pairs);
        read_reduction(p, &Rcol, nullptr);
        R.pairs_evaluated += col_pairs;
        if ((Rrow > Rcol ? Rrow : Rcol) + omega <= P.tol) {
          status = SINKHORN_OK;
          R.certified = 1;
          break;
        }
      }
      progress("multiscale: fine update %d: %lld row / %lld column tiles (%lld screened), R_A row "
               "%.4g column %.4g (%.3f s)", (int)R.fine_updates, (long long)rnnz, (long long)cnnz,
               (long long)rowL.nnz, Rrow, Rcol, now_s() - t_lift);
      if (R.fine_updates >= P.max_fine) break;
      cf = 1 - cf;  // accept the f-step
      prep_column_term(p, Xs, fs[cf], eps, Xs.H);
      sparse_halfstep(p, HalfStep{&Ys, &Xs, Xs.H, gs[1 - cg], nullptr, nullptr, eps, eps, false, gs[cg],
                                  &lx, fs[cf]},
                      P.B, cptr, cidx, col_pairs);
      R.pairs_evaluated += col_pairs;
      cg = 1 - cg;
      ++R.fine_updates;
    }
    R.R_A_row = Rrow;
    R.R_A_col = Rcol;
    // ---- back to the caller's order
    hipLaunchKernelGGL(k_scatter, grid1(((n + 255) / 256), 256), dim3(256), 0, st, fs[cf],
                       perm[0], n, f);
    SK_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_scatter, grid1(((m + 255) / 256), 256), dim3(256), 0, st, gs[cg],
                       perm[1], m, g);
    SK_LAUNCH_CHECK();
    SK_HIP(hipStreamSynchronize(st));
    const double t_end = now_s();
    R.seconds_fine = t_end - t_lift;
    R.seconds_total = t_end - t_start;
    R.peak_extra_bytes = thread_alloc_peak() - bytes0;
    if (rep) *rep = R;
    cleanup();
    return status;
  } catch (const Failure& e) {
    cleanup();
    set_last_error(e.msg);
    return e.code;
  } catch (...) {
    cleanup();
    set_last_error("unexpected exception");
    return SINKHORN_ERR_HIP;
  }
}

extern "C" int sinkhorn_sample_indices(int64_t count, int32_t k, uint64_t seed, uint64_t stream_id,
                                       void* stream, int32_t* out) {
  try {
    if (!out && k > 0) fail(SINKHORN_ERR_INVALID_ARG, "null pointer");
    if (count < 1 || count > INT32_MAX || k < 0) fail(SINKHORN_ERR_INVALID_ARG, "need 1 <= count <= 2^31 - 1 and k >= 0");
    if (k == 0) return SINKHORN_OK;
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(k_sample_idx, grid1(((k + 255) / 256), 256), dim3(256), 0, st, seed, stream_id,
                       count, k, out);
    SK_LAUNCH_CHECK();
    SK_HIP(hipStreamSynchronize(st));
    return SINKHORN_OK;
  } catch (const Failure& e) {
    set_last_error(e.msg);
    return e.code;
  } catch (...) {
    set_last_error("unexpected exception");
    return SINKHORN_ERR_HIP;
  }
}

extern "C" int sinkhorn_sampled_residual(sinkhorn_problem* p, double eps, const float* f, const float* g,
                                         int32_t side, int32_t k, uint64_t seed, double* est,
                                         double* se) {
  try {
    if (!p || !f || !g || !est || !se) fail(SINKHORN_ERR_INVALID_ARG, "null pointer");
    if (!(std::isfinite(eps) && eps > 0.0)) fail(SINKHORN_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (side != 0 && side != 1) fail(SINKHORN_ERR_INVALID_ARG, "side must be 0 (rows) or 1 (columns)");
    if (k < 2 || k > (1 << 24)) fail(SINKHORN_ERR_INVALID_ARG, "need 2 <= k <= 2^24");
    if (p->d > kMaxValuD) fail(SINKHORN_ERR_UNSUPPORTED, "sampled residual needs d <= 8");
    const Side& rows = side == 0 ? p->X : p->Y;
    Side& cols = side == 0 ? p->Y : p->X;
    ensure_partials(p, partial_floats_needed(p, k, round_up(k, kPad), cols.count));
    prep_column_term(p, cols, side == 0 ? g : f, eps, cols.H);
    reset_nonfinite(p);
    SampleSide S;
    sampled_residual(p, rows, cols, side == 0 ? f : g, eps, seed, (uint64_t)side, k, S, est, se);
    int32_t bad = 0;
    read_reduction(p, nullptr, &bad);
    if (bad) fail(SINKHORN_ERR_NONFINITE, "non-finite potential in the sampled check");
    return SINKHORN_OK;
  } catch (const Failure& e) {
    set_last_error(e.msg);
    return e.code;
  } catch (...) {
    set_last_error("unexpected exception");
    return SINKHORN_ERR_HIP;
  }
}
