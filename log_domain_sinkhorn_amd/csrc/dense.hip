// Dense online half-step for small d (difference form on VALU), its finalize
// step (split merge, potential, fused residual, next column term) and the
// deterministic reductions.
//
// FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport, §2.1: a half-step
// is a tiled streaming log-sum-exp over all pairs that never stores the cost.
// Here one lane owns R rows; the column tile (coordinates and column term) is
// wave-uniform and arrives through scalar loads, so every pair costs d subs,
// d squares (1 mul + d-1 fma), one fma for the exponent, one max, one sub, one
// exp2 and one add, all on the vector ALU.
#include <cfloat>
#include <cmath>
#include <cstring>

#include "internal.h"

namespace sk {
namespace {

// Base-2 exponential of the hardware (v_exp_f32). Arguments are <= 0 or -inf
// here, where it is accurate to about 1 ulp; -inf gives +0.
__device__ __forceinline__ float ex2(float v) { return __builtin_amdgcn_exp2f(v); }

// One wave = 64 lanes x R rows against the column range of one split.
// Block = 4 waves on 4 consecutive row tiles, all on the same split so the
// scalar-loaded column tile is shared through the scalar cache.
template <int D, int R>
__global__ __launch_bounds__(256) void k_lse_valu(
    const float* __restrict__ P, int64_t pstride,      // row side, SoA [D][pstride]
    const float* __restrict__ Q, int64_t qstride,      // column side, SoA [D][qstride]
    const float* __restrict__ H,                       // column term, log2 units
    float nkappa,                                      // -s * log2(e) / eps
    int64_t nchunks, int64_t chunks_per_split, int32_t nsplit, int64_t np,
    float* __restrict__ Mp, float* __restrict__ Sp, int64_t part_stride) {
  const int32_t s = (int32_t)(blockIdx.x % (uint32_t)nsplit);
  const int64_t rg = blockIdx.x / (uint32_t)nsplit;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t row0 = (rg * 4 + wave) * (64 * R) + lane;

  float x[R][D];
  float M[R], S[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int k = 0; k < D; ++k) x[r][k] = P[k * pstride + row0 + 64 * r];
    M[r] = -FLT_MAX;
    S[r] = 0.0f;
  }
  const float nk = nkappa;

  const int64_t c0 = (int64_t)s * chunks_per_split;
  const int64_t c1 = c0 + chunks_per_split < nchunks ? c0 + chunks_per_split : nchunks;
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t j0 = c * kChunk;
    float yv[D][kChunk];
    float hv[kChunk];
#pragma unroll
    for (int k = 0; k < D; ++k)
#pragma unroll
      for (int jj = 0; jj < kChunk; ++jj) yv[k][jj] = Q[k * qstride + j0 + jj];
#pragma unroll
    for (int jj = 0; jj < kChunk; ++jj) hv[jj] = H[j0 + jj];

#pragma unroll
    for (int r = 0; r < R; ++r) {
      float z[kChunk];
#pragma unroll
      for (int jj = 0; jj < kChunk; ++jj) {
        float dd = x[r][0] - yv[0][jj];
        float q = dd * dd;
#pragma unroll
        for (int k = 1; k < D; ++k) {
          dd = x[r][k] - yv[k][jj];
          q = __builtin_fmaf(dd, dd, q);
        }
        z[jj] = __builtin_fmaf(nk, q, hv[jj]);
      }
      float cm = z[0];
#pragma unroll
      for (int jj = 1; jj < kChunk; ++jj) cm = fmaxf(cm, z[jj]);
      const float Mn = fmaxf(M[r], cm);
      float acc = 0.0f;
#pragma unroll
      for (int jj = 0; jj < kChunk; ++jj) acc += ex2(z[jj] - Mn);
      S[r] = __builtin_fmaf(S[r], ex2(M[r] - Mn), acc);
      M[r] = Mn;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = row0 + 64 * r;
    if (i < np) {
      Mp[(int64_t)s * part_stride + i] = M[r];
      Sp[(int64_t)s * part_stride + i] = S[r];
    }
  }
}

// Deterministic block sum of one double per thread (256 threads).
__device__ double block_sum_256(double v) {
  __shared__ double sh[256];
  sh[threadIdx.x] = v;
  __syncthreads();
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  return sh[0];
}

// Merge the split partials of each row (fp64), write the potential, optionally
// the next column term of this side and the residual term
//   w_i |exp((prev_i - new_i)/eps) - 1|,
// summed per block into red_part.
__global__ __launch_bounds__(256) void k_finalize(
    const float* __restrict__ Mp, const float* __restrict__ Sp, int64_t part_stride,
    int32_t nsplit, int64_t np, double neg_eps_ln2, float* __restrict__ out,
    const float* __restrict__ prev, const float* __restrict__ w, double inv_eps,
    float* __restrict__ Hnext, double lam_next, double* __restrict__ red_part,
    int32_t* __restrict__ nonfinite) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  double term = 0.0;
  if (i < np) {
    double mx = -INFINITY;
    for (int32_t s = 0; s < nsplit; ++s) mx = fmax(mx, (double)Mp[(int64_t)s * part_stride + i]);
    double sum = 0.0;
    for (int32_t s = 0; s < nsplit; ++s) {
      const int64_t o = (int64_t)s * part_stride + i;
      sum += (double)Sp[o] * exp2((double)Mp[o] - mx);
    }
    const double L = mx + log2(sum);  // sum == 0 -> -inf -> potential +inf
    const double v = neg_eps_ln2 * L;
    const float v32 = (float)v;
    out[i] = v32;
    if (!isfinite(v32)) atomicAdd(nonfinite, 1);
    const double wi = (double)w[i];
    if (Hnext) Hnext[i] = (float)(log2(wi) + (double)v32 * lam_next);
    if (prev && wi > 0.0) term = wi * fabs(expm1(((double)prev[i] - v) * inv_eps));
  }
  if (red_part) {
    const double b = block_sum_256(term);
    if (threadIdx.x == 0) red_part[blockIdx.x] = b;
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

// Sum of count doubles in a fixed order (one block of 256 threads).
__global__ __launch_bounds__(256) void k_reduce(const double* __restrict__ part, int64_t count,
                                                double* __restrict__ out) {
  double acc = 0.0;
  for (int64_t k = threadIdx.x; k < count; k += 256) acc += part[k];
  const double s = block_sum_256(acc);
  if (threadIdx.x == 0) out[0] = s;
}

struct SplitPlan {
  int R;
  int32_t nsplit;
  int64_t cps;  // chunks per split
  int64_t nchunks;
  int64_t groups;  // row groups of 4 waves
};

constexpr int kRowsPerLane = 2;

SplitPlan plan_split(int64_t nrows, int64_t ncols) {
  SplitPlan sp;
  sp.R = kRowsPerLane;
  sp.nchunks = (ncols + kChunk - 1) / kChunk;
  sp.groups = (nrows + 256 * sp.R - 1) / (256 * sp.R);
  // aim at ~1024 workgroups (4096 waves) so all 256 CUs stay busy
  int64_t want = (1024 + sp.groups - 1) / sp.groups;
  int64_t maxsplit = sp.nchunks / 4 > 1 ? sp.nchunks / 4 : 1;  // >= 4 chunks per split
  if (want > 64) want = 64;
  if (want > maxsplit) want = maxsplit;
  if (want < 1) want = 1;
  if (want > 8) want = (want + 7) / 8 * 8;  // split -> XCD alignment
  sp.cps = (sp.nchunks + want - 1) / want;
  sp.nsplit = (int32_t)((sp.nchunks + sp.cps - 1) / sp.cps);
  return sp;
}

template <int D>
void launch_lse(sinkhorn_problem* p, const Side& rows, const Side& cols, const float* H,
                float nkappa, const SplitPlan& sp) {
  const dim3 grid((uint32_t)(sp.groups * sp.nsplit));
  hipLaunchKernelGGL((k_lse_valu<D, kRowsPerLane>), grid, dim3(256), 0, p->stream, rows.soa,
                     rows.padded, cols.soa, cols.padded, H, nkappa, sp.nchunks, sp.cps,
                     sp.nsplit, rows.count, p->Mpart, p->Spart, rows.padded);
  SK_LAUNCH_CHECK();
}

}  // namespace

int64_t partial_floats_needed(const sinkhorn_problem* p, int64_t nrows, int64_t rows_padded,
                              int64_t ncols) {
  (void)p;
  const SplitPlan sp = plan_split(nrows, ncols);
  return (int64_t)sp.nsplit * rows_padded;
}

void prep_column_term(sinkhorn_problem* p, const Side& side, const float* pot, double eps,
                      float* H) {
  const int64_t blocks = (side.count + 255) / 256;
  hipLaunchKernelGGL(k_column_term, dim3((uint32_t)blocks), dim3(256), 0, p->stream, side.w, pot,
                     side.count, kLog2e / eps, H);
  SK_LAUNCH_CHECK();
}

void dense_halfstep(sinkhorn_problem* p, const HalfStep& hs) {
  const Side& rows = *hs.rows;
  const Side& cols = *hs.cols;
  const SplitPlan sp = plan_split(rows.count, cols.count);
  if ((int64_t)sp.nsplit * rows.padded > p->part_cap) fail(SINKHORN_ERR_HIP, "partial buffer too small");
  const float nkappa = (float)(-p->scale * kLog2e / hs.eps);
  switch (p->d) {
    case 1: launch_lse<1>(p, rows, cols, hs.Hcols, nkappa, sp); break;
    case 2: launch_lse<2>(p, rows, cols, hs.Hcols, nkappa, sp); break;
    case 3: launch_lse<3>(p, rows, cols, hs.Hcols, nkappa, sp); break;
    case 4: launch_lse<4>(p, rows, cols, hs.Hcols, nkappa, sp); break;
    case 5: launch_lse<5>(p, rows, cols, hs.Hcols, nkappa, sp); break;
    case 6: launch_lse<6>(p, rows, cols, hs.Hcols, nkappa, sp); break;
    case 7: launch_lse<7>(p, rows, cols, hs.Hcols, nkappa, sp); break;
    case 8: launch_lse<8>(p, rows, cols, hs.Hcols, nkappa, sp); break;
    default: fail(SINKHORN_ERR_UNSUPPORTED, "VALU half-step supports d <= 8");
  }
  const int64_t fblocks = (rows.count + 255) / 256;
  if (hs.residual && fblocks > p->red_cap) fail(SINKHORN_ERR_HIP, "reduction buffer too small");
  hipLaunchKernelGGL(k_finalize, dim3((uint32_t)fblocks), dim3(256), 0, p->stream, p->Mpart,
                     p->Spart, rows.padded, sp.nsplit, rows.count, -hs.eps * kLn2, hs.pot_out,
                     hs.residual ? hs.pot_prev : nullptr, rows.w, 1.0 / hs.eps, hs.H_next,
                     kLog2e / hs.eps_next, hs.residual ? p->red_part : nullptr, p->nonfinite);
  SK_LAUNCH_CHECK();
  if (hs.residual) {
    hipLaunchKernelGGL(k_reduce, dim3(1), dim3(256), 0, p->stream, p->red_part, fblocks,
                       p->red_out);
    SK_LAUNCH_CHECK();
  }
}

void reset_nonfinite(sinkhorn_problem* p) { zero_i32(p->nonfinite, 1, p->stream); }

void read_reduction(sinkhorn_problem* p, double* value, int32_t* nonfinite) {
  SK_HIP(hipMemcpyAsync(p->host_red, p->red_out, sizeof(double), hipMemcpyDeviceToHost, p->stream));
  SK_HIP(hipMemcpyAsync(p->host_red + 1, p->nonfinite, sizeof(int32_t), hipMemcpyDeviceToHost,
                        p->stream));
  SK_HIP(hipStreamSynchronize(p->stream));
  if (value) *value = p->host_red[0];
  if (nonfinite) {
    int32_t v;
    memcpy(&v, p->host_red + 1, sizeof(int32_t));
    *nonfinite = v;
  }
}

}  // namespace sk
