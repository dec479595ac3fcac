// Transport-plan rows and the min_row threshold.
//
// moscot pull request #846, "Fix": entropic rows are built directly from the
// potentials, T[rows] = exp((f_i + g_j - C_ij)/eps) with the weights carried
// by the plan (T_ij = a_i b_j exp((f_i + g_j - C_ij)/eps) here), never through
// an n x m x k tensor; "Behavioural changes": min_row = min over rows with
// a_i > 0 of max_j T_ij, exact and independent of the row batch.
//
// The exponent E_ij = log2 T_ij is assembled in fp64 from per-row and
// per-column terms and rounded once before the fp32 exp2, so a row entry
// carries about |E| 2^-24 ln 2 relative error. Row maxima are exact: each
// workgroup reduces its share and merges it with an atomic max on an
// order-preserving integer key of E (max is order independent).
#include <cfloat>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>

#include <rocprim/device/device_scan.hpp>

#include "internal.h"

namespace sk {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float ex2(float v) { return __builtin_amdgcn_exp2f(v); }

// Monotone map float -> uint32 (larger float, larger key).
__device__ __forceinline__ uint32_t okey(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float okey_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Row terms for the selected rows: P_i = log2 a_i + lam f_i [- kappa ||x_i||^2].
__global__ __launch_bounds__(256) void k_row_terms(const int64_t* __restrict__ rows, int64_t row0,
                                                   int64_t k, const float* __restrict__ a,
                                                   const float* __restrict__ f,
                                                   const float* __restrict__ norm2, double lam,
                                                   double kappa, double* __restrict__ P,
                                                   int32_t* __restrict__ live,
                                                   uint32_t* __restrict__ keys) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= k) return;
  const int64_t i = rows ? rows[r] : row0 + r;
  double v = log2((double)a[i]) + lam * (double)f[i];
  if (norm2) v -= kappa * (double)norm2[i];
  P[r] = v;
  if (live) live[r] = a[i] > 0.0f ? 1 : 0;
  keys[r] = 0u;  // below every finite key
}

// Column terms (VALU path): Hd_j = log2 b_j + lam g_j in fp64.
__global__ __launch_bounds__(256) void k_col_terms(const float* __restrict__ b,
                                                  const float* __restrict__ g, int64_t m,
                                                  double lam, double* __restrict__ Hd) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j < m) Hd[j] = log2((double)b[j]) + lam * (double)g[j];
}

constexpr int kRB = 8;  // rows per workgroup (VALU materializer)

// VALU path (d <= 8): thread = column j (coalesced stores), kRB rows per block.
template <int D>
__global__ __launch_bounds__(256) void k_materialize_valu(
    const float* __restrict__ X, int64_t xs, const float* __restrict__ Y, int64_t ys, int64_t m,
    const int64_t* __restrict__ rows, int64_t row0, int64_t k, const double* __restrict__ P,
    const double* __restrict__ Hd, double kappa, float* __restrict__ T,
    uint32_t* __restrict__ keys) {
  __shared__ uint32_t sKey[256];
  const int64_t j = (int64_t)blockIdx.y * 256 + threadIdx.x;
  const int64_t rb = (int64_t)blockIdx.x * kRB;
  float yv[D];
  double hj = -INFINITY;
  if (j < m) {
#pragma unroll
    for (int q = 0; q < D; ++q) yv[q] = Y[q * ys + j];
    hj = Hd[j];
  } else {
#pragma unroll
    for (int q = 0; q < D; ++q) yv[q] = 0.0f;
  }
  for (int r = 0; r < kRB; ++r) {
    const int64_t rr = rb + r;
    if (rr >= k) break;  // uniform
    const int64_t i = rows ? rows[rr] : row0 + rr;
    // fp64 difference form: the fp32 coordinates subtract exactly, so the
    // exponent of a far entry (large kappa q) keeps full relative accuracy
    double dd = (double)X[i] - (double)yv[0];
    double q = dd * dd;
#pragma unroll
    for (int c = 1; c < D; ++c) {
      dd = (double)X[c * xs + i] - (double)yv[c];
      q = __builtin_fma(dd, dd, q);
    }
    const double E = __builtin_fma(-kappa, q, P[rr] + hj);
    const float e32 = (float)E;
    if (T && j < m) T[rr * m + j] = ex2(e32);
    sKey[threadIdx.x] = j < m ? okey(e32) : 0u;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) sKey[threadIdx.x] = max(sKey[threadIdx.x], sKey[threadIdx.x + w]);
      __syncthreads();
    }
    if (threadIdx.x == 0) atomicMax(&keys[rr], sKey[0]);
    __syncthreads();
  }
}

// max of two floats in one v_max_f32: fmaxf would first copy each operand
// through v_max(x, x) to quiet a signalling NaN, and neither operand can be
// one here (MFMA results and maxima of them)
__device__ __forceinline__ float vmax_f32(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// MFMA path (9 <= d <= 63): A = selected x rows scaled by 2 kappa (slot d :=
// 2 kappa, slot KP - 1 := the fp32 part P_hi of the row term), B = column
// tile of y from LDS (slot d = H'_j, slot KP - 1 = 1), so the chain yields
// 2 kappa (x_i . y_j + H'_j) + P_hi and E = that + P_lo (P_lo = P_i - P_hi in
// fp32): one add, one exp2 and one max per entry besides the store. The
// row maximum is taken before the add (rounding is monotone, so it equals
// the maximum of the stored exponents).
// A wave owns one tile of 32 rows (so the A fragment, accumulators, row terms
// and row maxima of a lane stay small enough for several waves per SIMD);
// lane (l32, kh) holds rows 8(r/4) + 4kh + r%4 at column l32, so the T stores
// are 128-byte row segments.
template <int KP>
__global__ __launch_bounds__(256) void k_materialize_mfma(
    const float* __restrict__ X, const float* __restrict__ Y, int32_t d, int64_t m,
    const int64_t* __restrict__ rows, int64_t row0, int64_t k, const double* __restrict__ P,
    double twokappa, int32_t G, int64_t ntiles, int64_t tps, float* __restrict__ T,
    uint32_t* __restrict__ keys) {
  constexpr int KH = KP / 2;
  constexpr int LW = KP + 1;
  constexpr int NV4 = 32 * KP / 4;
  constexpr int PER = (NV4 + 255) / 256;
  __shared__ float sY[2][32 * LW];
  const int32_t gs = (int32_t)(blockIdx.x % (uint32_t)G);
  const int64_t rt = blockIdx.x / (uint32_t)G;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int kh = lane >> 5;
  const int64_t rbase = rt * 128 + wave * 32;  // first selected row of this wave
  const float tk = (float)twokappa;

  float ax[KH];
  {
    const int64_t rr = rbase + l32;
    const int64_t i = rr < k ? (rows ? rows[rr] : row0 + rr) : -1;
    const float phi = i < 0 ? 0.0f : (float)P[rr];
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
      const int c = 2 * kk + kh;
      ax[kk] = i < 0 ? 0.0f : (c == KP - 1 ? phi : (c == d ? tk : tk * X[i * KP + c]));
    }
  }
  float plo[16], emax[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t rr = rbase + 8 * (r / 4) + 4 * kh + (r % 4);
    const double pr = rr < k ? P[rr] : 0.0;
    plo[r] = (float)(pr - (double)(float)pr);
    emax[r] = -INFINITY;
  }
  const int nrows = rbase + 32 <= k ? 32 : (int)(k - rbase);  // rows of this wave that exist
  float* Tw = (T && nrows > 0) ? T + (rbase + 4 * kh) * m : nullptr;

  const int64_t t0 = (int64_t)gs * tps;
  const int64_t t1 = t0 + tps < ntiles ? t0 + tps : ntiles;
  float4 pre[PER];
  auto gload = [&](int64_t t) {
    const float4* src = reinterpret_cast<const float4*>(Y + t * 32 * KP);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int idx = threadIdx.x + q * 256;
      if (idx < NV4) pre[q] = src[idx];
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int idx = threadIdx.x + q * 256;
      if (idx < NV4) {
        const int e = idx * 4;
        float* dst = &sY[buf][(e / KP) * LW + (e % KP)];
        dst[0] = pre[q].x;
        dst[1] = pre[q].y;
        dst[2] = pre[q].z;
        dst[3] = pre[q].w;
      }
    }
  };
  if (t0 < t1) {
    gload(t0);
    lstore(0);
  }
  __syncthreads();
  int buf = 0;
  for (int64_t t = t0; t < t1; ++t) {
    const bool more = t + 1 < t1;
    if (more) gload(t + 1);
    v16f acc = (v16f){};
    const float* ys = &sY[buf][l32 * LW + kh];
    float yb[KH];
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) yb[kk] = ys[2 * kk];
    // all B fragments in flight before the first MFMA waits on one
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KH; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(ax[kk], yb[kk], acc, 0, 0, 0);
    const int64_t j = t * 32 + l32;
    if (Tw) {
      float* Tj = Tw + j;
      if ((t + 1) * 32 <= m && nrows == 32) {
#pragma unroll
        for (int r = 0; r < 16; ++r) Tj[(int64_t)(8 * (r / 4) + (r % 4)) * m] = ex2(acc[r] + plo[r]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = 8 * (r / 4) + 4 * kh + (r % 4);  // row within the wave's tile
          if (j < m && lr < nrows) Tj[(int64_t)(8 * (r / 4) + (r % 4)) * m] = ex2(acc[r] + plo[r]);
        }
      }
    }
    // padding columns give -inf (their column term), absent rows are not read
#pragma unroll
    for (int r = 0; r < 16; ++r) emax[r] = vmax_f32(emax[r], acc[r]);
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  // max over the 32 columns held by the lanes of each half
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float v = emax[r];
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    const int64_t rr = rbase + 8 * (r / 4) + 4 * kh + (r % 4);
    if (l32 == 0 && rr < k && v > -INFINITY) atomicMax(&keys[rr], okey(v + plo[r]));
  }
}

// row_max[r] = exp2(E max) from the keys (0 key: no column -> 0).
__global__ __launch_bounds__(256) void k_keys_to_max(const uint32_t* __restrict__ keys, int64_t k,
                                                     float* __restrict__ row_max) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r < k) row_max[r] = keys[r] == 0u ? 0.0f : ex2(okey_inv(keys[r]));
}

// min over live rows of exp2(E max), into one key slot (order independent).
__global__ __launch_bounds__(256) void k_min_live(const uint32_t* __restrict__ keys,
                                                  const int32_t* __restrict__ live, int64_t k,
                                                  uint32_t* __restrict__ out_key) {
  __shared__ uint32_t sm[256];
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t v = 0xffffffffu;
  if (r < k && live[r]) v = keys[r];
  sm[threadIdx.x] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) sm[threadIdx.x] = min(sm[threadIdx.x], sm[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMin(out_key, sm[0]);
}

__global__ void k_set_u32(uint32_t* p, uint32_t v) {
  if (threadIdx.x == 0) *p = v;
}

// Count of row indices outside [0, n).
__global__ __launch_bounds__(256) void k_check_rows(const int64_t* __restrict__ rows, int64_t k,
                                                    int64_t n, uint32_t* __restrict__ bad) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r < k && (rows[r] < 0 || rows[r] >= n)) atomicAdd(bad, 1u);
}

template <int D>
void launch_valu(sinkhorn_problem* p, const int64_t* rows, int64_t row0, int64_t k,
                 const double* P, const double* Hd, double kappa, float* T, uint32_t* keys,
                 const ProfEv& pe) {
  const dim3 grid((uint32_t)((k + kRB - 1) / kRB), (uint32_t)((p->m + 255) / 256));
  hipExtLaunchKernelGGL((k_materialize_valu<D>), grid, dim3(256), 0, p->stream, pe.start, pe.stop, 0,
                        p->X.soa, p->X.padded, p->Y.soa, p->Y.padded, p->m, rows, row0, k, P, Hd,
                        kappa, T, keys);
  SK_LAUNCH_CHECK();
}

template <int KP>
void launch_mfma(sinkhorn_problem* p, const int64_t* rows, int64_t row0, int64_t k,
                 const double* P, double twokappa, float* T, uint32_t* keys, const ProfEv& pe) {
  const int64_t rtiles = (k + 127) / 128;
  const int64_t ntiles = (p->m + 31) / 32;
  // about two workgroups per CU, each streaming a long column range: shorter
  // ranges (more workgroups) measured slower, the per-workgroup set-up and
  // the row-maximum epilogue then weigh more
  int64_t want = (2 * (int64_t)p->num_cu + rtiles - 1) / rtiles;
  const int64_t maxsplit = ntiles / 4 > 1 ? ntiles / 4 : 1;
  if (want > maxsplit) want = maxsplit;
  if (want < 1) want = 1;
  const int64_t tps = (ntiles + want - 1) / want;
  const int32_t G = (int32_t)((ntiles + tps - 1) / tps);
  hipExtLaunchKernelGGL((k_materialize_mfma<KP>), grid1((rtiles * G), 256), dim3(256), 0,
                        p->stream, pe.start, pe.stop, 0, p->X.rowmaj, p->Y.rowmaj, p->d, p->m, rows,
                        row0, k, P, twokappa, G, ntiles, tps, T, keys);
  SK_LAUNCH_CHECK();
}

// Rows [row0, row0 + k) (rows == null) or rows[0..k): T (nullable) and keys.
void rows_pass(sinkhorn_problem* p, double eps, const float* f, const int64_t* rows, int64_t row0,
               int64_t k, double* P, int32_t* live, uint32_t* keys, const double* Hd, float* T) {
  const double lam = kLog2e / eps;
  const double kappa = p->scale * lam;
  const bool mf = p->d > kMaxValuD;
  hipLaunchKernelGGL(k_row_terms, grid1(((k + 255) / 256), 256), dim3(256), 0, p->stream, rows,
                     row0, k, p->X.w, f, mf ? p->X.norm2 : nullptr, lam, kappa, P, live, keys);
  SK_LAUNCH_CHECK();
  const ProfEv pe = prof_events(p, SINKHORN_PROF_MATERIALIZE);
  if (mf) {
    switch (p->kpad) {
#define SK_KP(v) case v: launch_mfma<v>(p, rows, row0, k, P, 2.0 * kappa, T, keys, pe); break;
      SK_KP(12) SK_KP(16) SK_KP(20) SK_KP(24) SK_KP(28) SK_KP(32) SK_KP(36)
      SK_KP(40) SK_KP(44) SK_KP(48) SK_KP(52) SK_KP(56) SK_KP(60) SK_KP(64) SK_KP(68)
#undef SK_KP
      default: fail(SINKHORN_ERR_UNSUPPORTED, "materializer: unsupported K");
    }
  } else {
    switch (p->d) {
      case 1: launch_valu<1>(p, rows, row0, k, P, Hd, kappa, T, keys, pe); break;
      case 2: launch_valu<2>(p, rows, row0, k, P, Hd, kappa, T, keys, pe); break;
      case 3: launch_valu<3>(p, rows, row0, k, P, Hd, kappa, T, keys, pe); break;
      case 4: launch_valu<4>(p, rows, row0, k, P, Hd, kappa, T, keys, pe); break;
      case 5: launch_valu<5>(p, rows, row0, k, P, Hd, kappa, T, keys, pe); break;
      case 6: launch_valu<6>(p, rows, row0, k, P, Hd, kappa, T, keys, pe); break;
      case 7: launch_valu<7>(p, rows, row0, k, P, Hd, kappa, T, keys, pe); break;
      case 8: launch_valu<8>(p, rows, row0, k, P, Hd, kappa, T, keys, pe); break;
      default: fail(SINKHORN_ERR_UNSUPPORTED, "materializer: unsupported d");
    }
  }
  prof_done(p, SINKHORN_PROF_MATERIALIZE, (double)k * (double)p->m);
}

// Column terms for this eps and g: the MFMA path writes H'_j into slot d of y,
// the VALU path fills Hd (fp64, caller-owned).
void column_terms(sinkhorn_problem* p, double eps, const float* g, double* Hd) {
  if (p->d > kMaxValuD) {
    mfma_column_term(p, p->Y, g, eps);
  } else {
    hipLaunchKernelGGL(k_col_terms, grid1(((p->m + 255) / 256), 256), dim3(256), 0, p->stream,
                       p->Y.w, g, p->m, kLog2e / eps, Hd);
    SK_LAUNCH_CHECK();
  }
}

// Sparsify: entries of row r of the batch buffer T [k][m] with T >= thr.
// One workgroup (256 threads) per row.
__global__ __launch_bounds__(256) void k_row_count(const float* __restrict__ T, int64_t m, float thr,
                                                   int64_t* __restrict__ counts) {
  __shared__ int64_t sc[4];
  const int64_t r = blockIdx.x;
  const float* row = T + r * m;
  int64_t c = 0;
  for (int64_t j = threadIdx.x; j < m; j += 256) c += row[j] >= thr ? 1 : 0;
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if ((threadIdx.x & 63) == 0) sc[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) counts[r] = sc[0] + sc[1] + sc[2] + sc[3];
}

// Writes the surviving entries of row r in increasing column order at
// ptr[r]: column index and value. Wave ballots give each entry its rank
// within a 256-column step; LDS carries the wave totals.
__global__ __launch_bounds__(256) void k_row_fill(const float* __restrict__ T, int64_t m, float thr,
                                                  const int64_t* __restrict__ ptr,
                                                  int32_t* __restrict__ col,
                                                  float* __restrict__ val) {
  __shared__ int32_t sw[4];
  const int64_t r = blockIdx.x;
  const float* row = T + r * m;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int64_t out = ptr[r];
  for (int64_t j0 = 0; j0 < m; j0 += 256) {
    const int64_t j = j0 + threadIdx.x;
    const float v = j < m ? row[j] : 0.0f;
    const bool keep = j < m && v >= thr;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
    if (lane == 0) sw[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int64_t base = out;
    for (int w = 0; w < wave; ++w) base += sw[w];
    if (keep) {
      const int64_t o = base + __builtin_popcountll(bal & below);
      col[o] = (int32_t)j;
      val[o] = v;
    }
    out += sw[0] + sw[1] + sw[2] + sw[3];
    __syncthreads();  // sw reuse
  }
}

__global__ void k_set_i64(int64_t* p, int64_t v) {
  if (threadIdx.x == 0) *p = v;
}

void materialize_checks(sinkhorn_problem* p, double eps, const float* f, const float* g,
                        const int64_t* rows, int64_t k, const float* T) {
  if (!p || !f || !g || !rows || !T) fail(SINKHORN_ERR_INVALID_ARG, "null pointer");
  if (!(std::isfinite(eps) && eps > 0.0)) fail(SINKHORN_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (k < 0) fail(SINKHORN_ERR_INVALID_ARG, "k must be >= 0");
}

// Rows rows[0..k) of the plan into T [k][m] (and their maxima into row_max
// when non-null), with the per-call buffers P [k] and keys [k + 1] (device)
// and, for d <= 8, Hd [m]; every value they hold is written here before it is
// read. Checks the row indices first (one synchronization) and synchronizes
// at the end.
void materialize_into(sinkhorn_problem* p, double eps, const float* f, const float* g,
                      const int64_t* rows, int64_t k, float* T, float* row_max, double* P,
                      uint32_t* keys, double* Hd) {
  hipLaunchKernelGGL(k_set_u32, dim3(1), dim3(64), 0, p->stream, keys + k, 0u);
  SK_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_check_rows, grid1(((k + 255) / 256), 256), dim3(256), 0, p->stream, rows, k,
                     p->n, keys + k);
  SK_LAUNCH_CHECK();
  SK_HIP(hipMemcpyAsync(p->host_tmp, keys + k, sizeof(uint32_t), hipMemcpyDeviceToHost, p->stream));
  SK_HIP(hipStreamSynchronize(p->stream));
  uint32_t nbad;
  memcpy(&nbad, p->host_tmp, sizeof(uint32_t));
  if (nbad) fail(SINKHORN_ERR_INVALID_ARG, "row index outside [0, n)");
  column_terms(p, eps, g, Hd);
  rows_pass(p, eps, f, rows, 0, k, P, nullptr, keys, Hd, T);
  if (row_max) {
    hipLaunchKernelGGL(k_keys_to_max, grid1(((k + 255) / 256), 256), dim3(256), 0, p->stream, keys,
                       k, row_max);
    SK_LAUNCH_CHECK();
  }
  SK_HIP(hipStreamSynchronize(p->stream));
}

// ---- the allocation-free variant's device memory
//
// One array per GPU, in the code object's data, held until the process ends:
// the row terms P, the fp64 column terms Hd and the row-maximum keys of one
// call of sinkhorn_materialize_rows_noalloc. Host code never uses the
// array's name as an address (on the host it only names the symbol): every
// use goes through the device address hipGetSymbolAddress returned for the
// GPU, recorded once per device.
constexpr int64_t kStaticRows = 4096;              // rows per call, at most
constexpr int64_t kStaticCols = int64_t(1) << 21;  // columns per call when d <= 8, at most
constexpr int64_t kStaticOffP = 0;
constexpr int64_t kStaticOffHd = kStaticOffP + kStaticRows * 8;
constexpr int64_t kStaticOffKeys = kStaticOffHd + kStaticCols * 8;
constexpr int64_t kStaticBytes = kStaticOffKeys + (kStaticRows + 64) * 4;

__device__ __align__(256) unsigned char scratch[kStaticBytes];

std::mutex g_scratch_mu;
std::unordered_map<int, unsigned char*> g_scratch;  // device -> address of its copy of scratch

unsigned char* static_scratch(int device) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch.find(device);
  if (it == g_scratch.end())
    fail(SINKHORN_ERR_HIP, "static scratch of device " + std::to_string(device) + " not set up");
  return it->second;
}

struct Scratch {
  double* P = nullptr;
  double* Hd = nullptr;
  int32_t* live = nullptr;
  uint32_t* keys = nullptr;
  ~Scratch() {
    dev_free(P);
    dev_free(Hd);
    dev_free(live);
    dev_free(keys);
  }
};

}  // namespace

// The device address of the current device's copy of the static scratch,
// looked up once per device; called by sinkhorn_init with the handle's device
// current.
void static_scratch_setup(int device) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch.count(device)) return;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  check_hip(e, "hipGetSymbolAddress(scratch)");
  if (!ptr) fail(SINKHORN_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
  g_scratch[device] = static_cast<unsigned char*>(ptr);
}

}  // namespace sk

using namespace sk;

extern "C" {

int sinkhorn_materialize_rows(sinkhorn_problem* p, double eps, const float* f, const float* g,
                              const int64_t* rows, int64_t k, float* T, float* row_max) {
  try {
    materialize_checks(p, eps, f, g, rows, k, T);
    if (k == 0) return SINKHORN_OK;
    Scratch s;
    s.P = (double*)dev_alloc(sizeof(double) * k);
    s.keys = (uint32_t*)dev_alloc(sizeof(uint32_t) * (k + 1));
    if (p->d <= kMaxValuD) s.Hd = (double*)dev_alloc(sizeof(double) * p->m);
    materialize_into(p, eps, f, g, rows, k, T, row_max, s.P, s.keys, s.Hd);
    return SINKHORN_OK;
  } catch (const Failure& e) {
    set_last_error(e.msg);
    return e.code;
  } catch (...) {
    set_last_error("unexpected exception");
    return SINKHORN_ERR_HIP;
  }
}

int sinkhorn_materialize_rows_noalloc(sinkhorn_problem* p, double eps, const float* f,
                                      const float* g, const int64_t* rows, int64_t k, float* T,
                                      float* row_max) {
  try {
    materialize_checks(p, eps, f, g, rows, k, T);
    if (k > kStaticRows)
      fail(SINKHORN_ERR_INVALID_ARG, "materialize_rows_noalloc: k = " + std::to_string(k) +
                                         " rows exceed its limit of " + std::to_string(kStaticRows));
    if (p->d <= kMaxValuD && p->m > kStaticCols)
      fail(SINKHORN_ERR_INVALID_ARG, "materialize_rows_noalloc: m = " + std::to_string(p->m) +
                                         " columns exceed its limit of " +
                                         std::to_string(kStaticCols) + " for d <= 8");
    if (k == 0) return SINKHORN_OK;
    unsigned char* base = static_scratch(p->device);
    double* P = reinterpret_cast<double*>(base + kStaticOffP);
    double* Hd = reinterpret_cast<double*>(base + kStaticOffHd);
    uint32_t* keys = reinterpret_cast<uint32_t*>(base + kStaticOffKeys);
    materialize_into(p, eps, f, g, rows, k, T, row_max, P, keys, p->d <= kMaxValuD ? Hd : nullptr);
    return SINKHORN_OK;
  } catch (const Failure& e) {
    set_last_error(e.msg);
    return e.code;
  } catch (...) {
    set_last_error("unexpected exception");
    return SINKHORN_ERR_HIP;
  }
}

int sinkhorn_min_row(sinkhorn_problem* p, double eps, const float* f, const float* g, float* out) {
  try {
    if (!p || !f || !g || !out) fail(SINKHORN_ERR_INVALID_ARG, "null pointer");
    if (!(std::isfinite(eps) && eps > 0.0)) fail(SINKHORN_ERR_INVALID_ARG, "eps must be finite and > 0");
    const int64_t batch = 16384;
    const int64_t kb = p->n < batch ? p->n : batch;
    Scratch s;
    s.P = (double*)dev_alloc(sizeof(double) * kb);
    s.keys = (uint32_t*)dev_alloc(sizeof(uint32_t) * (kb + 1));
    s.live = (int32_t*)dev_alloc(sizeof(int32_t) * kb);
    if (p->d <= kMaxValuD) s.Hd = (double*)dev_alloc(sizeof(double) * p->m);
    column_terms(p, eps, g, s.Hd);
    uint32_t* best = s.keys + kb;
    hipLaunchKernelGGL(k_set_u32, dim3(1), dim3(64), 0, p->stream, best, 0xffffffffu);
    SK_LAUNCH_CHECK();
    for (int64_t r0 = 0; r0 < p->n; r0 += kb) {
      const int64_t k = p->n - r0 < kb ? p->n - r0 : kb;
      rows_pass(p, eps, f, nullptr, r0, k, s.P, s.live, s.keys, s.Hd, nullptr);
      hipLaunchKernelGGL(k_min_live, grid1(((k + 255) / 256), 256), dim3(256), 0, p->stream,
                         s.keys, s.live, k, best);
      SK_LAUNCH_CHECK();
    }
    // the value through the device exp2 the plan entries use, so that
    // "T_ij >= min_row" keeps the largest entry of every row with mass
    float* v = reinterpret_cast<float*>(s.live);
    hipLaunchKernelGGL(k_keys_to_max, dim3(1), dim3(256), 0, p->stream, best, (int64_t)1, v);
    SK_LAUNCH_CHECK();
    uint32_t key = 0;
    float val = 0.0f;
    SK_HIP(hipMemcpyAsync(&p->host_tmp[0], best, sizeof(uint32_t), hipMemcpyDeviceToHost, p->stream));
    SK_HIP(hipMemcpyAsync(&p->host_tmp[1], v, sizeof(float), hipMemcpyDeviceToHost, p->stream));
    SK_HIP(hipStreamSynchronize(p->stream));
    memcpy(&key, &p->host_tmp[0], sizeof(uint32_t));
    memcpy(&val, &p->host_tmp[1], sizeof(float));
    *out = key == 0xffffffffu ? NAN : val;  // NaN: no row carries mass
    return SINKHORN_OK;
  } catch (const Failure& e) {
    set_last_error(e.msg);
    return e.code;
  } catch (...) {
    set_last_error("unexpected exception");
    return SINKHORN_ERR_HIP;
  }
}

int sinkhorn_sparsify(sinkhorn_problem* p, double eps, const float* f, const float* g,
                      float threshold, int64_t batch, int64_t* row_ptr, int32_t* col, float* val,
                      int64_t cap, int64_t* nnz_out) {
  try {
    if (!p || !f || !g || !row_ptr || !nnz_out) fail(SINKHORN_ERR_INVALID_ARG, "null pointer");
    if (!(std::isfinite(eps) && eps > 0.0)) fail(SINKHORN_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (!(std::isfinite(threshold) && threshold > 0.0f))
      fail(SINKHORN_ERR_INVALID_ARG, "threshold must be finite and > 0");
    if ((col == nullptr) != (val == nullptr)) fail(SINKHORN_ERR_INVALID_ARG, "col and val go together");
    if (p->m >= ((int64_t)1 << 31)) fail(SINKHORN_ERR_UNSUPPORTED, "column index needs m < 2^31");
    const int64_t n = p->n, m = p->m;
    if (batch <= 0) batch = 1024;
    const int64_t maxb = ((int64_t)1 << 28) / m > 1 ? ((int64_t)1 << 28) / m : 1;  // <= 1 GiB buffer
    if (batch > maxb) batch = maxb;
    if (batch > n) batch = n;
    Scratch s;
    s.P = (double*)dev_alloc(sizeof(double) * batch);
    s.keys = (uint32_t*)dev_alloc(sizeof(uint32_t) * batch);
    if (p->d <= kMaxValuD) s.Hd = (double*)dev_alloc(sizeof(double) * m);
    float* T = (float*)dev_alloc(sizeof(float) * batch * m);
    int64_t* counts = nullptr;
    void* temp = nullptr;
    auto cleanup = [&] {
      dev_free(T);
      dev_free(counts);
      dev_free(temp);
    };
    try {
      counts = (int64_t*)dev_alloc(sizeof(int64_t) * batch);
      size_t tb = 0;
      SK_HIP(rocprim::exclusive_scan(nullptr, tb, counts, row_ptr, (int64_t)0, (size_t)batch,
                                     rocprim::plus<int64_t>(), p->stream));
      temp = dev_alloc(tb > 0 ? tb : 1);
      column_terms(p, eps, g, s.Hd);
      const bool fill = col != nullptr;
      int64_t total = 0;
      for (int64_t r0 = 0; r0 < n; r0 += batch) {
        const int64_t k = n - r0 < batch ? n - r0 : batch;
        rows_pass(p, eps, f, nullptr, r0, k, s.P, nullptr, s.keys, s.Hd, T);
        hipLaunchKernelGGL(k_row_count, grid1(k, 256), dim3(256), 0, p->stream, T, m, threshold,
                           counts);
        SK_LAUNCH_CHECK();
        // row_ptr[r0 .. r0 + k) = total + exclusive prefix of the batch counts
        SK_HIP(rocprim::exclusive_scan(temp, tb, counts, row_ptr + r0, total, (size_t)k,
                                       rocprim::plus<int64_t>(), p->stream));
        int64_t last = 0, cnt = 0;
        SK_HIP(hipMemcpyAsync(&p->host_tmp[0], row_ptr + r0 + k - 1, sizeof(int64_t),
                              hipMemcpyDeviceToHost, p->stream));
        SK_HIP(hipMemcpyAsync(&p->host_tmp[1], counts + k - 1, sizeof(int64_t), hipMemcpyDeviceToHost,
                              p->stream));
        SK_HIP(hipStreamSynchronize(p->stream));
        memcpy(&last, &p->host_tmp[0], sizeof(int64_t));
        memcpy(&cnt, &p->host_tmp[1], sizeof(int64_t));
        const int64_t after = last + cnt;
        if (fill && after <= cap) {
          hipLaunchKernelGGL(k_row_fill, grid1(k, 256), dim3(256), 0, p->stream, T, m, threshold,
                             row_ptr + r0, col, val);
          SK_LAUNCH_CHECK();
        }
        total = after;
      }
      hipLaunchKernelGGL(k_set_i64, dim3(1), dim3(64), 0, p->stream, row_ptr + n, total);
      SK_LAUNCH_CHECK();
      SK_HIP(hipStreamSynchronize(p->stream));
      *nnz_out = total;
      cleanup();
      if (!fill) return SINKHORN_OK;
      return total <= cap ? SINKHORN_OK : SINKHORN_ERR_CAPACITY;
    } catch (...) {
      (void)hipStreamSynchronize(p->stream);
      cleanup();
      throw;
    }
  } catch (const Failure& e) {
    set_last_error(e.msg);
    return e.code;
  } catch (...) {
    set_last_error("unexpected exception");
    return SINKHORN_ERR_HIP;
  }
}

}  // extern "C"
