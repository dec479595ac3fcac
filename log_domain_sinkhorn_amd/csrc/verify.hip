// Tile verification.
//
// FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport, §3.2: the tiles
// that pass the block-pair screen are checked with their exact mass over the
// B^2 point pairs before they are admitted (§C.5 measures the trade-off).
// Read here as the exact form of the screen's own per-tile guarantee: with
//   s_i = sum_{j in J} b_j exp((f_i + g_j - C_ij)/eps)   (row share / a_i)
//   t_j = sum_{i in I} a_i exp((f_i + g_j - C_ij)/eps)   (column share / b_j)
// a candidate (I, J) is dropped iff every s_i <= delta_rel and every
// t_j <= delta_rel, so an omitted tile still takes at most delta_rel a_i from
// row i and delta_rel b_j from column j and the a-priori bound on the omitted
// mass is unchanged. A row block that would lose every candidate keeps them
// all, then likewise a column block (keeping tiles never weakens the bound,
// and a block without tiles would fall back to a dense update).
//
// Kernel: one wave per candidate tile of 128 x 128 points, lanes as an 8 x 8
// grid: lane (r, c) holds rows r, r + 8, ... (16) and walks columns c, c + 8,
// ... (16), so every row sum and column sum is lane-local until a 3-step
// shuffle reduction over the 8 lanes that share it. Per pair: the shifted
// squared distance (d subs, d fmas), one fma for the exponent, one exp2 and
// two fmas into the row and column sums. A NaN share keeps the tile.
//
// Compaction: the kept flags are counted and written per row block in order
// (one wave per row block, ballot prefix), and the column-major list is a
// stable radix sort of (column block, row block) pairs, so both lists are
// deterministic.
#include <cmath>

#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/device/device_scan.hpp>

#include "verify.h"

namespace sk {
namespace {

__device__ __forceinline__ float vex2(float v) { return __builtin_amdgcn_exp2f(v); }

struct VerifyArgs {
  const float* xs;  // row side SoA [D][xstride]
  int64_t xstride;
  const float* f;   // [n]
  const float* a;   // [n]
  int64_t n;
  const float* ys;  // column side SoA [D][ystride]
  int64_t ystride;
  const float* g;   // [m]
  const float* b;   // [m]
  int64_t m;
  const int64_t* ptr;  // [nb + 1]
  const int32_t* idx;  // [nnz]
  int64_t nnz;
  int64_t nb;
  float inv_s;   // 1 / s
  float lam;     // log2(e) / eps
  float nkappa;  // -s log2(e) / eps
  float delta;
  uint8_t* keep;
};

template <int D>
__device__ __forceinline__ void verify_tile(const VerifyArgs& A, int64_t e) {
  // row block of candidate e: the last I with ptr[I] <= e
  int64_t lo = 0, hi = A.nb;
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) >> 1;
    if (A.ptr[mid] <= e) lo = mid;
    else hi = mid;
  }
  const int64_t I = lo;
  const int64_t J = A.idx[e];
  const int lane = threadIdx.x & 63;
  const int r8 = lane & 7;
  const int c8 = lane >> 3;

  // rows: u = -f / s folds the row potential into the first squared term
  float x[16][D], u[16], aw[16], R[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int64_t i = I * kVerifyB + r8 + 8 * q;
    const bool ok = i < A.n;
    const int64_t ic = ok ? i : A.n - 1;  // clamped: the loads need no branch
#pragma unroll
    for (int k = 0; k < D; ++k) x[q][k] = A.xs[k * A.xstride + ic];
    const float fv = A.f[ic], av = A.a[ic];
    u[q] = ok ? -fv * A.inv_s : INFINITY;
    aw[q] = ok ? av : 0.0f;
    R[q] = 0.0f;
  }
  bool big = false;
  // column data of step bb + 1 is loaded while step bb computes
  float yn[D], gn, bn;
  auto load_col = [&](int bb) {
    const int64_t j = J * kVerifyB + c8 + 8 * bb;
    const bool ok = j < A.m;
    const int64_t jc = ok ? j : A.m - 1;
#pragma unroll
    for (int k = 0; k < D; ++k) yn[k] = A.ys[k * A.ystride + jc];
    const float gv = A.g[jc], bv = A.b[jc];
    gn = ok ? gv : -INFINITY;
    bn = ok ? bv : 0.0f;
  };
  load_col(0);
#pragma unroll 1
  for (int bb = 0; bb < 16; ++bb) {
    float y[D];
#pragma unroll
    for (int k = 0; k < D; ++k) y[k] = yn[k];
    const float lg = A.lam * gn;
    const float bj = bn;
    if (bb + 1 < 16) load_col(bb + 1);
    float c = 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float dd = x[q][0] - y[0];
      float s = __builtin_fmaf(dd, dd, u[q]);
#pragma unroll
      for (int k = 1; k < D; ++k) {
        dd = x[q][k] - y[k];
        s = __builtin_fmaf(dd, dd, s);
      }
      const float w = vex2(__builtin_fmaf(s, A.nkappa, lg));
      R[q] = __builtin_fmaf(bj, w, R[q]);
      c = __builtin_fmaf(aw[q], w, c);
    }
    // column share: the 8 lanes of this column (lanes 8 c8 + 0..7)
    c += __shfl_xor(c, 1, 64);
    c += __shfl_xor(c, 2, 64);
    c += __shfl_xor(c, 4, 64);
    big = big || !(c <= A.delta);
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    // row share: the 8 lanes of this row (lanes r8 + 8 * 0..7)
    float r = R[q];
    r += __shfl_xor(r, 8, 64);
    r += __shfl_xor(r, 16, 64);
    r += __shfl_xor(r, 32, 64);
    big = big || !(r <= A.delta);
  }
  const uint64_t any = __ballot(big);
  if (lane == 0) A.keep[e] = any != 0 ? 1 : 0;
}

// Tiles are taken in a wave-stride loop: a grid of one wave per tile would
// exceed the 2^32 work-items of one dispatch at 2^24 points.
template <int D>
__global__ __launch_bounds__(256) void k_verify(VerifyArgs A) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t step = (int64_t)gridDim.x * 4;
  for (int64_t e = (int64_t)blockIdx.x * 4 + wave; e < A.nnz; e += step)
    verify_tile<D>(A, e);
}
// One wave per row block: a block whose candidates all failed keeps them all.
__global__ __launch_bounds__(64) void k_row_fallback(const int64_t* __restrict__ ptr, int64_t nb,
                                                     uint8_t* __restrict__ keep) {
  const int64_t I = blockIdx.x;
  if (I >= nb) return;
  const int64_t s = ptr[I], e = ptr[I + 1];
  bool any = false;
  for (int64_t k = s + threadIdx.x; k < e; k += 64) any = any || keep[k] != 0;
  if (__ballot(any) != 0 || s == e) return;
  for (int64_t k = s + threadIdx.x; k < e; k += 64) keep[k] = 1;
}

__global__ __launch_bounds__(256) void k_zero_i32v(int32_t* __restrict__ v, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) v[i] = 0;
}

__global__ __launch_bounds__(256) void k_col_mark(const int32_t* __restrict__ idx, int64_t nnz,
                                                  const uint8_t* __restrict__ keep,
                                                  int32_t* __restrict__ colany) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < nnz && keep[e]) __hip_atomic_store(&colany[idx[e]], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void k_col_fallback(const int32_t* __restrict__ idx, int64_t nnz,
                                                      const int32_t* __restrict__ colany,
                                                      uint8_t* __restrict__ keep) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < nnz && !keep[e] && colany[idx[e]] == 0) keep[e] = 1;
}

// One wave per row block: kept count (cnt[nb] = 0 closes the scan).
__global__ __launch_bounds__(64) void k_keep_count(const int64_t* __restrict__ ptr, int64_t nb,
                                                   const uint8_t* __restrict__ keep,
                                                   int64_t* __restrict__ cnt) {
  const int64_t I = blockIdx.x;
  if (I > nb) return;
  if (I == nb) {
    if (threadIdx.x == 0) cnt[nb] = 0;
    return;
  }
  int64_t c = 0;
  for (int64_t k = ptr[I] + threadIdx.x; k < ptr[I + 1]; k += 64) c += keep[k] ? 1 : 0;
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if (threadIdx.x == 0) cnt[I] = c;
}

// One wave per row block: kept tiles in candidate order.
__global__ __launch_bounds__(64) void k_keep_fill(const int64_t* __restrict__ ptr, int64_t nb,
                                                  const int32_t* __restrict__ idx,
                                                  const uint8_t* __restrict__ keep,
                                                  const int64_t* __restrict__ vptr,
                                                  int32_t* __restrict__ vidx,
                                                  int32_t* __restrict__ vrow) {
  const int64_t I = blockIdx.x;
  if (I >= nb) return;
  const int lane = threadIdx.x;
  int64_t out = vptr[I];
  for (int64_t base = ptr[I]; base < ptr[I + 1]; base += 64) {
    const int64_t k = base + lane;
    const bool on = k < ptr[I + 1] && keep[k];
    const uint64_t bal = __ballot(on);
    if (on) {
      const int64_t pos = out + __popcll(bal & ((1ull << lane) - 1ull));
      vidx[pos] = idx[k];
      vrow[pos] = (int32_t)I;
    }
    out += __popcll(bal);
  }
}

// tptr[J] = first position of column block J in the sorted keys, J in [0, mb].
__global__ __launch_bounds__(256) void k_col_bounds(const int32_t* __restrict__ skey, int64_t kept,
                                                    int64_t mb, int64_t* __restrict__ tptr) {
  const int64_t J = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (J > mb) return;
  int64_t lo = 0, hi = kept;  // first k with skey[k] >= J
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (skey[mid] < J) lo = mid + 1;
    else hi = mid;
  }
  tptr[J] = lo;
}

template <int D>
void launch_verify(hipStream_t st, const VerifyArgs& A) {
  constexpr int64_t kMaxGroups = 1 << 20;  // 2^28 work-items
  const int64_t want = (A.nnz + 3) / 4;
  hipLaunchKernelGGL((k_verify<D>), grid1((want < kMaxGroups ? want : kMaxGroups), 256), dim3(256),
                     0, st, A);
  SK_LAUNCH_CHECK();
}

int end_bit_for(int64_t mb) {
  int b = 1;
  while (b < 31 && (int64_t(1) << b) <= mb) ++b;
  return b;
}

}  // namespace

VerifyScratch::~VerifyScratch() {
  dev_free(keep);
  dev_free(colany);
  dev_free(cnt);
  dev_free(vrow);
  dev_free(skey);
  dev_free(temp);
}

void VerifyScratch::reserve(int64_t nnz, int64_t nb, int64_t mb) {
  if (nnz > nnz_cap) {
    dev_free(keep);
    dev_free(vrow);
    dev_free(skey);
    keep = nullptr;
    vrow = skey = nullptr;
    nnz_cap = 0;
    const int64_t want = nnz + nnz / 4 + 1024;
    keep = (uint8_t*)dev_alloc((size_t)want);
    vrow = (int32_t*)dev_alloc(sizeof(int32_t) * want);
    skey = (int32_t*)dev_alloc(sizeof(int32_t) * want);
    nnz_cap = want;
  }
  if (nb + 1 > nb_cap) {
    dev_free(cnt);
    cnt = nullptr;
    cnt = (int64_t*)dev_alloc(sizeof(int64_t) * (nb + 1));
    nb_cap = nb + 1;
  }
  if (mb > mb_cap) {
    dev_free(colany);
    colany = nullptr;
    colany = (int32_t*)dev_alloc(sizeof(int32_t) * (mb > 0 ? mb : 1));
    mb_cap = mb;
  }
}

int64_t verify_tiles(sinkhorn_problem* p, const Side& rows, const Side& cols, const float* f,
                     const float* g, double eps, double delta_rel, const int64_t* ptr,
                     const int32_t* idx, int64_t nnz, int64_t nb, int64_t mb, int64_t* vptr,
                     int32_t* vidx, int64_t* tptr, int32_t* tidx, VerifyScratch& s) {
  hipStream_t st = p->stream;
  s.reserve(nnz, nb, mb);
  const double lam = kLog2e / eps;
  VerifyArgs A;
  A.xs = rows.soa;
  A.xstride = rows.padded;
  A.f = f;
  A.a = rows.w;
  A.n = rows.count;
  A.ys = cols.soa;
  A.ystride = cols.padded;
  A.g = g;
  A.b = cols.w;
  A.m = cols.count;
  A.ptr = ptr;
  A.idx = idx;
  A.nnz = nnz;
  A.nb = nb;
  A.inv_s = (float)(1.0 / p->scale);
  A.lam = (float)lam;
  A.nkappa = (float)(-p->scale * lam);
  A.delta = (float)delta_rel;
  A.keep = s.keep;
  if (nnz > 0) {
    switch (p->d) {
      case 1: launch_verify<1>(st, A); break;
      case 2: launch_verify<2>(st, A); break;
      case 3: launch_verify<3>(st, A); break;
      default: fail(SINKHORN_ERR_UNSUPPORTED, "tile verification needs d <= 3");
    }
    hipLaunchKernelGGL(k_row_fallback, grid1(nb, 64), dim3(64), 0, st, ptr, nb, s.keep);
    SK_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_zero_i32v, grid1(((mb + 255) / 256), 256), dim3(256), 0, st, s.colany, mb);
    SK_LAUNCH_CHECK();
    const uint32_t eb = (uint32_t)((nnz + 255) / 256);
    hipLaunchKernelGGL(k_col_mark, dim3(eb), dim3(256), 0, st, idx, nnz, s.keep, s.colany);
    SK_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_col_fallback, dim3(eb), dim3(256), 0, st, idx, nnz, s.colany, s.keep);
    SK_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(k_keep_count, grid1((nb + 1), 64), dim3(64), 0, st, ptr, nb, s.keep, s.cnt);
  SK_LAUNCH_CHECK();
  size_t tb = 0;
  SK_HIP(rocprim::exclusive_scan(nullptr, tb, s.cnt, vptr, (int64_t)0, (size_t)(nb + 1),
                                 rocprim::plus<int64_t>(), st));
  size_t sb = 0;
  const int ebits = end_bit_for(mb);
  SK_HIP(rocprim::radix_sort_pairs(nullptr, sb, vidx, s.skey, s.vrow, tidx, (size_t)nnz, 0, ebits, st));
  const size_t need = tb > sb ? tb : sb;
  if (need > s.temp_bytes) {
    SK_HIP(hipStreamSynchronize(st));
    dev_free(s.temp);
    s.temp = nullptr;
    s.temp_bytes = 0;
    s.temp = dev_alloc(need);
    s.temp_bytes = need;
  }
  SK_HIP(rocprim::exclusive_scan(s.temp, tb, s.cnt, vptr, (int64_t)0, (size_t)(nb + 1),
                                 rocprim::plus<int64_t>(), st));
  int64_t kept = 0;
  SK_HIP(hipMemcpyAsync(&kept, vptr + nb, sizeof(int64_t), hipMemcpyDeviceToHost, st));
  SK_HIP(hipStreamSynchronize(st));
  if (kept < 0 || kept > nnz) fail(SINKHORN_ERR_HIP, "tile verification: bad kept count");
  if (nb > 0) {
    hipLaunchKernelGGL(k_keep_fill, grid1(nb, 64), dim3(64), 0, st, ptr, nb, idx, s.keep, vptr,
                       vidx, s.vrow);
    SK_LAUNCH_CHECK();
  }
  if (kept > 0) {
    size_t sb2 = s.temp_bytes;
    SK_HIP(rocprim::radix_sort_pairs(s.temp, sb2, vidx, s.skey, s.vrow, tidx, (size_t)kept, 0,
                                     ebits, st));
  }
  hipLaunchKernelGGL(k_col_bounds, grid1(((mb + 1 + 255) / 256), 256), dim3(256), 0, st, s.skey,
                     kept, mb, tptr);
  SK_LAUNCH_CHECK();
  return kept;
}

}  // namespace sk

using namespace sk;

namespace {

template <class F>
int vguarded(F&& body) {
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

}  // namespace

extern "C" int sinkhorn_verify_tiles(sinkhorn_problem* p, double eps, const float* f, const float* g,
                                     int32_t B, double delta_rel, const int64_t* ptr,
                                     const int32_t* idx, int64_t* vptr, int32_t* vidx,
                                     int64_t* tptr, int32_t* tidx, int64_t* kept_out) {
  return vguarded([&] {
    if (!p || !f || !g || !ptr || !vptr || !tptr || !kept_out)
      fail(SINKHORN_ERR_INVALID_ARG, "null pointer");
    if (!(std::isfinite(eps) && eps > 0.0)) fail(SINKHORN_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (!(std::isfinite(delta_rel) && delta_rel > 0.0))
      fail(SINKHORN_ERR_INVALID_ARG, "delta_rel must be finite and > 0");
    if (B != kVerifyB) fail(SINKHORN_ERR_UNSUPPORTED, "tile verification needs B = 128");
    if (p->d > 3) fail(SINKHORN_ERR_UNSUPPORTED, "tile verification needs d <= 3");
    const int64_t nb = (p->n + B - 1) / B, mb = (p->m + B - 1) / B;
    int64_t ends[2] = {0, 0};
    SK_HIP(hipMemcpyAsync(&ends[0], ptr, sizeof(int64_t), hipMemcpyDeviceToHost, p->stream));
    SK_HIP(hipMemcpyAsync(&ends[1], ptr + nb, sizeof(int64_t), hipMemcpyDeviceToHost, p->stream));
    SK_HIP(hipStreamSynchronize(p->stream));
    if (ends[0] != 0 || ends[1] < 0) fail(SINKHORN_ERR_INVALID_ARG, "tile list must start at 0");
    const int64_t nnz = ends[1];
    if (nnz > 0 && (!idx || !vidx || !tidx)) fail(SINKHORN_ERR_INVALID_ARG, "null pointer");
    check_csr(p, ptr, nb, idx, mb);
    VerifyScratch s;
    *kept_out = verify_tiles(p, p->X, p->Y, f, g, eps, delta_rel, ptr, idx, nnz, nb, mb, vptr, vidx,
                             tptr, tidx, s);
    SK_HIP(hipStreamSynchronize(p->stream));
    return SINKHORN_OK;
  });
}
