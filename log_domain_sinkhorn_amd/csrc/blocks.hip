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
  RowFinal F;
};

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
                                                        const float* __restrict__ H) {
  __shared__ TileLds L;
  const int64_t tile = A.order ? (int64_t)A.order[blockIdx.x] : (int64_t)blockIdx.x;
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
// Sort key of each row tile: the bit length of its row block's list of
// admitted column blocks (lists within a factor of two share a key; an
// empty list means a pass over all columns: the largest key, 63).
constexpr int kKeyBits = 6;
__global__ __launch_bounds__(256) void k_tile_keys(const int64_t* __restrict__ ptr, int64_t tiles,
                                                   int32_t B, uint32_t* __restrict__ key,
                                                   int32_t* __restrict__ val) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= tiles) return;
  const int64_t I = t * kRowsPerTile / B;
  const int64_t c = ptr[I + 1] - ptr[I];
  key[t] = c > 0 ? 64u - (uint32_t)__clzll((unsigned long long)c) : (1u << kKeyBits) - 1;
  val[t] = (int32_t)t;
}

// The row tiles of a sparse half-step, longest lists first by powers of two
// and in tile order within a power (a stable radix sort of the bit lengths):
// the rare lists tens of times the average no longer start late and run
// alone at the end, while the workgroups running together still take
// neighbouring row blocks, whose column blocks overlap in L2. Measured at
// 2^24: 798 ms per launch in tile order, 778 ms with the exact lengths
// sorted, 765 ms so; on verified lists 446, 460 and 446 ms.
const int32_t* heavy_first(sinkhorn_problem* p, const int64_t* ptr, int64_t tiles, int32_t B) {
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
  hipLaunchKernelGGL(k_tile_keys, grid1(((tiles + 255) / 256), 256), dim3(256), 0, st, ptr, tiles,
                     B, kin, vin);
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
  return vout;
}

template <int D>
void launch_sparse(sinkhorn_problem* p, const SparseArgs& A, int64_t tiles, bool shifted,
                   const ProfEv& pe) {
  if (shifted)
    hipExtLaunchKernelGGL((k_lse_sparse<D, true>), grid1(tiles, kThreads), dim3(kThreads), 0, p->stream,
                          pe.start, pe.stop, 0, A, A.Q, A.H);
  else
    hipExtLaunchKernelGGL((k_lse_sparse<D, false>), grid1(tiles, kThreads), dim3(kThreads), 0,
                          p->stream, pe.start, pe.stop, 0, A, A.Q, A.H);
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
  A.order = heavy_first(p, ptr, tiles, B);
  A.F = make_rowfinal(p, hs);
  auto launch = [&](const SparseArgs& a, bool sh, const ProfEv& pe) {
    switch (p->d) {
      case 1: launch_sparse<1>(p, a, tiles, sh, pe); break;
      case 2: launch_sparse<2>(p, a, tiles, sh, pe); break;
      case 3: launch_sparse<3>(p, a, tiles, sh, pe); break;
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
