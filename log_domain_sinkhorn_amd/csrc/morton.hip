// Morton (Z-order) codes and a stable Morton order of two clouds.
//
// FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport, §3: Morton sorting
// makes spatially compact cells and blocks of consecutive points contiguous.
// Layout of the code (the pages fix none): one bounding box over both clouds,
// 21 bits per axis,
//   q_k = min(2^21 - 1, floor((p_k - lo_k) * (2^21 / (hi_k - lo_k))))  in fp64
// (q_k = 0 on a flat axis), bit b of axis k at position d*b + k. The factor
// 2^21/(hi_k - lo_k) is divided once on the host; the device does one fp64
// subtraction and one multiplication per axis (no contraction), so the codes
// are bit-exact against any IEEE fp64 evaluation of the same formula. The
// order is a stable LSD radix sort of (code, original index) pairs, so equal
// codes keep their input order.
#include <cfloat>
#include <cmath>
#include <vector>

#include <rocprim/device/device_radix_sort.hpp>

#include "internal.h"

namespace sk {
namespace {

constexpr int kBits = 21;
constexpr int kBoxBlock = 256;
constexpr int kBoxPer = 16;  // points per thread in the bounding-box pass

// Per-block min and max of each axis: part[block][2*d] (min then max).
__global__ __launch_bounds__(kBoxBlock) void k_bbox(const float* __restrict__ pts, int64_t ps,
                                                    int64_t as, int64_t count, int32_t d,
                                                    float* __restrict__ part) {
  __shared__ float smin[3][kBoxBlock];
  __shared__ float smax[3][kBoxBlock];
  float lo[3] = {FLT_MAX, FLT_MAX, FLT_MAX};
  float hi[3] = {-FLT_MAX, -FLT_MAX, -FLT_MAX};
  const int64_t base = (int64_t)blockIdx.x * kBoxBlock * kBoxPer;
  for (int q = 0; q < kBoxPer; ++q) {
    const int64_t i = base + q * kBoxBlock + threadIdx.x;
    if (i < count)
      for (int k = 0; k < d; ++k) {
        const float v = pts[i * ps + k * as];
        lo[k] = fminf(lo[k], v);
        hi[k] = fmaxf(hi[k], v);
      }
  }
  for (int k = 0; k < d; ++k) {
    smin[k][threadIdx.x] = lo[k];
    smax[k][threadIdx.x] = hi[k];
  }
  __syncthreads();
  for (int w = kBoxBlock / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w)
      for (int k = 0; k < d; ++k) {
        smin[k][threadIdx.x] = fminf(smin[k][threadIdx.x], smin[k][threadIdx.x + w]);
        smax[k][threadIdx.x] = fmaxf(smax[k][threadIdx.x], smax[k][threadIdx.x + w]);
      }
    __syncthreads();
  }
  if (threadIdx.x == 0)
    for (int k = 0; k < d; ++k) {
      part[blockIdx.x * 2 * d + k] = smin[k][0];
      part[blockIdx.x * 2 * d + d + k] = smax[k][0];
    }
}

struct Box {
  double lo[3];
  double factor[3];
};

__global__ __launch_bounds__(256) void k_codes(const float* __restrict__ pts, int64_t ps,
                                               int64_t as, int64_t count, int32_t d, Box box,
                                               uint64_t* __restrict__ codes,
                                               int32_t* __restrict__ idx) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  uint64_t code = 0;
  for (int k = 0; k < d; ++k) {
    const double v = __dmul_rn(__dsub_rn((double)pts[i * ps + k * as], box.lo[k]), box.factor[k]);
    double fq = floor(v);
    const double top = (double)((1 << kBits) - 1);
    if (fq > top) fq = top;
    const uint64_t q = (uint64_t)fq;
    for (int b = 0; b < kBits; ++b) code |= ((q >> b) & 1ull) << (d * b + k);
  }
  codes[i] = code;
  idx[i] = (int32_t)i;
}

void bbox(const float* pts, int64_t ps, int64_t as, int64_t count, int32_t d, hipStream_t st,
          float* lo, float* hi) {
  const int64_t per_block = (int64_t)kBoxBlock * kBoxPer;
  const int64_t blocks = (count + per_block - 1) / per_block;
  float* part = (float*)dev_alloc(sizeof(float) * blocks * 2 * d);
  hipLaunchKernelGGL(k_bbox, grid1(blocks, kBoxBlock), dim3(kBoxBlock), 0, st, pts, ps, as, count, d,
                     part);
  SK_LAUNCH_CHECK();
  std::vector<float> h((size_t)(blocks * 2 * d));
  SK_HIP(hipMemcpyAsync(h.data(), part, sizeof(float) * h.size(), hipMemcpyDeviceToHost, st));
  SK_HIP(hipStreamSynchronize(st));
  dev_free(part);
  for (int64_t b = 0; b < blocks; ++b)
    for (int k = 0; k < d; ++k) {
      lo[k] = std::fmin(lo[k], h[b * 2 * d + k]);
      hi[k] = std::fmax(hi[k], h[b * 2 * d + d + k]);
    }
}

}  // namespace

// Points are read as pts[i * ps + k * as] (row-major: ps = d, as = 1; SoA:
// ps = 1, as = padded length).
void morton_sort_strided(const float* x, int64_t xps, int64_t xas, const float* y, int64_t yps,
                         int64_t yas, int64_t n, int64_t m, int32_t d, hipStream_t st,
                         uint64_t* codes_x, int32_t* perm_x, uint64_t* codes_y, int32_t* perm_y) {
  if (d < 1 || d > 3) fail(SINKHORN_ERR_INVALID_ARG, "Morton order needs 1 <= d <= 3");
  float lo[3] = {FLT_MAX, FLT_MAX, FLT_MAX}, hi[3] = {-FLT_MAX, -FLT_MAX, -FLT_MAX};
  bbox(x, xps, xas, n, d, st, lo, hi);
  bbox(y, yps, yas, m, d, st, lo, hi);
  Box box;
  for (int k = 0; k < 3; ++k) {
    box.lo[k] = k < d ? (double)lo[k] : 0.0;
    const double span = k < d ? (double)hi[k] - (double)lo[k] : 0.0;
    box.factor[k] = span > 0.0 ? (double)(1 << kBits) / span : 0.0;
  }
  const int64_t big = n > m ? n : m;
  uint64_t* ktmp = (uint64_t*)dev_alloc(sizeof(uint64_t) * big);
  int32_t* vtmp = (int32_t*)dev_alloc(sizeof(int32_t) * big);
  void* temp = nullptr;
  try {
    size_t temp_bytes = 0;
    SK_HIP(rocprim::radix_sort_pairs(nullptr, temp_bytes, ktmp, codes_x, vtmp, perm_x,
                                     (size_t)big, 0, d * kBits, st));
    temp = dev_alloc(temp_bytes);
    for (int side = 0; side < 2; ++side) {
      const float* pts = side == 0 ? x : y;
      const int64_t ps = side == 0 ? xps : yps;
      const int64_t as = side == 0 ? xas : yas;
      const int64_t count = side == 0 ? n : m;
      uint64_t* kout = side == 0 ? codes_x : codes_y;
      int32_t* vout = side == 0 ? perm_x : perm_y;
      hipLaunchKernelGGL(k_codes, grid1(((count + 255) / 256), 256), dim3(256), 0, st, pts, ps,
                         as, count, d, box, ktmp, vtmp);
      SK_LAUNCH_CHECK();
      size_t tb = temp_bytes;
      SK_HIP(rocprim::radix_sort_pairs(temp, tb, ktmp, kout, vtmp, vout, (size_t)count, 0,
                                       d * kBits, st));
    }
    SK_HIP(hipStreamSynchronize(st));
  } catch (...) {
    dev_free(ktmp);
    dev_free(vtmp);
    dev_free(temp);
    throw;
  }
  dev_free(ktmp);
  dev_free(vtmp);
  dev_free(temp);
}

void morton_sort(const float* x, const float* y, int64_t n, int64_t m, int32_t d, hipStream_t st,
                 uint64_t* codes_x, int32_t* perm_x, uint64_t* codes_y, int32_t* perm_y) {
  morton_sort_strided(x, d, 1, y, d, 1, n, m, d, st, codes_x, perm_x, codes_y, perm_y);
}

void morton_sort_soa(const float* x, int64_t xpad, const float* y, int64_t ypad, int64_t n,
                     int64_t m, int32_t d, hipStream_t st, uint64_t* codes_x, int32_t* perm_x,
                     uint64_t* codes_y, int32_t* perm_y) {
  morton_sort_strided(x, 1, xpad, y, 1, ypad, n, m, d, st, codes_x, perm_x, codes_y, perm_y);
}

}  // namespace sk

extern "C" int sinkhorn_morton_order(const float* x, const float* y, int64_t n, int64_t m,
                                     int32_t d, void* stream, uint64_t* codes_x, int32_t* perm_x,
                                     uint64_t* codes_y, int32_t* perm_y) {
  try {
    if (!x || !y || !codes_x || !perm_x || !codes_y || !perm_y)
      sk::fail(SINKHORN_ERR_INVALID_ARG, "null pointer");
    if (n < 1 || m < 1 || n > INT32_MAX || m > INT32_MAX)
      sk::fail(SINKHORN_ERR_INVALID_ARG, "n and m must be in [1, 2^31)");
    sk::morton_sort(x, y, n, m, d, (hipStream_t)stream, codes_x, perm_x, codes_y, perm_y);
    return SINKHORN_OK;
  } catch (const sk::Failure& e) {
    sk::set_last_error(e.msg);
    return e.code;
  } catch (...) {
    sk::set_last_error("unexpected exception");
    return SINKHORN_ERR_HIP;
  }
}

extern "C" int sinkhorn_morton_sort(sinkhorn_problem* p, int32_t side, int32_t* perm_out,
                                    uint64_t* codes_out) {
  uint64_t* other_codes = nullptr;
  int32_t* other_perm = nullptr;
  try {
    if (!p || !perm_out || !codes_out) sk::fail(SINKHORN_ERR_INVALID_ARG, "null pointer");
    if (side != 0 && side != 1) sk::fail(SINKHORN_ERR_INVALID_ARG, "side must be 0 (x) or 1 (y)");
    if (p->d > 3 || !p->X.soa || !p->Y.soa)
      sk::fail(SINKHORN_ERR_UNSUPPORTED, "Morton codes are built for d <= 3");
    if (p->n > INT32_MAX || p->m > INT32_MAX)
      sk::fail(SINKHORN_ERR_INVALID_ARG, "n and m must be < 2^31");
    // both sides share one bounding box, so both are quantized; the other
    // side's codes and order go to temporary buffers
    const int64_t other = side == 0 ? p->m : p->n;
    other_codes = (uint64_t*)sk::dev_alloc(sizeof(uint64_t) * other);
    other_perm = (int32_t*)sk::dev_alloc(sizeof(int32_t) * other);
    uint64_t* cx = side == 0 ? codes_out : other_codes;
    int32_t* px = side == 0 ? perm_out : other_perm;
    uint64_t* cy = side == 1 ? codes_out : other_codes;
    int32_t* py = side == 1 ? perm_out : other_perm;
    sk::morton_sort_soa(p->X.soa, p->X.padded, p->Y.soa, p->Y.padded, p->n, p->m, p->d, p->stream,
                        cx, px, cy, py);
    sk::dev_free(other_codes);
    sk::dev_free(other_perm);
    return SINKHORN_OK;
  } catch (const sk::Failure& e) {
    sk::dev_free(other_codes);
    sk::dev_free(other_perm);
    sk::set_last_error(e.msg);
    return e.code;
  } catch (...) {
    sk::dev_free(other_codes);
    sk::dev_free(other_perm);
    sk::set_last_error("unexpected exception");
    return SINKHORN_ERR_HIP;
  }
}
