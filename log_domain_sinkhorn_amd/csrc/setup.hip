// Handle set-up: device layouts of the two clouds, weight checks, the fp64
// mean squared distance, and memory helpers.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <unordered_map>

#include "internal.h"

namespace sk {
namespace {

// [count][d] row-major -> [d][padded] SoA with zero padding.
__global__ __launch_bounds__(256) void k_to_soa(const float* __restrict__ pts, int64_t count,
                                                int32_t d, int64_t padded,
                                                float* __restrict__ soa) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= padded) return;
  for (int32_t k = 0; k < d; ++k) soa[(int64_t)k * padded + i] = i < count ? pts[i * d + k] : 0.0f;
}

__global__ __launch_bounds__(256) void k_fill(float* __restrict__ v, int64_t count, float value) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) v[i] = value;
}

__global__ __launch_bounds__(256) void k_fill64(double* __restrict__ v, int64_t count, double value) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) v[i] = value;
}

__global__ __launch_bounds__(256) void k_widen(const float* __restrict__ src, int64_t count,
                                               double* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) dst[i] = (double)src[i];
}

__global__ __launch_bounds__(256) void k_narrow(const double* __restrict__ src, int64_t count,
                                                float* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) dst[i] = (float)src[i];
}

__global__ __launch_bounds__(256) void k_copy(const float* __restrict__ src, int64_t count,
                                              float* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) dst[i] = src[i];
}

// Per block: sum of weights (fp64), count of non-finite coordinates/weights.
__global__ __launch_bounds__(256) void k_check(const float* __restrict__ pts,
                                               const float* __restrict__ w, int64_t count,
                                               int32_t d, double* __restrict__ part,
                                               int32_t* __restrict__ bad) {
  __shared__ double sh[256];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  double v = 0.0;
  int nb = 0;
  if (i < count) {
    const float wi = w[i];
    if (!isfinite(wi)) ++nb;
    v = (double)wi;
    for (int32_t k = 0; k < d; ++k)
      if (!isfinite(pts[i * d + k])) ++nb;
  }
  if (nb) atomicAdd(bad, nb);
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = sh[0];
}

__global__ __launch_bounds__(256) void k_sum_blocks(const double* __restrict__ part, int64_t count,
                                                    double* __restrict__ out) {
  __shared__ double sh[256];
  double acc = 0.0;
  for (int64_t k = threadIdx.x; k < count; k += 256) acc += part[k];
  sh[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = sh[0];
}

__global__ void k_zero_i32(int32_t* v, int32_t count) {
  const int32_t i = (int32_t)(blockIdx.x * 256 + threadIdx.x);
  if (i < count) v[i] = 0;
}

// Column sums and squared norms per dimension: grid (chunks, d); block (c, k)
// sums x[i][k] and x[i][k]^2 over its chunk of points into part[k][c][2].
__global__ __launch_bounds__(256) void k_moments(const float* __restrict__ pts, int64_t count,
                                                 int32_t d, int64_t chunk,
                                                 double* __restrict__ part) {
  __shared__ double s1[256];
  __shared__ double s2[256];
  const int64_t c = blockIdx.x;
  const int32_t k = (int32_t)blockIdx.y;
  const int64_t lo = c * chunk;
  const int64_t hi = lo + chunk < count ? lo + chunk : count;
  double a1 = 0.0, a2 = 0.0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 256) {
    const double v = (double)pts[i * d + k];
    a1 += v;
    a2 += v * v;
  }
  s1[threadIdx.x] = a1;
  s2[threadIdx.x] = a2;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      s1[threadIdx.x] += s1[threadIdx.x + s];
      s2[threadIdx.x] += s2[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int64_t o = ((int64_t)k * gridDim.x + c) * 2;
    part[o] = s1[0];
    part[o + 1] = s2[0];
  }
}

// part[k][c][2] -> out[k][2] (fixed order over c).
__global__ __launch_bounds__(256) void k_moments_reduce(const double* __restrict__ part,
                                                        int64_t nchunk, int32_t d,
                                                        double* __restrict__ out) {
  const int32_t k = (int32_t)(blockIdx.x * 256 + threadIdx.x);
  if (k >= d) return;
  double a1 = 0.0, a2 = 0.0;
  for (int64_t c = 0; c < nchunk; ++c) {
    a1 += part[((int64_t)k * nchunk + c) * 2];
    a2 += part[((int64_t)k * nchunk + c) * 2 + 1];
  }
  out[2 * k] = a1;
  out[2 * k + 1] = a2;
}

inline uint32_t blocks_for(int64_t count) { return (uint32_t)((count + 255) / 256); }

}  // namespace

// Per-dimension (sum, sum of squares) of a cloud, on the host after a sync.
void moments(const float* pts, int64_t count, int32_t d, hipStream_t st, double* host_out) {
  const int64_t nchunk = count < 256 * 64 ? 1 : (count + 256 * 64 - 1) / (256 * 64);
  const int64_t chunk = (count + nchunk - 1) / nchunk;
  double* part = (double*)dev_alloc(sizeof(double) * 2 * nchunk * d);
  double* out = (double*)dev_alloc(sizeof(double) * 2 * d);
  hipLaunchKernelGGL(k_moments, dim3((uint32_t)nchunk, (uint32_t)d), dim3(256), 0, st, pts, count,
                     d, chunk, part);
  SK_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_moments_reduce, grid1(((d + 255) / 256), 256), dim3(256), 0, st, part,
                     nchunk, d, out);
  SK_LAUNCH_CHECK();
  SK_HIP(hipMemcpyAsync(host_out, out, sizeof(double) * 2 * d, hipMemcpyDeviceToHost, st));
  SK_HIP(hipStreamSynchronize(st));
  dev_free(part);
  dev_free(out);
}

// Device memory held by the library: every allocation goes through
// dev_alloc, so the current amount, its peak and the largest single buffer
// are exact (per process, all handles).
namespace {
std::mutex g_mem_mu;
std::unordered_map<void*, size_t> g_mem_size;
int64_t g_mem_current = 0, g_mem_peak = 0, g_mem_largest = 0;
thread_local int64_t t_current = 0, t_peak = 0;
}  // namespace

int64_t thread_alloc_current() { return t_current; }
void thread_alloc_mark() { t_peak = t_current; }
int64_t thread_alloc_peak() { return t_peak; }

void* dev_alloc(size_t bytes) {
  void* p = nullptr;
  if (bytes == 0) bytes = 256;
  const hipError_t e = hipMalloc(&p, bytes);
  if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) {
    (void)hipGetLastError();
    fail(SINKHORN_ERR_OOM, "hipMalloc of " + std::to_string(bytes) + " bytes failed");
  }
  check_hip(e, "hipMalloc");
  std::lock_guard<std::mutex> lock(g_mem_mu);
  g_mem_size[p] = bytes;
  g_mem_current += (int64_t)bytes;
  g_mem_peak = std::max(g_mem_peak, g_mem_current);
  g_mem_largest = std::max(g_mem_largest, (int64_t)bytes);
  t_current += (int64_t)bytes;
  t_peak = std::max(t_peak, t_current);
  return p;
}

void dev_free(void* p) {
  if (!p) return;
  {
    std::lock_guard<std::mutex> lock(g_mem_mu);
    auto it = g_mem_size.find(p);
    if (it != g_mem_size.end()) {
      g_mem_current -= (int64_t)it->second;
      t_current -= (int64_t)it->second;
      g_mem_size.erase(it);
    }
  }
  (void)hipFree(p);
}

void device_memory(int64_t* current, int64_t* peak, int64_t* largest, bool reset) {
  std::lock_guard<std::mutex> lock(g_mem_mu);
  if (current) *current = g_mem_current;
  if (peak) *peak = g_mem_peak;
  if (largest) *largest = g_mem_largest;
  if (reset) {
    g_mem_peak = g_mem_current;
    g_mem_largest = 0;
  }
}

void* host_alloc(size_t bytes) {
  void* p = nullptr;
  const hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    fail(SINKHORN_ERR_OOM, "hipHostMalloc failed");
  }
  return p;
}

void* host_alloc_coherent(size_t bytes) {
  void* p = nullptr;
  const hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocMapped | hipHostMallocCoherent);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    fail(SINKHORN_ERR_OOM, "hipHostMalloc failed");
  }
  return p;
}

void host_free(void* p) {
  if (p) (void)hipHostFree(p);
}

void zero_i32(int32_t* v, int32_t count, hipStream_t st) {
  hipLaunchKernelGGL(k_zero_i32, grid1(((count + 255) / 256), 256), dim3(256), 0, st, v, count);
  SK_LAUNCH_CHECK();
}

void fill_f32(float* v, int64_t count, float value, hipStream_t st) {
  if (count <= 0) return;
  hipLaunchKernelGGL(k_fill, dim3(blocks_for(count)), dim3(256), 0, st, v, count, value);
  SK_LAUNCH_CHECK();
}

void copy_f32(const float* src, int64_t count, float* dst, hipStream_t st) {
  if (count <= 0) return;
  hipLaunchKernelGGL(k_copy, dim3(blocks_for(count)), dim3(256), 0, st, src, count, dst);
  SK_LAUNCH_CHECK();
}

void fill_f64(double* v, int64_t count, double value, hipStream_t st) {
  if (count <= 0) return;
  hipLaunchKernelGGL(k_fill64, grid1((count + 255) / 256, 256), dim3(256), 0, st, v, count, value);
  SK_LAUNCH_CHECK();
}

void widen_f32(const float* src, int64_t count, double* dst, hipStream_t st) {
  if (count <= 0) return;
  hipLaunchKernelGGL(k_widen, grid1((count + 255) / 256, 256), dim3(256), 0, st, src, count, dst);
  SK_LAUNCH_CHECK();
}

void narrow_f64(const double* src, int64_t count, float* dst, hipStream_t st) {
  if (count <= 0) return;
  hipLaunchKernelGGL(k_narrow, grid1((count + 255) / 256, 256), dim3(256), 0, st, src, count, dst);
  SK_LAUNCH_CHECK();
}

void side_init(sinkhorn_problem* p, Side& s, const float* pts, const float* w, int64_t count,
               bool with64) {
  const int32_t d = p->d;
  hipStream_t st = p->stream;
  s.count = count;
  s.padded = round_up(count, kPad);
  s.w = (float*)dev_alloc(sizeof(float) * count);
  if (w)
    copy_f32(w, count, s.w, st);
  else
    fill_f32(s.w, count, (float)(1.0 / (double)count), st);
  s.H = (float*)dev_alloc(sizeof(float) * s.padded);
  fill_f32(s.H, s.padded, -INFINITY, st);
  if (d <= kMaxValuD) {
    s.soa = (float*)dev_alloc(sizeof(float) * (size_t)d * s.padded);
    hipLaunchKernelGGL(k_to_soa, dim3(blocks_for(s.padded)), dim3(256), 0, st, pts, count, d,
                       s.padded, s.soa);
    SK_LAUNCH_CHECK();
    if (with64) {  // the fp64 half-steps read widened coordinates and an fp64 column term
      s.soa64 = (double*)dev_alloc(sizeof(double) * (size_t)d * s.padded);
      widen_f32(s.soa, (int64_t)d * s.padded, s.soa64, st);
      s.H64 = (double*)dev_alloc(sizeof(double) * s.padded);
      fill_f64(s.H64, s.padded, -INFINITY, st);
      s.Hhi = (float*)dev_alloc(sizeof(float) * s.padded);
      s.Wlo = (float*)dev_alloc(sizeof(float) * s.padded);
    }
  }
  // weight sum and finiteness of coordinates and weights
  const uint32_t nb = blocks_for(count);
  double* part = (double*)dev_alloc(sizeof(double) * nb);
  double* out = (double*)dev_alloc(sizeof(double));
  int32_t* badc = (int32_t*)dev_alloc(sizeof(int32_t));
  zero_i32(badc, 1, st);
  hipLaunchKernelGGL(k_check, dim3(nb), dim3(256), 0, st, pts, s.w, count, d, part, badc);
  SK_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_sum_blocks, dim3(1), dim3(256), 0, st, part, (int64_t)nb, out);
  SK_LAUNCH_CHECK();
  SK_HIP(hipMemcpyAsync(p->host_tmp, out, sizeof(double), hipMemcpyDeviceToHost, st));
  SK_HIP(hipMemcpyAsync(p->host_tmp + 1, badc, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  SK_HIP(hipStreamSynchronize(st));
  dev_free(part);
  dev_free(out);
  dev_free(badc);
  s.wsum = p->host_tmp[0];
  int32_t bad;
  memcpy(&bad, p->host_tmp + 1, sizeof(int32_t));
  if (bad) fail(SINKHORN_ERR_NONFINITE, "non-finite coordinate or weight at init");
  if (!(s.wsum > 0.0) || !std::isfinite(s.wsum)) fail(SINKHORN_ERR_INVALID_ARG, "weights must have a positive finite sum");
}

void side_free(Side& s) {
  dev_free(s.soa);
  dev_free(s.soa64);
  dev_free(s.H64);
  dev_free(s.Hhi);
  dev_free(s.Wlo);
  dev_free(s.rowmaj);
  dev_free(s.norm2);
  dev_free(s.w);
  dev_free(s.H);
  s = Side();
}

double device_mean_sqeuclid(const float* x, const float* y, int64_t n, int64_t m, int32_t d,
                            hipStream_t st) {
  double* hx = (double*)host_alloc(sizeof(double) * 2 * d);
  double* hy = (double*)host_alloc(sizeof(double) * 2 * d);
  double mean = 0.0;
  try {
    moments(x, n, d, st, hx);
    moments(y, m, d, st, hy);
    double sx2 = 0.0, sy2 = 0.0, dot = 0.0;
    for (int32_t k = 0; k < d; ++k) {
      sx2 += hx[2 * k + 1];
      sy2 += hy[2 * k + 1];
      dot += (hx[2 * k] / (double)n) * (hy[2 * k] / (double)m);
    }
    mean = sx2 / (double)n + sy2 / (double)m - 2.0 * dot;
  } catch (...) {
    host_free(hx);
    host_free(hy);
    throw;
  }
  host_free(hx);
  host_free(hy);
  return mean;
}

}  // namespace sk
