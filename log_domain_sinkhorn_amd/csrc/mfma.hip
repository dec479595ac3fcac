// Dense online half-step for larger d (9 <= d <= 63) with the cross term on
// fp32 MFMA.
//
// FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport, §2.1: the
// half-steps are tiled reductions whose cross term is a dense matrix product;
// working memory stays O((n + m) d).
//
// With both clouds centred on c = (mean x + mean y)/2 (the cost is unchanged),
//   log2-exponent z_ij = 2 kappa (x_i . y_j + H'_j) - kappa ||x_i||^2,
//   H'_j = (log2 b_j + g_j log2(e)/eps) / (2 kappa) - ||y_j||^2 / 2,
//   kappa = s log2(e) / eps,
// so f_i = s ||x_i||^2 - eps ln2 LSE2_j(2 kappa D_ij) with
//   D_ij = sum_k y_jk x_ik + H'_j.
// Each side is stored row-major [padded][KP] with KP = round_up(d + 2, 4):
// slots 0..d-1 hold the centred coordinates, slot d holds H' of that side
// (written whenever the side is the column side, -inf on padding rows), slot
// KP - 1 holds 1, the rest zeros. In registers the row side takes 2 kappa x
// for the coordinates, 2 kappa for slot d and -c_i for slot KP - 1, where c_i
// is the row's running shift, so one v_mfma_f32_32x32x2f32 chain over KP
// produces 2 kappa D_ij - c_i directly; every column j of a 32-point tile
// lands in one of 16 accumulator registers of a lane whose lane % 32 selects
// the row i, and the log-sum-exp runs over those registers.
//
// The shift c_i is an integer no smaller than some exponent already seen in
// the row, so the row sum S_i = sum 2^(z - c_i) stays >= 1/2 and nothing
// underflows that matters; it is raised (and S_i rescaled) only when a tile
// holds an exponent more than 64 above it, or at the row's first finite
// tile. Every other tile costs one exp2 and one add per pair on the VALU,
// which runs serially with the matrix pipe on this SIMD.
//
// Mapping: a workgroup = 4 waves x 2 row tiles of 32 (256 rows); all waves of
// a workgroup stream the same column tiles, staged in LDS (double-buffered,
// odd row stride so the per-lane column reads are bank-conflict free). G
// workgroups per row block split the columns when the rows alone give too few
// workgroups; their partials are merged by the shared merge kernel.
#include <cfloat>
#include <cmath>

#include "rowfinal.h"

namespace sk {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float ex2(float v) { return __builtin_amdgcn_exp2f(v); }

constexpr int kMW = 4;                     // waves per workgroup
constexpr int kIT = 2;                     // 32-row tiles per wave
constexpr int kRowsPerWG = kMW * kIT * 32; // 256

struct MfmaArgs {
  const float* P;   // row side [padded][KP]
  const float* Q;   // column side [padded][KP]
  int32_t d;
  float twokappa;   // 2 s log2(e) / eps
  int32_t G;
  int64_t ntiles;   // column tiles of 32 points
  int64_t tps;      // column tiles per split
  float* Mp;
  float* Sp;
  RowFinal F;
};

template <int KP>
__global__ __launch_bounds__(256) void k_lse_mfma(MfmaArgs A) {
  constexpr int KH = KP / 2;
  constexpr int LW = KP + 1;           // odd LDS row stride
  constexpr int NV4 = 32 * KP / 4;     // float4 per column tile
  constexpr int PER = (NV4 + 255) / 256;
  __shared__ float sY[2][32 * LW];
  __shared__ double sRed[256];

  const int32_t gs = (int32_t)(blockIdx.x % (uint32_t)A.G);
  const int64_t tile = blockIdx.x / (uint32_t)A.G;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int kh = lane >> 5;
  const int64_t ibase = tile * kRowsPerWG + wave * (kIT * 32);

  // B operands: row i = ibase + it*32 + l32, k = 2 kk + kh; slot KP - 1
  // (lanes with kh = 1, kk = KH - 1) carries -c_i, starting at 0
  const float tk = A.twokappa;
  float bx[kIT][KH];
#pragma unroll
  for (int it = 0; it < kIT; ++it)
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
      const int k = 2 * kk + kh;
      const float v = A.P[(ibase + it * 32 + l32) * KP + k];
      bx[it][kk] = k == A.d ? tk : (k == KP - 1 ? 0.0f : tk * v);
    }

  const int64_t t0 = (int64_t)gs * A.tps;
  const int64_t t1 = t0 + A.tps < A.ntiles ? t0 + A.tps : A.ntiles;
  float c[kIT], S[kIT];
  bool have[kIT];  // the row has seen a finite exponent (same on both lanes of a row)
#pragma unroll
  for (int it = 0; it < kIT; ++it) {
    c[it] = 0.0f;
    S[it] = 0.0f;
    have[it] = false;
  }
  float4 pre[PER];
  auto gload = [&](int64_t t) {
    const float4* src = reinterpret_cast<const float4*>(A.Q + t * 32 * KP);
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
    v16f acc[kIT];
#pragma unroll
    for (int it = 0; it < kIT; ++it) acc[it] = (v16f){};
    const float* ys = &sY[buf][l32 * LW + kh];
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
      const float a = ys[2 * kk];
#pragma unroll
      for (int it = 0; it < kIT; ++it)
        acc[it] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bx[it][kk], acc[it], 0, 0, 0);
    }
    // acc = z - c: one exp2 and one add per pair unless a shift must move
    float s[kIT];
    bool need = false;
#pragma unroll
    for (int it = 0; it < kIT; ++it) {
      float v = ex2(acc[it][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) v += ex2(acc[it][r]);
      s[it] = v;
      need = need || !have[it] || !(v <= 0x1p64f);
    }
    if (__ballot(need) == 0) {
#pragma unroll
      for (int it = 0; it < kIT; ++it) S[it] += s[it];
    } else {
      // all lanes: raise each row's shift to the ceiling of the tile's
      // largest exponent when that is above it (or set it at the row's first
      // finite tile), then add the tile relative to the new shift
#pragma unroll
      for (int it = 0; it < kIT; ++it) {
        float cm = acc[it][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) cm = fmaxf(cm, acc[it][r]);
        cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
        if (cm > -INFINITY) {
          float k = ceilf(cm);
          if (have[it]) k = fmaxf(k, 0.0f);
          float v = 0.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) v += ex2(acc[it][r] - k);
          S[it] = __builtin_fmaf(S[it], ex2(-k), v);
          c[it] += k;
          have[it] = true;
          if (kh) bx[it][KH - 1] = -c[it];
        }
      }
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // lanes l and l + 32 hold the same row: merge the two halves
  double term = 0.0;
  int bad = 0;
#pragma unroll
  for (int it = 0; it < kIT; ++it) {
    const float M = have[it] ? c[it] : -FLT_MAX;
    const float Mo = __shfl_xor(M, 32, 64);
    const float So = __shfl_xor(S[it], 32, 64);
    const float mx = fmaxf(M, Mo);
    const float s = __builtin_fmaf(S[it], ex2(M - mx), So * ex2(Mo - mx));
    const int64_t i = ibase + it * 32 + l32;
    if (kh == 0 && i < A.F.np) {
      if (A.G > 1) {
        A.Mp[(int64_t)gs * A.F.np + i] = mx;
        A.Sp[(int64_t)gs * A.F.np + i] = s;
      } else {
        term += finalize_row(A.F, i, mx, (double)s, &bad);
      }
    }
  }
  if (A.G == 1) {
    if (bad) atomicAdd(&A.F.ctl->nonfinite, bad);
    if (A.F.prev) {
      sRed[threadIdx.x] = term;
      __syncthreads();
#pragma unroll
      for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) sRed[threadIdx.x] += sRed[threadIdx.x + w];
        __syncthreads();
      }
      if (threadIdx.x == 0) A.F.red_part[tile] = sRed[0];
    }
  }
}

// Centred row-major layout: slot d = 0 for real rows, -inf for padding rows,
// slot kp - 1 = 1, norm2 = ||centred fp32 point||^2 (fp64 sum, rounded once).
__global__ __launch_bounds__(256) void k_centre(const float* __restrict__ pts, int64_t count,
                                                int32_t d, int32_t kp, int64_t padded,
                                                const double* __restrict__ c,
                                                float* __restrict__ out,
                                                float* __restrict__ norm2) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= padded) return;
  double n2 = 0.0;
  for (int32_t k = 0; k < kp; ++k) {
    float v = 0.0f;
    if (i < count && k < d) {
      v = (float)((double)pts[i * d + k] - c[k]);
      n2 += (double)v * (double)v;
    } else if (k == d && i >= count) {
      v = -INFINITY;
    } else if (k == kp - 1) {
      v = 1.0f;
    }
    out[i * kp + k] = v;
  }
  norm2[i] = (float)n2;
}

// H'_j = (log2 w_j + pot_j lam) / (2 kappa) - norm2_j / 2 into slot d.
__global__ __launch_bounds__(256) void k_column_term_mfma(const float* __restrict__ w,
                                                          const float* __restrict__ pot,
                                                          const float* __restrict__ norm2,
                                                          int64_t count, double lam,
                                                          double inv2k, float* __restrict__ slot,
                                                          int32_t kp) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j < count)
    slot[j * kp] = (float)((log2((double)w[j]) + (double)pot[j] * lam) * inv2k -
                           0.5 * (double)norm2[j]);
}

// Merge of the G split partials [G][np] (fp32 shift or max, fp32 sum) of
// each row, then finalize; with F.prev the residual terms are summed per
// 256-row block. A workgroup holds 256 rows and 4 groups of 4 waves: group q
// folds splits q, q + 4, ... of its rows (coalesced across the rows) with a
// running maximum, and the first group combines the four in group order, so
// the result does not depend on timing.
constexpr int kMergeGroups = 4;

__global__ __launch_bounds__(256 * kMergeGroups) void k_merge_splits(RowFinal F, int32_t G,
                                                                     const float* __restrict__ Mp,
                                                                     const float* __restrict__ Sp) {
  __shared__ float sM[kMergeGroups][256];
  __shared__ double sS[kMergeGroups][256];
  __shared__ double sRed[256];
  const int r = threadIdx.x & 255;
  const int q = threadIdx.x >> 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + r;
  float mx = -FLT_MAX;
  double sum = 0.0;
  if (i < F.np) {
    for (int32_t t = q; t < G; t += kMergeGroups) {
      const int64_t o = (int64_t)t * F.np + i;
      const float m = Mp[o];
      const double s = (double)Sp[o];
      if (m > mx) {
        sum = __builtin_fma(sum, (double)ex2(mx - m), s);
        mx = m;
      } else {
        sum = __builtin_fma(s, (double)ex2(m - mx), sum);
      }
    }
  }
  sM[q][r] = mx;
  sS[q][r] = sum;
  __syncthreads();
  double term = 0.0;
  int bad = 0;
  if (q == 0 && i < F.np) {
    float m = sM[0][r];
#pragma unroll
    for (int k = 1; k < kMergeGroups; ++k) m = fmaxf(m, sM[k][r]);
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < kMergeGroups; ++k) s = __builtin_fma(sS[k][r], (double)ex2(sM[k][r] - m), s);
    term = finalize_row(F, i, (double)m, s, &bad);
  }
  if (bad) atomicAdd(&F.ctl->nonfinite, bad);
  if (F.prev) {
    if (q == 0) sRed[r] = term;
    __syncthreads();
#pragma unroll
    for (int w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) sRed[threadIdx.x] += sRed[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) F.red_part[blockIdx.x] = sRed[0];
  }
}

void merge_splits(sinkhorn_problem* p, const RowFinal& F, int32_t G) {
  const int64_t nblocks = (F.np + 255) / 256;
  hipLaunchKernelGGL(k_merge_splits, grid1(nblocks, 256 * kMergeGroups), dim3(256 * kMergeGroups), 0,
                     p->stream, F, G, p->Mpart, p->Spart);
  SK_LAUNCH_CHECK();
  if (F.prev) launch_reduce(p, nblocks);
}

struct MPlan {
  int32_t G;
  int64_t tps;
  int64_t ntiles;
  int64_t tiles;
};

// Workgroups of k_lse_mfma<KP> resident on the whole chip at once (queried
// once per instantiation, thread-safe as in the VALU path).
template <int KP>
int64_t slots_kp(sinkhorn_problem* p) {
  static const int per_cu = [] {
    int nb = 0;
    SK_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_lse_mfma<KP>, 256, 0));
    return nb > 0 ? nb : 1;
  }();
  return (int64_t)per_cu * p->num_cu;
}

int64_t mfma_slots(sinkhorn_problem* p) {
  switch (p->kpad) {
    case 12: return slots_kp<12>(p);
    case 16: return slots_kp<16>(p);
    case 20: return slots_kp<20>(p);
    case 24: return slots_kp<24>(p);
    case 28: return slots_kp<28>(p);
    case 32: return slots_kp<32>(p);
    case 36: return slots_kp<36>(p);
    case 40: return slots_kp<40>(p);
    case 44: return slots_kp<44>(p);
    case 48: return slots_kp<48>(p);
    case 52: return slots_kp<52>(p);
    case 56: return slots_kp<56>(p);
    case 60: return slots_kp<60>(p);
    case 64: return slots_kp<64>(p);
    case 68: return slots_kp<68>(p);
    default: fail(SINKHORN_ERR_UNSUPPORTED, "MFMA half-step: unsupported K");
  }
}

// Column splits G per 256-row block: enough workgroups for six rounds of the
// resident slots (every workgroup carries the same number of column tiles,
// so the last, partly filled round costs at most a sixth), a multiple of 8
// once it reaches 8 (workgroups are dealt to the 8 XCDs in turn, so each XCD
// then streams its own column splits), at most 64 and at least 8 column
// tiles per split.
MPlan mplan(int64_t nrows, int64_t ncols, int64_t slots) {
  MPlan mp;
  mp.ntiles = (ncols + 31) / 32;
  mp.tiles = (nrows + kRowsPerWG - 1) / kRowsPerWG;
  int64_t want = (6 * slots + mp.tiles - 1) / mp.tiles;
  if (want >= 8) want = (want + 7) / 8 * 8;
  const int64_t maxsplit = mp.ntiles / 8 > 1 ? mp.ntiles / 8 : 1;
  if (want > 64) want = 64;
  if (want > maxsplit) want = maxsplit;
  // tiles * G workgroups must fit one dispatch
  const int64_t fit = max_blocks_1d(256) / mp.tiles;
  if (want > fit) want = fit;
  if (want < 1) want = 1;
  mp.tps = (mp.ntiles + want - 1) / want;
  mp.G = (int32_t)((mp.ntiles + mp.tps - 1) / mp.tps);
  return mp;
}

template <int KP>
void launch_kp(sinkhorn_problem* p, const MfmaArgs& A, int64_t blocks, double pairs) {
  const ProfEv pe = prof_events(p, SINKHORN_PROF_DENSE);
  hipExtLaunchKernelGGL((k_lse_mfma<KP>), grid1(blocks, 256), dim3(256), 0, p->stream, pe.start,
                        pe.stop, 0, A);
  SK_LAUNCH_CHECK();
  prof_done(p, SINKHORN_PROF_DENSE, pairs);
}

}  // namespace

int64_t mfma_partial_floats(sinkhorn_problem* p, int64_t nrows, int64_t ncols) {
  const MPlan mp = mplan(nrows, ncols, mfma_slots(p));
  return mp.G > 1 ? (int64_t)mp.G * nrows : 1;
}

void setup_mfma(sinkhorn_problem* p, const float* x, const float* y) {
  const int32_t d = p->d;
  if (d > kMaxMfmaD) fail(SINKHORN_ERR_UNSUPPORTED, "d must be <= 63");
  p->kpad = (int32_t)round_up(d + 2, 4);
  std::vector<double> mx(2 * d), my(2 * d), c(d);
  moments(x, p->n, d, p->stream, mx.data());
  moments(y, p->m, d, p->stream, my.data());
  for (int32_t k = 0; k < d; ++k)
    c[k] = 0.5 * (mx[2 * k] / (double)p->n + my[2 * k] / (double)p->m);
  double* dc = (double*)dev_alloc(sizeof(double) * d);
  SK_HIP(hipMemcpyAsync(dc, c.data(), sizeof(double) * d, hipMemcpyHostToDevice, p->stream));
  for (int side = 0; side < 2; ++side) {
    Side& s = side == 0 ? p->X : p->Y;
    const float* pts = side == 0 ? x : y;
    s.rowmaj = (float*)dev_alloc(sizeof(float) * s.padded * p->kpad);
    s.norm2 = (float*)dev_alloc(sizeof(float) * s.padded);
    hipLaunchKernelGGL(k_centre, grid1(((s.padded + 255) / 256), 256), dim3(256), 0, p->stream,
                       pts, s.count, d, p->kpad, s.padded, dc, s.rowmaj, s.norm2);
    SK_LAUNCH_CHECK();
  }
  SK_HIP(hipStreamSynchronize(p->stream));
  dev_free(dc);
}

void mfma_column_term(sinkhorn_problem* p, const Side& side, const float* pot, double eps) {
  const double kappa = p->scale * kLog2e / eps;
  hipLaunchKernelGGL(k_column_term_mfma, grid1(((side.count + 255) / 256), 256), dim3(256), 0,
                     p->stream, side.w, pot, side.norm2, side.count, kLog2e / eps,
                     1.0 / (2.0 * kappa), side.rowmaj + p->d, p->kpad);
  SK_LAUNCH_CHECK();
}

void mfma_halfstep(sinkhorn_problem* p, const HalfStep& hs) {
  const Side& rows = *hs.rows;
  const Side& cols = *hs.cols;
  const MPlan mp = mplan(rows.count, cols.count, mfma_slots(p));
  if (mp.G > 1 && (int64_t)mp.G * rows.count > p->part_cap) fail(SINKHORN_ERR_HIP, "partial buffer too small");
  if (mp.tiles > p->red_cap || (rows.count + 255) / 256 > p->red_cap)
    fail(SINKHORN_ERR_HIP, "reduction buffer too small");
  MfmaArgs A;
  A.P = rows.rowmaj;
  A.Q = cols.rowmaj;
  A.d = p->d;
  const double kappa = p->scale * kLog2e / hs.eps;
  A.twokappa = (float)(2.0 * kappa);
  A.G = mp.G;
  A.ntiles = mp.ntiles;
  A.tps = mp.tps;
  A.Mp = p->Mpart;
  A.Sp = p->Spart;
  A.F = make_rowfinal(p, hs);
  A.F.norm2 = rows.norm2;
  A.F.row_scale = p->scale;
  if (hs.H_next) {
    const double kappa_next = p->scale * kLog2e / hs.eps_next;
    A.F.Hnext = rows.rowmaj + p->d;
    A.F.hstride = p->kpad;
    A.F.hmul = 1.0 / (2.0 * kappa_next);
    A.F.hnorm = 0.5;
  }
  const int64_t blocks = mp.tiles * mp.G;
  const double pairs = (double)rows.count * (double)cols.count;
  switch (p->kpad) {
    case 12: launch_kp<12>(p, A, blocks, pairs); break;
    case 16: launch_kp<16>(p, A, blocks, pairs); break;
    case 20: launch_kp<20>(p, A, blocks, pairs); break;
    case 24: launch_kp<24>(p, A, blocks, pairs); break;
    case 28: launch_kp<28>(p, A, blocks, pairs); break;
    case 32: launch_kp<32>(p, A, blocks, pairs); break;
    case 36: launch_kp<36>(p, A, blocks, pairs); break;
    case 40: launch_kp<40>(p, A, blocks, pairs); break;
    case 44: launch_kp<44>(p, A, blocks, pairs); break;
    case 48: launch_kp<48>(p, A, blocks, pairs); break;
    case 52: launch_kp<52>(p, A, blocks, pairs); break;
    case 56: launch_kp<56>(p, A, blocks, pairs); break;
    case 60: launch_kp<60>(p, A, blocks, pairs); break;
    case 64: launch_kp<64>(p, A, blocks, pairs); break;
    case 68: launch_kp<68>(p, A, blocks, pairs); break;
    default: fail(SINKHORN_ERR_UNSUPPORTED, "MFMA half-step: unsupported K");
  }
  if (mp.G > 1)
    merge_splits(p, A.F, mp.G);
  else if (A.F.prev)
    launch_reduce(p, mp.tiles);
}

}  // namespace sk
