// Internal declarations shared by the host entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cmath>
#include <cstdint>
#include <string>
#include <vector>

#include "launch_plan.h"
#include "sinkhorn.h"

namespace sk {

// ---------------------------------------------------------------- errors
struct Failure {
  int code;
  std::string msg;
};

[[noreturn]] void fail(int code, const std::string& msg);
void check_hip(hipError_t e, const char* what);
void set_last_error(const std::string& msg);
// Progress line on stderr (flushed) when the environment variable
// SINKHORN_LOG is set to a non-empty value other than "0"; printf format.
void progress(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

#define SK_HIP(call) ::sk::check_hip((call), #call)
#define SK_LAUNCH_CHECK() ::sk::check_hip(hipGetLastError(), "kernel launch")

// Grid of a 1-D launch of `blocks` workgroups of `threads` work-items;
// SINKHORN_ERR_UNSUPPORTED when it exceeds what one dispatch can hold
// (launch_plan.h), instead of a launch that would drop workgroups.
inline dim3 grid1(int64_t blocks, int64_t threads) {
  if (!grid_fits(blocks, threads))
    fail(SINKHORN_ERR_UNSUPPORTED, "launch of " + std::to_string(blocks) + " x " +
                                       std::to_string(threads) +
                                       " work-items exceeds one dispatch (2^32 - 1)");
  return dim3((uint32_t)blocks);
}

// ---------------------------------------------------------------- constants
constexpr double kLog2e = 1.4426950408889634074;  // 1 / ln 2
constexpr double kLn2 = 0.69314718055994530942;
// Every side is stored padded to a multiple of this many points; padding has
// zero coordinates and a -inf column term, so it never contributes.
constexpr int64_t kPad = 1024;
// Points per column chunk of the VALU kernel (one scalar load per array).
constexpr int kChunk = 16;
// Largest d served by the VALU difference-form kernel; above it the cross
// term runs on MFMA.
constexpr int kMaxValuD = 8;
// Largest d served by the MFMA kernel (K = d + 1 rounded up to 4 stays <= 64).
constexpr int kMaxMfmaD = 63;
// Row tiles per MFMA kernel uses 32-point tiles, K padded to a multiple of 4.
constexpr int kMfmaTile = 32;

inline int64_t round_up(int64_t v, int64_t q) { return (v + q - 1) / q * q; }

// ---------------------------------------------------------------- device memory
void* dev_alloc(size_t bytes);
void dev_free(void* p);
// device bytes allocated minus freed by the calling host thread, and the
// largest value that count reached since thread_alloc_mark() (which starts
// a new interval at the current count)
int64_t thread_alloc_current();
void thread_alloc_mark();
int64_t thread_alloc_peak();
void* host_alloc(size_t bytes);  // pinned
void* host_alloc_coherent(size_t bytes);  // pinned, mapped, coherent with device writes
void host_free(void* p);

// One cloud as stored by a handle.
struct Side {
  int64_t count = 0;   // points
  int64_t padded = 0;  // round_up(count, kPad)
  float* soa = nullptr;    // [d][padded] coordinates (VALU path), zero padding
  float* rowmaj = nullptr; // [padded][kpad] centred coordinates, column term, 1 (MFMA path)
  float* norm2 = nullptr;  // [padded] ||centred point||^2 (MFMA path)
  float* w = nullptr;      // [count] weights
  float* H = nullptr;      // [padded] column term of this side, -inf padding
  double* soa64 = nullptr; // [d][padded] coordinates widened to fp64 (fp64 half-steps, d <= 3)
  double* H64 = nullptr;   // [padded] fp64 column term, -inf padding (fp64 half-steps)
  float* Hhi = nullptr;    // [padded] H64 split for the shifted precise loop: an integer ...
  float* Wlo = nullptr;    // [padded] ... and the weight 2^(H64 - Hhi) (fp32)
  double wsum = 0.0;
};

// Results a half-step leaves on the device; read back with one copy.
struct Ctl {
  double residual;     // last fused residual (sum over rows of w_i |exp((prev_i - new_i)/eps) - 1|)
  int32_t nonfinite;   // non-finite potentials written since the last reset
  int32_t pad;
};

struct LocalFrame;

// Per-launch description of one dense half-step "rows against columns".
struct HalfStep {
  const Side* rows;
  const Side* cols;
  const float* Hcols;      // column term (log2 units) of the column side
  float* pot_out;          // [rows.count]
  const float* pot_prev;   // nullable, for the residual
  float* H_next;           // nullable: column term of the row side for the next step
  double eps;              // eps of this half-step
  double eps_next;         // eps used for H_next
  bool residual;
  // previous potential of the row side: enables the shifted pair loop (its
  // fixed per-row shift is estimated from it); null runs the exact loop
  const float* shift_pot = nullptr;
  // sparse half-steps in shifted mode: the column side's tile-local frame
  // (built for the same B) and the column side's potentials, from which the
  // frame's weights are refreshed; null runs every tile in the difference form
  LocalFrame* frame = nullptr;
  const float* cols_pot = nullptr;
};

// One dense half-step with fp64 potentials, column terms and pair
// arithmetic (dense64.hip, d <= 3).
struct HalfStep64 {
  const Side* rows;
  const Side* cols;
  const double* Hcols;      // fp64 column term (log2 units) of the column side
  float* out32;             // new potential of the row side, fp32 (nullable)
  double* out64;            // the same in fp64 (nullable)
  const float* prev32;      // previous potential for the residual (nullable) ...
  const double* prev64;     // ... or this one (nullable)
  double* Hnext;            // nullable: fp64 column term of the row side for the next step
  double eps;               // eps of this half-step
  double eps_next;          // eps used for Hnext
  bool residual;
  // previous potential of the row side (fp64): sets each row's shift; null
  // runs the exact two-pass form
  const double* shift_pot;
};

}  // namespace sk

struct sinkhorn_problem {
  int64_t n = 0, m = 0;
  int32_t d = 0;
  int32_t kpad = 0;  // MFMA K (d + 2 rounded up to a multiple of 4), 0 on the VALU path
  double scale = 1.0;
  hipStream_t stream = nullptr;
  sk::Side X, Y;
  // split-m partials of the row reduction: [max_split][max(npad, mpad)] each
  float* Mpart = nullptr;
  float* Spart = nullptr;
  int64_t part_cap = 0;  // floats per partial array
  float* bary_part = nullptr;  // barycentric weighted-sum partials, grown on demand
  int64_t bary_cap = 0;        // floats in bary_part
  // residual block partials, arrival counters and the reduced values
  double* red_part = nullptr;   // [red_cap]
  int64_t red_cap = 0;
  int32_t* tile_flag = nullptr; // [red_cap] tiles marked for the exact recompute, zero between launches
  // sparse half-steps: dispatch order of the row tiles (heaviest first), grown on demand
  uint32_t* order_key = nullptr;  // [2 * order_cap] sort keys, in then out
  int32_t* order_val = nullptr;   // [2 * order_cap] tile indices, in then out
  int64_t order_cap = 0;
  void* order_temp = nullptr;     // rocPRIM sort storage
  size_t order_temp_bytes = 0;
  sk::Ctl* ctl = nullptr;       // device control block
  sk::Ctl* host_ctl = nullptr;  // pinned, host-coherent mirror (the residual kernel writes it)
  sk::Ctl* host_ctl_dev = nullptr;  // device address of host_ctl
  int32_t device = 0;           // the HIP device the handle was created on
  int32_t num_cu = 0;           // compute units of the device
  double* host_tmp = nullptr;   // [8] pinned scratch
  // solve scratch: double-buffered potentials
  float* fbuf[2] = {nullptr, nullptr};
  float* gbuf[2] = {nullptr, nullptr};
  // fp64 dense path (d <= 3 unless SINKHORN_FLAG_FP32_PAIRS): the solve's
  // fp64 potentials and a row-shift scratch
  bool precise = false;
  uint32_t flags = 0;
  double* fbuf64[2] = {nullptr, nullptr};
  double* gbuf64[2] = {nullptr, nullptr};
  double* shift64 = nullptr;  // [max(n, m)]
  int64_t workspace_bytes = 0;  // device bytes the handle holds
  hipEvent_t ev = nullptr;
  // measurement hook: event pairs around pair-loop kernel launches
  int32_t prof = 0;                 // SINKHORN_PROF_* kinds being timed
  std::vector<hipEvent_t> prof_ev;  // 2 per launch, reused across reads
  size_t prof_used = 0;             // launches recorded since the last read
  double prof_pairs = 0.0;
};

namespace sk {

// setup.hip helpers
void zero_i32(int32_t* v, int32_t count, hipStream_t st);
void fill_f64(double* v, int64_t count, double value, hipStream_t st);
void widen_f32(const float* src, int64_t count, double* dst, hipStream_t st);
void narrow_f64(const double* src, int64_t count, float* dst, hipStream_t st);
void fill_f32(float* v, int64_t count, float value, hipStream_t st);
void copy_f32(const float* src, int64_t count, float* dst, hipStream_t st);

// measurement hook (api.hip): call around a pair-loop kernel launch
// Profiling of one launch of `kind`: events for hipExtLaunchKernelGGL, which
// the dispatch itself records at the kernel's start and end (null when `kind`
// is not being profiled); prof_done after the launch counts it.
struct ProfEv {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
ProfEv prof_events(sinkhorn_problem* p, int32_t kind);
void prof_done(sinkhorn_problem* p, int32_t kind, double pairs);

// dense.hip
// Column split of the dense VALU pair kernels for nrows x ncols: G splits of
// cps chunks over nchunks chunks of kChunk columns (trailing splits may be
// empty), tiles of 128 rows.
struct SplitInfo {
  int32_t G;     // a power of two
  int32_t glog;  // log2 G
  int64_t cps, nchunks, tiles;
};
SplitInfo dense_split(sinkhorn_problem* p, int64_t nrows, int64_t ncols);
int64_t partial_floats_needed(sinkhorn_problem* p, int64_t nrows, int64_t rows_padded,
                              int64_t ncols);
void prep_column_term(sinkhorn_problem* p, const Side& side, const float* pot, double eps,
                      float* H);
void dense_halfstep(sinkhorn_problem* p, const HalfStep& hs);
// dense64.hip
void dense_halfstep64(sinkhorn_problem* p, const HalfStep64& hs);
void prep_column_term64(sinkhorn_problem* p, const Side& side, const float* pot32,
                        const double* pot64, double eps, double* H);
int64_t dense64_partial_floats(sinkhorn_problem* p, int64_t nrows, int64_t ncols);
// enqueue the copy of the control block to its pinned mirror
void copy_ctl(sinkhorn_problem* p);
// returns (residual sum, nonfinite count) after a synchronizing read
void read_reduction(sinkhorn_problem* p, double* value, int32_t* nonfinite);
void reset_nonfinite(sinkhorn_problem* p);
// row groups of the pair kernel for a side of `rows` points (for buffer sizing)
int64_t row_groups(int64_t rows);

// setup.hip
// with64: also the fp64 coordinates and column term of the fp64 half-steps
void side_init(sinkhorn_problem* p, Side& s, const float* pts, const float* w, int64_t count,
               bool with64);
void side_free(Side& s);
// per-dimension (sum, sum of squares) of a device cloud [count][d] -> host [d][2]
void moments(const float* pts, int64_t count, int32_t d, hipStream_t st, double* host_out);
// mfma.hip (d > kMaxValuD)
void setup_mfma(sinkhorn_problem* p, const float* x, const float* y);
void mfma_halfstep(sinkhorn_problem* p, const HalfStep& hs);
void mfma_column_term(sinkhorn_problem* p, const Side& side, const float* pot, double eps);
int64_t mfma_partial_floats(sinkhorn_problem* p, int64_t nrows, int64_t ncols);

// blocks.hip: per-block summaries of a side in its stored order
constexpr int64_t kGrp = 64;  // blocks per screen group

struct BlockSummary {
  int64_t nb = 0;        // blocks
  int32_t B = 0;         // points per block
  double* lo = nullptr;  // [3][nb] per-axis minimum (fp32 values widened)
  double* hi = nullptr;  // [3][nb] per-axis maximum
  double* lw = nullptr;  // [nb] log(points * max weight), C library log on the host
  double* F = nullptr;   // [nb] maximum potential, refreshed per screen
  // groups of kGrp consecutive blocks for the screen's skip test
  int64_t ng = 0;
  double* glo = nullptr;  // [3][ng] union box
  double* ghi = nullptr;
  double* glw = nullptr;  // [ng] maximum log W
  double* gF = nullptr;   // [ng] maximum potential, refreshed with F
  void release();
};
void block_static(sinkhorn_problem* p, const Side& s, int32_t B, BlockSummary& out);

// Tile-local frame of one side for the shifted sparse half-steps (d <= 3).
// Static per side and B: the centre o_J of each block's bounding box, the
// radius R_J of the block about it, and every point's offset y_j - o_J
// (fp32). Refreshed before each half-step from the side's potentials, in
// fp64: h'_j = log2 w_j + lam pot_j - kappa ||y_j - o_J||^2, its block maximum
// m_J and the point's weight 2^(h'_j - m_J) rounded to fp32 (0 for massless
// points and padding; m_J = -inf for a block without mass).
struct LocalFrame {
  int64_t nb = 0;          // blocks
  int32_t B = 0;           // points per block
  int64_t stride = 0;      // the side's padded count
  float* rec = nullptr;    // per 16-point chunk d rows of 16 offsets from the block
                           // centre, then 16 weights; 0 on padding
  float* ctr = nullptr;    // [nb][4]: o_J in the first d slots, R_J in slot 3
  double* mx = nullptr;    // [nb] m_J
  void release();
};
void frame_build(sinkhorn_problem* p, const Side& s, int32_t B, LocalFrame& out);
void frame_weights(sinkhorn_problem* p, const Side& s, const float* pot, double eps, LocalFrame& fr);
void block_potential_max(sinkhorn_problem* p, const float* pot, int64_t count, BlockSummary& s);
int64_t screen_tiles(sinkhorn_problem* p, const BlockSummary& rows, const BlockSummary& cols,
                     double eps, double delta_rel, int64_t* ptr, int32_t* idx, int64_t cap,
                     int64_t* counts_tmp);
int64_t count_empty_rows(sinkhorn_problem* p, const int64_t* ptr, int64_t nr);
void sparse_halfstep(sinkhorn_problem* p, const HalfStep& hs, int32_t B, const int64_t* ptr,
                     const int32_t* idx, double pairs);
void check_csr(sinkhorn_problem* p, const int64_t* ptr, int64_t nr, const int32_t* idx, int64_t nc);
// dispatch order of the row tiles (128 rows) of a sparse list with block
// size B: one entry per workgroup (*slots of them), a tile index or -1, in the
// handle's scratch; one run of tiles per XCD, longest lists first in each
const int32_t* heavy_first(sinkhorn_problem* p, const int64_t* ptr, int64_t tiles, int32_t B,
                           int64_t dense_work, int64_t* slots);

// api.hip: annealed dense solve between two sides (X rows, Y columns), f/g
// in/out, F/G scratch pairs; stall_window > 0 adds the stall stop rule
struct SolveOut {
  int64_t halfsteps = 0, iters = 0, final_iters = 0;
  double pairs = 0.0, row_l1 = NAN, col_l1 = NAN, seconds = 0.0;
  int32_t stages = 0, converged = 0;
  bool stalled = false;
  int status = SINKHORN_OK;
  std::vector<double> history;  // row residual at every check at eps_target
};
SolveOut dense_solve(sinkhorn_problem* p, Side& X, Side& Y, float* f, float* g, float* F[2],
                     float* G[2], const sinkhorn_schedule& s, int32_t stall_window,
                     double stall_rel);

// morton.hip: sorted codes and the original index of each sorted point
void morton_sort(const float* x, const float* y, int64_t n, int64_t m, int32_t d, hipStream_t st,
                 uint64_t* codes_x, int32_t* perm_x, uint64_t* codes_y, int32_t* perm_y);
void morton_sort_soa(const float* x, int64_t xpad, const float* y, int64_t ypad, int64_t n,
                     int64_t m, int32_t d, hipStream_t st, uint64_t* codes_x, int32_t* perm_x,
                     uint64_t* codes_y, int32_t* perm_y);

// materialize.hip: records the device address of the static scratch of the
// allocation-free materializer for `device` (the current device), once
void static_scratch_setup(int device);

double device_mean_sqeuclid(const float* x, const float* y, int64_t n, int64_t m, int32_t d,
                            hipStream_t st);

}  // namespace sk
