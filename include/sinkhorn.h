/*
 * sinkhorn.h - C ABI of the MI355X (gfx950) online log-domain Sinkhorn library.
 *
 * Problem (FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport, §2.1):
 * entropic optimal transport between source points x (n x d) with weights a
 * and target points y (m x d) with weights b under the squared-Euclidean
 * cost C_ij = s * ||x_i - y_j||^2, where the cost scale s is a number resolved
 * once by the caller (moscot pull request #846, "Two correctness traps": the
 * scale travels as a resolved value, never re-derived from a subset).
 *
 * Conventions shared by every entry point:
 *   plan      pi_ij = a_i b_j exp((f_i + g_j - C_ij) / eps)
 *   f-step    f_i = -eps * LSE_j( log b_j + (g_j - C_ij) / eps )
 *   g-step    g_j = -eps * LSE_i( log a_i + (f_i - C_ij) / eps )
 *   residual  R_row = sum_i |sum_j pi_ij - a_i|,  R_col = sum_j |sum_i pi_ij - b_j|
 * The cost is recomputed on the fly and never stored; working memory is
 * O((n + m) d) (FlashSinkhorn 2, §2.1).
 *
 * Memory and streams:
 *   - Every float / int array argument is a DEVICE pointer unless marked
 *     "host". Arrays are contiguous; points are row-major [count][d]; weights
 *     and potentials are [count] in the caller's point order.
 *   - The caller owns all argument buffers. A problem handle copies x, y, a, b
 *     at init (the caller may free them afterwards) and owns only its
 *     O((n + m) d) workspace.
 *   - All device work is enqueued on the stream given at init (a hipStream_t
 *     passed as void*; NULL means the null stream). Calls that return host
 *     values (residuals, counts, thresholds, reports) synchronize that stream.
 *   - A handle must not be used from two host threads at once; separate
 *     handles (each on its own stream) may be used from separate threads
 *     concurrently, and give the same results as when used one at a time.
 *
 * Errors: every function returns an int status. 0 = SINKHORN_OK, positive =
 * success with a note, negative = error. No exception or abort crosses the
 * ABI. sinkhorn_last_error() gives a detail string for the calling thread.
 * Index arithmetic is 64-bit throughout (n * m may exceed 2^31).
 *
 * Progress: with the environment variable SINKHORN_LOG set (to anything but
 * "" or "0"), sinkhorn_solve prints a line per annealing stage and at its end,
 * and sinkhorn_solve_multiscale a line per stage and per fine update, on
 * stderr.
 */
#ifndef SINKHORN_H
#define SINKHORN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SINKHORN_OK 0
#define SINKHORN_NOT_CONVERGED 1      /* iteration cap reached; outputs are valid */
#define SINKHORN_ERR_INVALID_ARG (-1) /* bad size, null pointer, eps or scale not finite and > 0 */
#define SINKHORN_ERR_OOM (-2)         /* device or pinned host allocation failed */
#define SINKHORN_ERR_HIP (-3)         /* HIP runtime or launch error (detail in sinkhorn_last_error) */
#define SINKHORN_ERR_CAPACITY (-4)    /* output list too small; *nnz_out holds the required count */
#define SINKHORN_ERR_NONFINITE (-5)   /* a potential or residual came out NaN or infinite */
#define SINKHORN_ERR_MASS (-6)        /* sum(a) and sum(b) differ by more than 1e-5 relative */
#define SINKHORN_ERR_UNSUPPORTED (-7) /* valid request this build does not implement */

typedef struct sinkhorn_problem sinkhorn_problem; /* opaque handle */

/* Annealing schedule (FlashSinkhorn 2, §3.1 and §B.2: annealing in eps with
 * warm starts). Stages eps_start, eps_start*eps_factor, ... while above
 * eps_target, each running iters_per_stage full iterations (f-step then
 * g-step). Then at eps_target: exactly fixed_iters iterations if fixed_iters > 0;
 * otherwise iterate until max(R_row, R_col) <= tol (tested after every full
 * iteration when check_every <= 1, else after every check_every-th), at most
 * max_iters iterations. */
typedef struct {
  double eps_start;
  double eps_target;
  double eps_factor;      /* in (0, 1) */
  int32_t iters_per_stage;
  int32_t fixed_iters;
  double tol;
  int32_t max_iters;
  int32_t check_every;
} sinkhorn_schedule;

/* Filled by sinkhorn_solve (host struct). history / history_cap are inputs:
 * a host buffer (may be NULL with history_cap = 0) that receives the row
 * residuals of the last history_cap checks at eps_target, oldest first;
 * history_len returns how many checks there were (it may exceed the cap). */
typedef struct {
  int64_t halfsteps;       /* dense or sparse potential updates launched */
  int64_t iters;           /* full iterations, all stages */
  int64_t final_iters;     /* full iterations at eps_target */
  double pairs_evaluated;  /* point pairs visited by all half-steps */
  double row_l1;           /* R_row of the returned potentials */
  double col_l1;           /* R_col of the returned potentials */
  double seconds;          /* host wall time of the call */
  int32_t stages;          /* annealing stages run (eps_target not counted) */
  int32_t converged;       /* 1 if the stop test passed */
  double* history;         /* in: host buffer for the residual history, or NULL */
  int32_t history_cap;     /* in: its capacity in doubles (0 with NULL) */
  int32_t history_len;     /* out: residual checks made at eps_target */
  double seconds_per_halfstep;  /* out: seconds / halfsteps (host wall time) */
  int64_t workspace_bytes;      /* out: device bytes the handle holds (its O((n + m) d) workspace) */
  int64_t peak_extra_bytes;     /* out: most device memory the call held beyond the handle's */
} sinkhorn_report;

/* Human-readable name of a status code. Never NULL. */
const char* sinkhorn_strerror(int code);
/* Detail of the last error raised on the calling host thread ("" if none). */
const char* sinkhorn_last_error(void);

/* Unweighted mean of ||x_i - y_j||^2 over all n*m pairs, computed on the device
 * in fp64 through mean||x||^2 + mean||y||^2 - 2 mean(x) . mean(y). This is the
 * "mean" cost scaling that moscot #846 resolves once over the full clouds
 * ("Two correctness traps"); pass 1 / mean as cost_scale. x [n][d], y [m][d]
 * device; mean_out host. Synchronizes the stream. */
int sinkhorn_mean_sqeuclid(const float* x, const float* y, int64_t n, int64_t m, int32_t d,
                           void* stream, double* mean_out);

/* Create a problem handle: copies x [n][d], y [m][d] (device) and the weights
 * a [n], b [m] (device; NULL = uniform 1/n, 1/m) into device-resident layouts.
 * Requires n, m >= 1, 1 <= d <= 63 (d <= 8 runs the difference form on the
 * vector ALU, larger d the MFMA cross term on centred clouds), cost_scale finite and > 0, weights >= 0
 * (negative weights are not checked and give undefined results); returns
 * SINKHORN_ERR_MASS if |sum a - sum b| > 1e-5 * max(sum a, sum b), and
 * SINKHORN_ERR_NONFINITE if a coordinate or weight is NaN or infinite.
 * The handle (host pointer) is written to *out. In moscot #846 the row
 * materializer is built once and then called per batch of row indices, the
 * geometry resolved before the row loop; the handle plays that role.
 * flags: 0, or SINKHORN_FLAG_FP32_PAIRS (below); other bits are refused. */
int sinkhorn_init(sinkhorn_problem** out, const float* x, const float* y, const float* a,
                  const float* b, int64_t n, int64_t m, int32_t d, double cost_scale,
                  uint32_t flags, void* stream);

/* For d <= 3 the dense half-steps (and the dense solve's potentials between
 * them) compute in fp64 up to the shifted exponent, whose exp2 is fp32
 * (FlashSinkhorn 2, §A.1: the arithmetic's precision moves the potentials):
 * with |potential| >> eps an fp32 column term, row shift or stored potential
 * rounds each half-step by ~1e-5 eps in a way that depends on the iterate,
 * and thousands of iterations at small eps integrate it (2e-2 eps after 2229
 * iterations at eps = 1e-4). This flag selects the fp32 pair loop instead:
 * about 1.4x faster on this chip, and within 1e-5 max(eps, |f|) per
 * half-step, but its solves drift as described. d > 3 always runs fp32. */
#define SINKHORN_FLAG_FP32_PAIRS 1u

/* Release the handle and its workspace (synchronizes its stream). NULL is a no-op. */
int sinkhorn_destroy(sinkhorn_problem* p);

/* Device memory the library holds in this process, over all handles (host
 * outputs; any may be NULL): the bytes allocated now, the peak and the largest
 * single buffer since the last reset; reset != 0 then sets the peak to the
 * current amount and the largest buffer to 0. Every device allocation of the
 * library goes through one allocator, so the figures are exact; buffers the
 * caller passes in are not counted. For callers that check the working
 * memory of a call, in the way moscot #846 ("fix(sparsify): materialize
 * transport-matrix rows ...", its memory measurements) checks that row
 * extraction no longer grows with n * m * k. Needs no device. */
int sinkhorn_device_memory(int64_t* current_bytes, int64_t* peak_bytes, int64_t* largest_bytes,
                           int32_t reset);

/* Sizes of a handle (host outputs; any may be NULL). */
int sinkhorn_problem_info(const sinkhorn_problem* p, int64_t* n, int64_t* m, int32_t* d,
                          double* cost_scale);

/* One dense f-step (FlashSinkhorn 2, §2.1: the source dual update as a tiled
 * streaming log-sum-exp; the cost is recomputed per pair and never stored):
 *   f_out_i = -eps * LSE_j( log b_j + (g_j - C_ij) / eps ),  g [m] -> f_out [n].
 * If f_prev [n] and row_l1 (host) are both non-NULL, also returns the row
 * residual of the state (f_prev, g), which equals
 *   sum_i a_i |exp((f_prev_i - f_out_i) / eps) - 1|
 * because the f-step makes every row sum to a_i (and synchronizes).
 * f_out may not alias g or f_prev. An all -inf row (every b_j = 0) gives
 * f_out = +inf and SINKHORN_ERR_NONFINITE. */
int sinkhorn_halfstep_f(sinkhorn_problem* p, double eps, const float* g, float* f_out,
                        const float* f_prev, double* row_l1);

/* The g-step, the same reduction with the roles of the sides swapped:
 *   g_out_j = -eps * LSE_i( log a_i + (f_i - C_ij) / eps ),  f [n] -> g_out [m];
 * col_l1 (host, with g_prev) is the column residual of the state (f, g_prev). */
int sinkhorn_halfstep_g(sinkhorn_problem* p, double eps, const float* f, float* g_out,
                        const float* g_prev, double* col_l1);

/* Exact L1 marginal residuals of (f, g) (FlashSinkhorn 2, §3.1: the exact
 * residual is an O(nm) pass): one row pass and one column pass over all pairs,
 * writing no potential. row_l1 and col_l1 are host pointers (either may be NULL). */
int sinkhorn_marginal_residual(sinkhorn_problem* p, double eps, const float* f, const float* g,
                               double* row_l1, double* col_l1);

/* Annealed dense solve (FlashSinkhorn 2, §2.1 alternating updates, §3.1
 * annealing). f [n], g [m] are in/out warm starts (zeros for a cold start);
 * on return they hold the potentials whose residual passed the stop test (the
 * last full iteration when fixed_iters > 0). rep (host) may be NULL.
 * Returns SINKHORN_NOT_CONVERGED when max_iters ran out. */
int sinkhorn_solve(sinkhorn_problem* p, const sinkhorn_schedule* sched, float* f, float* g,
                   sinkhorn_report* rep);

/* Entropic transport-plan rows (moscot #846, "Fix": T[rows] = exp((f + g - C)/eps)
 * built directly from the potentials, never through an n x m x k tensor):
 *   T[r][j] = a_i b_j exp((f_i + g_j - C_ij) / eps),  i = rows[r],
 * rows int64 [k] device (0 <= rows[r] < n), T [k][m] device fp32 row-major,
 * row_max [k] device (may be NULL) = max_j T[r][j]. */
int sinkhorn_materialize_rows(sinkhorn_problem* p, double eps, const float* f, const float* g,
                              const int64_t* rows, int64_t k, float* T, float* row_max);

/* sinkhorn_materialize_rows for callers that cannot allocate device memory
 * during the call (code that must not call hipMalloc: tight serving loops
 * over row batches, harnesses that forbid allocation). Same arguments,
 * results and synchronization as sinkhorn_materialize_rows (the same kernels,
 * so the same values bit for bit), but the call allocates nothing: its
 * per-call buffers (row terms, row-maximum keys and, for d <= 8, fp64 column
 * terms) live in one fixed array in the library's device memory, 16.8 MB per
 * GPU, set up by sinkhorn_init and held until the process ends. Limits:
 * k <= 4096 rows per call, and m <= 2^21 columns when d <= 8 (no limit on m
 * for d > 8); beyond them the call returns SINKHORN_ERR_INVALID_ARG and does
 * nothing. Every call on one GPU shares that array: calls that overlap in
 * time on the same GPU (other host threads, other streams) race and give
 * undefined results; calls one after the other are independent. */
int sinkhorn_materialize_rows_noalloc(sinkhorn_problem* p, double eps, const float* f,
                                      const float* g, const int64_t* rows, int64_t k, float* T,
                                      float* row_max);

/* min over rows with a_i > 0 of max_j T_ij (moscot #846, "Behavioural changes":
 * the largest threshold that keeps every row non-empty, exact and independent
 * of the batch; rows without mass take no part). Computed in row batches
 * without storing T. out (host) is NaN when every a_i is 0. */
int sinkhorn_min_row(sinkhorn_problem* p, double eps, const float* f, const float* g,
                     float* out);

/* Morton (Z-order) codes and a stable Morton order of both clouds
 * (FlashSinkhorn 2, §3: Morton sorting makes cells and blocks of consecutive
 * points spatially compact). d <= 3; 21 bits per axis over the bounding box of
 * x and y together, q_k = min(2^21 - 1, floor((p_k - lo_k) * (2^21 / (hi_k - lo_k))))
 * in fp64 (0 on a flat axis), bit b of axis k at position d*b + k; ties keep
 * the original order. Outputs (device): codes_x [n] / codes_y [m] sorted codes,
 * perm_x [n] / perm_y [m] original index of each sorted point. */
int sinkhorn_morton_order(const float* x, const float* y, int64_t n, int64_t m, int32_t d,
                          void* stream, uint64_t* codes_x, int32_t* perm_x, uint64_t* codes_y,
                          int32_t* perm_y);

/* The same Morton order for one side of a handle (side 0: x, 1: y), from
 * the handle's own copies of the clouds: both sides are quantized over the
 * bounding box of x and y together, exactly as sinkhorn_morton_order does,
 * so codes_out [count] (device, sorted) and perm_out [count] (device,
 * original index of each sorted point) equal that call's outputs for the
 * side. d <= 3 (SINKHORN_ERR_UNSUPPORTED otherwise). Allocates the other
 * side's codes and order for the duration of the call; synchronizes the
 * handle's stream. */
int sinkhorn_morton_sort(sinkhorn_problem* p, int32_t side, int32_t* perm_out,
                         uint64_t* codes_out);

/* Block-pair screen (FlashSinkhorn 2, §3.2 and §B.3: block-level potential
 * maxima and bounding boxes; §A.3: an omitted tile drops at most
 * delta_rel * a_i per row and delta_rel * b_j per column). Blocks are B
 * consecutive points of the handle's clouds in their stored order (sort them
 * first). Tile (I, J) is omitted iff, in fp64,
 *   (F_I + G_J) - D_IJ <= eps * (log(delta_rel) - max(log W^a_I, log W^b_J))
 * with F_I = max f over I, G_J = max g over J, D_IJ = s * sum_k gap_k^2,
 * gap_k = max(0, lo_Jk - hi_Ik, lo_Ik - hi_Jk), W = points * max weight of the
 * block. transpose = 0 gives the row-major list (ptr [NB+1] over source blocks,
 * idx = admitted target blocks in increasing order); transpose = 1 the
 * column-major list of the same tiles (ptr [MB+1], idx = source blocks).
 * ptr int64 and idx int32 are device arrays; cap is idx's capacity. *nnz_out
 * (host) gets the tile count; if it exceeds cap the call returns
 * SINKHORN_ERR_CAPACITY and idx is not written. 1 <= B <= 1024. */
int sinkhorn_block_screen(sinkhorn_problem* p, double eps, const float* f, const float* g,
                          int32_t B, double delta_rel, int32_t transpose, int64_t* ptr,
                          int32_t* idx, int64_t cap, int64_t* nnz_out);

/* Tile verification (FlashSinkhorn 2, §3.2: screened tiles are checked with
 * their exact mass over the B^2 point pairs; §C.5). Input: a row-major
 * candidate list ptr [NB+1] (ptr[0] = 0) / idx [nnz] as written by
 * sinkhorn_block_screen (transpose = 0), B = 128, d <= 3. A candidate (I, J)
 * is dropped iff at (f, g), for every i in I,
 *   sum_{j in J} b_j exp((f_i + g_j - C_ij)/eps) <= delta_rel
 * and for every j in J,
 *   sum_{i in I} a_i exp((f_i + g_j - C_ij)/eps) <= delta_rel
 * (each dropped tile then takes at most delta_rel a_i from row i and
 * delta_rel b_j from column j, the screen's own guarantee; sums in fp32, a NaN
 * keeps the tile). A row block that would lose every candidate keeps them all,
 * then likewise a column block. Outputs (device, caller-owned): vptr [NB+1] /
 * vidx the kept tiles row-major in candidate order, tptr [MB+1] / tidx the
 * same tiles column-major (source blocks increasing per target block); vidx
 * and tidx need room for nnz entries. *kept_out (host) = kept count.
 * Synchronizes the handle's stream. */
int sinkhorn_verify_tiles(sinkhorn_problem* p, double eps, const float* f, const float* g,
                          int32_t B, double delta_rel, const int64_t* ptr, const int32_t* idx,
                          int64_t* vptr, int32_t* vidx, int64_t* tptr, int32_t* tidx,
                          int64_t* kept_out);

/* Sparse f-step on a row-major tile list (FlashSinkhorn 2, §3.2: log-sum-exp
 * over admitted tiles only; a block with no admitted tile takes a dense
 * update). Same outputs as sinkhorn_halfstep_f, with the residual (when
 * f_prev and row_l1 are given) taken over the same support. With f_prev the
 * rows carry shifts from it and each admitted tile is evaluated about its
 * column block's bounding-box centre: per-column weights and per-tile scales
 * in fp64 (rounded once), the cross terms of each 16 x 16 pair block on the
 * matrix cores in fp32. A tile whose rows lie too far from the block for the
 * fp32 range, or whose block's weights span more than the normal fp32 range,
 * takes the plain difference form. The call then holds (4 d + 4) B of device
 * memory per column point and 24 B per column block until it returns.
 * Synchronizes the handle's stream. */
int sinkhorn_sparse_halfstep_f(sinkhorn_problem* p, double eps, const float* g, int32_t B,
                               const int64_t* ptr, const int32_t* idx, float* f_out,
                               const float* f_prev, double* row_l1);

/* Sparse g-step on the column-major list of the same tiles. */
int sinkhorn_sparse_halfstep_g(sinkhorn_problem* p, double eps, const float* f, int32_t B,
                               const int64_t* ptr, const int32_t* idx, float* g_out,
                               const float* g_prev, double* col_l1);

/* Multiscale solve parameters (FlashSinkhorn 2, §1, §3, §3.1, §3.2, §B.1, §B.2). */
typedef struct {
  int32_t B;                /* block size (points per block) */
  int32_t p_bits;           /* Morton prefix bits of a cell; <= 0: floor(log2(2 max(NB, MB))) */
  double eps;               /* target eps */
  double tol;               /* stop when max(R_A,row, R_A,col) + Omega <= tol */
  double delta_scale;       /* delta_rel = delta_scale / max(NB, MB); Omega = delta_scale */
  double coarse_eps_start;  /* coarse annealing start */
  double coarse_factor;     /* coarse annealing factor */
  int32_t coarse_iters_per_stage;
  double coarse_tol;        /* coarse stop: R <= coarse_tol, ... */
  int32_t coarse_max;       /* ... or this many iterations at the target eps, ... */
  int32_t stall_window;     /* ... or R > (1 - stall_rel) * R of stall_window iterations before */
  double stall_rel;
  int32_t max_fine;         /* cap on fine updates */
  int32_t verify;           /* nonzero: verify the screened tiles (sinkhorn_verify_tiles rule,
                               B = 128) before each fine update's half-steps */
  /* Adaptive coarse-to-fine switch (FlashSinkhorn 2, §3.1, §B.2), when nonzero: the coarse
   * stage runs in batches of check_every centroid updates (the first after the annealing
   * stages), each ending early on coarse_tol or a stall; after each batch the potentials are
   * lifted and accepted, with no fine update, when est + 3 SE < tol holds on both sides
   * (est, SE: sampled L1 residual estimate and its standard error; check_samples indices per side,
   * check_samples_max when that interval straddles tol; the same indices at every check).
   * Otherwise batches continue until the coarse stage converges, stalls or reaches
   * coarse_max, and the certified fine loop follows. Sample k of a side of size c is
   * word k % 4 of Philox4x64-10 at counter (k / 4 + 1, 0, 0, 0) with key
   * (sample_seed, side), side 0 for x and 1 for y, modulo c. */
  int32_t adaptive;
  int32_t check_every;
  int32_t check_samples;
  int32_t check_samples_max;
  uint64_t sample_seed;
  /* Continuation, when nonzero: no cells, coarse stage or lift; the fine
   * loop starts from f and g as given (caller's order) and runs as above. */
  int32_t warm_start;
} sinkhorn_multiscale_params;

typedef struct {
  int64_t coarse_iters;
  int64_t fine_updates;
  int64_t ncells_x, ncells_y;
  int64_t last_tiles;       /* admitted tiles of the last mask */
  double pairs_evaluated;   /* all point pairs visited (coarse, lift, fine, checks) */
  double R_A_row, R_A_col;  /* admitted-plan residuals of the returned potentials */
  double omega;             /* a-priori omitted-mass bound */
  double seconds_total, seconds_sort, seconds_coarse, seconds_lift, seconds_fine;
  int32_t certified;
  int64_t last_candidates;  /* screened tiles of the last mask (= last_tiles without verify) */
  int32_t accepted_by_sample;  /* adaptive: a lift passed the sampled check (no fine update) */
  int64_t checks;              /* adaptive: sampled checks run */
  int64_t last_check_samples;  /* samples per side of the last check */
  double last_check[4];        /* its row estimate, row standard error, column estimate, column
                                  standard error */
  int64_t peak_extra_bytes;    /* most device memory the call held beyond the handle's */
} sinkhorn_multiscale_report;

/* Block-sparse multiscale solve for d <= 3 (FlashSinkhorn 2): Morton sort,
 * Morton-prefix cells with mass-weighted centroids, annealed coarse Sinkhorn
 * on the cells, lift of the coarse potentials to the points, then fine updates
 * that each rebuild the block-pair mask and run the sparse f- and g-steps,
 * stopping when the certificate max(R_A,row, R_A,col) + Omega <= tol holds.
 * f [n], g [m] (device) receive the potentials in the caller's order (with
 * warm_start they also give the starting potentials); rep (host) may be
 * NULL. Returns SINKHORN_NOT_CONVERGED at the fine cap. */
int sinkhorn_solve_multiscale(sinkhorn_problem* p, const sinkhorn_multiscale_params* prm,
                              float* f, float* g, sinkhorn_multiscale_report* rep);

/* Sample indices of the sampled residual checks (FlashSinkhorn 2, §B.2: 1024
 * indices per side, up to 8192): out[k] (device int32) = word k % 4 of
 * Philox4x64-10 (Salmon et al., SC 2011) at counter (k / 4 + 1, 0, 0, 0) with
 * key (seed, stream_id), modulo count; uniform with replacement, and a longer
 * draw repeats a shorter one. 1 <= count < 2^31. Synchronizes `stream`. */
int sinkhorn_sample_indices(int64_t count, int32_t k, uint64_t seed, uint64_t stream_id, void* stream,
                            int32_t* out);

/* Sampled marginal residual (FlashSinkhorn 2, §3.1: sampled row sums cost
 * O(md)): draws k indices of one side of the handle's clouds in their stored
 * order (side 0: rows of x, stream 0; side 1: rows of y, stream 1; indices as
 * sinkhorn_sample_indices with this seed), evaluates each drawn row's
 * |sum_j pi_ij - w_i| at (f, g) with one dense half-step of those rows, and
 * returns (host) the estimate count * mean and its standard error
 * count * std (k - 1 in the variance) / sqrt(k) of the L1 residual of that
 * side. 2 <= k <= 2^24, d <= 8. Synchronizes the handle's stream. */
int sinkhorn_sampled_residual(sinkhorn_problem* p, double eps, const float* f, const float* g,
                              int32_t side, int32_t k, uint64_t seed, double* est, double* se);

/* Sparsified plan (moscot pull request #846: thresholding on the device and
 * moving only the surviving values and indices): every entry T_ij >= threshold,
 * as CSR in the caller's row order. row_ptr [n + 1] (device int64) is always
 * written; col [cap] (device int32 column indices, increasing within a row)
 * and val [cap] (device fp32 T_ij) when both are given and cap >= nnz. Entries
 * are computed exactly as sinkhorn_materialize_rows computes them, `batch`
 * rows at a time (<= 0: 1024; at most 2^28 entries per batch), so only
 * surviving entries are stored. threshold must be finite and > 0, so rows
 * without mass keep no entry; with the value sinkhorn_min_row returns, every
 * row with mass keeps at least its largest entry. nnz_out (host) receives
 * the count. Returns SINKHORN_ERR_CAPACITY when col/val are given but cap <
 * nnz (row_ptr and nnz_out are still valid). Synchronizes the stream. */
int sinkhorn_sparsify(sinkhorn_problem* p, double eps, const float* f, const float* g,
                      float threshold, int64_t batch, int64_t* row_ptr, int32_t* col, float* val,
                      int64_t cap, int64_t* nnz_out);

/* Barycentric projection of plan rows and the source-coordinate gradient
 * (FlashSinkhorn 2, §A.2): with the target side and g held fixed,
 *   T_i    = sum_j pi_ij y_j / sum_j pi_ij
 *          = sum_j w_ij y_j / sum_j w_ij,   w_ij = b_j exp((g_j - C_ij)/eps)
 *   grad_i = 2 s a_i (x_i - T_i)            (the derivative in x_i, C = s||x - y||^2)
 * The row factor of the plan cancels, so only g enters; f_hint (device [n],
 * nullable) is used only to choose each row's shift in the streaming sum (the
 * f-step potential of g is best; NULL runs the running-max loop). T and grad
 * (device, [n][d] row-major fp32, caller order) may each be NULL, not both.
 * d <= 8; ERR_UNSUPPORTED otherwise. Asynchronous on the handle's stream. */
int sinkhorn_barycentric(sinkhorn_problem* p, double eps, const float* g, const float* f_hint,
                         float* T, float* grad);

/* The same on the block mask (FlashSinkhorn 2, §A.4, masked gradient): row
 * block I of B stored points averages over the columns of its admitted tiles
 * (ptr/idx as from sinkhorn_block_screen; all columns for a block with none).
 * B a multiple of 128 (at most 1024), d <= 3. The launches are asynchronous
 * on the handle's stream; before them the tile-list check and the dispatch
 * plan (the list lengths per XCD run) synchronize it. */
int sinkhorn_sparse_barycentric(sinkhorn_problem* p, double eps, const float* g,
                                const float* f_hint, int32_t B, const int64_t* ptr,
                                const int32_t* idx, float* T, float* grad);

/* Measurement hook. `kinds` is a bit set of the kernels to time: every later
 * launch of a selected kernel carries two HIP events that its own dispatch
 * records at the kernel's start and end (hipExtLaunchKernelGGL), so the time
 * is the kernel's alone; 0 stops recording.
 *   SINKHORN_PROF_DENSE        dense pair-loop reductions: the shifted VALU loop
 *                              and the MFMA kernel
 *   SINKHORN_PROF_SPARSE       sparse (block-masked) pair-loop reductions
 *   SINKHORN_PROF_MATERIALIZE  plan-row materializer
 *   SINKHORN_PROF_BARY         dense barycentric pair kernel
 *   SINKHORN_PROF_DENSE_EXACT  dense VALU pair loop in exact mode (residual
 *                              passes without a shift estimate)
 * sinkhorn_profile_read synchronizes the stream and returns (host pointers,
 * any may be NULL) the summed kernel time of the recorded launches in ms, their
 * number, and the point pairs (materializer: entries) they evaluated; it then
 * clears the record. */
#define SINKHORN_PROF_DENSE 1
#define SINKHORN_PROF_SPARSE 2
#define SINKHORN_PROF_MATERIALIZE 4
#define SINKHORN_PROF_BARY 8
#define SINKHORN_PROF_DENSE_EXACT 16
int sinkhorn_profile_enable(sinkhorn_problem* p, int32_t kinds);
int sinkhorn_profile_read(sinkhorn_problem* p, double* kernel_ms, int64_t* launches,
                          double* pairs);

/* Issue-rate probe: the vector-ALU ceiling of this device for the pair
 * kernels' instruction mix, measured rather than taken from a data sheet
 * (FlashSinkhorn 2, §C.6 accounts for its kernels' cost in instructions per
 * pair). Runs one probe kernel of `iters` iterations on `stream` (NULL: the
 * null stream) over 8 waves per SIMD of every compute unit and returns (host
 * pointers, any may be NULL) the lane-instructions retired per second of the
 * counted class, the point pairs per second for the pair probes (0
 * otherwise) and the kernel time in ms (HIP events around the launch, after
 * one warm-up launch). Kinds (each iteration four independent chains):
 *   SINKHORN_PROBE_FMA_F32        v_fma_f32 on VGPRs; counts the FMAs
 *   SINKHORN_PROBE_EXP_F32        v_exp_f32 alone; counts the exps
 *   SINKHORN_PROBE_FMA_F64        v_fma_f64 on VGPRs; counts the FMAs
 *   SINKHORN_PROBE_PAIR_F32       one d = 3 pair of the dense half-step's fp32
 *                                 loop: 3 v_sub_f32 (scalar operand), v_fma_f32,
 *                                 2 v_fmac_f32, v_fma_f32 (scalar operand),
 *                                 v_exp_f32, v_add_f32; counts the 8 non-exp
 *   SINKHORN_PROBE_PAIR_F32_NOEXP the same without the v_exp_f32
 *   SINKHORN_PROBE_PAIR_F64       the same pair in fp64 up to the exponent:
 *                                 3 v_add_f64, 4 v_fma_f64, v_cvt_f32_f64,
 *                                 v_exp_f32, v_add_f32; counts the 9 non-exp
 *   SINKHORN_PROBE_SUB_F32        v_sub_f32 with a scalar operand
 *   SINKHORN_PROBE_FMAC_F32       v_fmac_f32 (accumulator in the destination)
 *   SINKHORN_PROBE_ADD_F64        v_add_f64 with a scalar operand
 *   SINKHORN_PROBE_CVT_F32_F64    v_cvt_f32_f64 (the CVT probe also sums its
 *                                 results: 4 v_add_f32 per 4 conversions,
 *                                 not counted)
 *   SINKHORN_PROBE_PAIR_TILE_F32  one pair of a tile-local expanded form:
 *                                 v_mul_f32 + 2 v_fmac_f32 (scalar column
 *                                 offsets), v_exp_f32, v_fmac_f32 (scalar
 *                                 column weight); counts the 4 non-exp
 *   SINKHORN_PROBE_PAIR_SPLIT_F32 one pair of the dense split form: 3
 *                                 v_sub_f32, v_mul_f32 + 2 v_fmac_f32,
 *                                 v_sub_f32 (scalar integer column term),
 *                                 v_fmac_f32, v_exp_f32, v_fmac_f32 (scalar
 *                                 weight); counts the 9 non-exp
 *   SINKHORN_PROBE_PAIR_TILE_MFMA the same form with the cross terms on the
 *                                 matrix cores, as the sparse half-step
 *                                 runs it: per wave four 16 x 16 pair
 *                                 blocks, each 3 v_mfma_f32_4x4x1_16b_f32
 *                                 (one per coordinate), then v_exp_f32 and
 *                                 v_fmac_f32 per pair; counts the 1 fmac
 * Synchronizes `stream`. */
#define SINKHORN_PROBE_FMA_F32 0
#define SINKHORN_PROBE_EXP_F32 1
#define SINKHORN_PROBE_FMA_F64 2
#define SINKHORN_PROBE_PAIR_F32 3
#define SINKHORN_PROBE_PAIR_F32_NOEXP 4
#define SINKHORN_PROBE_PAIR_F64 5
#define SINKHORN_PROBE_SUB_F32 6
#define SINKHORN_PROBE_FMAC_F32 7
#define SINKHORN_PROBE_ADD_F64 8
#define SINKHORN_PROBE_CVT_F32_F64 9
#define SINKHORN_PROBE_PAIR_TILE_F32 10
#define SINKHORN_PROBE_PAIR_SPLIT_F32 11
#define SINKHORN_PROBE_PAIR_TILE_MFMA 12
int sinkhorn_probe_issue_rate(int32_t kind, int32_t iters, void* stream, double* lane_instr_per_s,
                              double* pairs_per_s, double* kernel_ms);

#ifdef __cplusplus
}
#endif

#endif /* SINKHORN_H */
