// Entry points whose kernels are not in this build yet: they validate nothing
// and report SINKHORN_ERR_UNSUPPORTED.
#include "internal.h"


extern "C" {
int sinkhorn_morton_order(const float*, const float*, int64_t, int64_t, int32_t, void*, uint64_t*,
                          int32_t*, uint64_t*, int32_t*) {
  return SINKHORN_ERR_UNSUPPORTED;
}
int sinkhorn_block_screen(sinkhorn_problem*, double, const float*, const float*, int32_t, double,
                          int32_t, int64_t*, int32_t*, int64_t, int64_t*) {
  return SINKHORN_ERR_UNSUPPORTED;
}
int sinkhorn_sparse_halfstep_f(sinkhorn_problem*, double, const float*, int32_t, const int64_t*,
                               const int32_t*, float*, const float*, double*) {
  return SINKHORN_ERR_UNSUPPORTED;
}
int sinkhorn_sparse_halfstep_g(sinkhorn_problem*, double, const float*, int32_t, const int64_t*,
                               const int32_t*, float*, const float*, double*) {
  return SINKHORN_ERR_UNSUPPORTED;
}
int sinkhorn_solve_multiscale(sinkhorn_problem*, const sinkhorn_multiscale_params*, float*, float*,
                              sinkhorn_multiscale_report*) {
  return SINKHORN_ERR_UNSUPPORTED;
}
}
