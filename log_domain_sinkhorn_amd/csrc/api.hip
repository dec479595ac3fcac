// C ABI entry points: argument checks, handle life cycle, half-steps, the
// exact residual and the annealed dense solve driver.
#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "internal.h"

namespace sk {

namespace {
thread_local std::string g_last_error;
}

void set_last_error(const std::string& msg) { g_last_error = msg; }

void fail(int code, const std::string& msg) { throw Failure{code, msg}; }

void progress(const char* fmt, ...) {
  static const bool on = [] {
    const char* e = std::getenv("SINKHORN_LOG");
    return e && *e && std::strcmp(e, "0") != 0;
  }();
  if (!on) return;
  va_list ap;
  va_start(ap, fmt);
  std::fputs("[sinkhorn] ", stderr);
  std::vfprintf(stderr, fmt, ap);
  std::fputc('\n', stderr);
  std::fflush(stderr);
  va_end(ap);
}

void check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    (void)hipGetLastError();
    fail(SINKHORN_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  }
}

ProfEv prof_events(sinkhorn_problem* p, int32_t kind) {
  ProfEv e;
  if (!(p->prof & kind)) return e;
  if (p->prof_ev.size() < 2 * (p->prof_used + 1)) {
    for (int k = 0; k < 2; ++k) {
      hipEvent_t ev;
      SK_HIP(hipEventCreate(&ev));
      p->prof_ev.push_back(ev);
    }
  }
  e.start = p->prof_ev[2 * p->prof_used];
  e.stop = p->prof_ev[2 * p->prof_used + 1];
  return e;
}

void prof_done(sinkhorn_problem* p, int32_t kind, double pairs) {
  if (!(p->prof & kind)) return;
  ++p->prof_used;
  p->prof_pairs += pairs;
}

namespace {

template <class F>
int guard(F&& body) {
  try {
    g_last_error.clear();
    return body();
  } catch (const Failure& f) {
    g_last_error = f.msg;
    return f.code;
  } catch (const std::bad_alloc&) {
    g_last_error = "host allocation failed";
    return SINKHORN_ERR_OOM;
  } catch (...) {
    g_last_error = "unexpected exception";
    return SINKHORN_ERR_HIP;
  }
}

inline void require(bool ok, const char* what) {
  if (!ok) fail(SINKHORN_ERR_INVALID_ARG, what);
}

inline void require_eps(double eps) {
  require(std::isfinite(eps) && eps > 0.0, "eps must be finite and > 0");
}

void problem_free(sinkhorn_problem* p) {
  if (!p) return;
  if (p->stream) (void)hipStreamSynchronize(p->stream);
  side_free(p->X);
  side_free(p->Y);
  dev_free(p->Mpart);
  dev_free(p->Spart);
  dev_free(p->bary_part);
  dev_free(p->red_part);
  dev_free(p->tile_flag);
  dev_free(p->order_key);
  dev_free(p->order_val);
  dev_free(p->order_temp);
  dev_free(p->ctl);
  host_free(p->host_ctl);
  host_free(p->host_tmp);
  for (int k = 0; k < 2; ++k) {
    dev_free(p->fbuf[k]);
    dev_free(p->gbuf[k]);
    dev_free(p->fbuf64[k]);
    dev_free(p->gbuf64[k]);
  }
  dev_free(p->shift64);
  if (p->ev) (void)hipEventDestroy(p->ev);
  for (hipEvent_t e : p->prof_ev) (void)hipEventDestroy(e);
  delete p;
}

// f-step (rows = X) or g-step (rows = Y) with caller buffers.
void halfstep(sinkhorn_problem* p, bool fside, double eps, const float* other, float* out,
              const float* prev, double* l1) {
  require(p != nullptr, "null handle");
  require_eps(eps);
  require(other != nullptr && out != nullptr, "null potential");
  require(out != other && (prev == nullptr || out != prev), "output aliases an input");
  Side& rows = fside ? p->X : p->Y;
  Side& cols = fside ? p->Y : p->X;
  const bool residual = prev != nullptr && l1 != nullptr;
  if (p->precise) {
    prep_column_term64(p, cols, other, nullptr, eps, cols.H64);
    reset_nonfinite(p);
    const double* shift = nullptr;
    if (prev) {  // the previous potential estimates the row shifts
      widen_f32(prev, rows.count, p->shift64, p->stream);
      shift = p->shift64;
    }
    HalfStep64 hs{&rows, &cols, cols.H64, out, nullptr, prev, nullptr, nullptr, eps, eps, residual,
                  shift};
    dense_halfstep64(p, hs);
  } else {
    prep_column_term(p, cols, other, eps, cols.H);
    reset_nonfinite(p);
    HalfStep hs{&rows, &cols, cols.H, out, prev, nullptr, eps, eps, residual};
    hs.shift_pot = prev;  // the previous potential estimates the row shifts
    dense_halfstep(p, hs);
  }
  if (l1) {
    double v = 0.0;
    int32_t bad = 0;
    read_reduction(p, &v, &bad);
    *l1 = residual ? v : NAN;
    if (bad) fail(SINKHORN_ERR_NONFINITE, "non-finite potential in half-step");
  }
}

double seconds_since(std::chrono::steady_clock::time_point t0) {
  return std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
}

}  // namespace

SolveOut dense_solve(sinkhorn_problem* p, Side& X, Side& Y, float* f, float* g, float* F[2],
                     float* G[2], const sinkhorn_schedule& s, int32_t stall_window,
                     double stall_rel) {
  if (!(std::isfinite(s.eps_target) && s.eps_target > 0.0))
    fail(SINKHORN_ERR_INVALID_ARG, "eps_target must be finite and > 0");
  if (!(std::isfinite(s.eps_start) && s.eps_start >= s.eps_target))
    fail(SINKHORN_ERR_INVALID_ARG, "eps_start must be >= eps_target");
  if (!(s.eps_start == s.eps_target || (s.eps_factor > 0.0 && s.eps_factor < 1.0)))
    fail(SINKHORN_ERR_INVALID_ARG, "eps_factor must be in (0, 1)");
  if (s.iters_per_stage < 0 || s.fixed_iters < 0) fail(SINKHORN_ERR_INVALID_ARG, "negative iteration count");
  if (!(s.fixed_iters > 0 || (s.max_iters >= 1 && s.tol >= 0.0)))
    fail(SINKHORN_ERR_INVALID_ARG, "need max_iters >= 1 and tol >= 0");
  const auto t0 = std::chrono::steady_clock::now();
  hipStream_t st = p->stream;
  const double pairs = (double)X.count * (double)Y.count;
  // the handle's own clouds on the fp64 path iterate with fp64 potentials,
  // column terms and pair arithmetic (dense64.hip); other sides (the
  // multiscale cells) in fp32
  const bool precise = p->precise && &X == &p->X && &Y == &p->Y;
  double* F64[2] = {p->fbuf64[0], p->fbuf64[1]};
  double* G64[2] = {p->gbuf64[0], p->gbuf64[1]};
  if (precise) {
    widen_f32(f, X.count, F64[0], st);
    widen_f32(g, Y.count, G64[0], st);
  } else {
    copy_f32(f, X.count, F[0], st);
    copy_f32(g, Y.count, G[0], st);
  }
  reset_nonfinite(p);
  int cur = 0;
  SolveOut o;

  // f-step from state `from` into state 1 - from (fused residual of state
  // `from` when `residual`; with `hnext`, the next column term of X for eps)
  auto fstep = [&](int from, double eps, bool residual, bool hnext) {
    if (precise) {
      HalfStep64 hs{&X, &Y, Y.H64, nullptr, F64[1 - from], nullptr, F64[from],
                    hnext ? X.H64 : nullptr, eps, eps, residual, F64[from]};
      dense_halfstep64(p, hs);
    } else {
      HalfStep hs{&X, &Y, Y.H, F[1 - from], F[from], hnext ? X.H : nullptr, eps, eps, residual};
      hs.shift_pot = F[from];
      dense_halfstep(p, hs);
    }
  };
  // g-step from state `from` (the next column term of Y for eps_next)
  auto gstep = [&](int from, double eps, double eps_next, bool residual, bool hnext) {
    if (precise) {
      HalfStep64 hs{&Y, &X, X.H64, nullptr, G64[1 - from], nullptr, G64[from],
                    hnext ? Y.H64 : nullptr, eps, eps_next, residual, G64[from]};
      dense_halfstep64(p, hs);
    } else {
      HalfStep hs{&Y, &X, X.H, G[1 - from], G[from], hnext ? Y.H : nullptr, eps, eps_next, residual};
      hs.shift_pot = G[from];
      dense_halfstep(p, hs);
    }
  };
  auto yterm = [&](int state, double eps) {
    if (precise)
      prep_column_term64(p, Y, nullptr, G64[state], eps, Y.H64);
    else
      prep_column_term(p, Y, G[state], eps, Y.H);
  };
  auto xterm = [&](int state, double eps) {
    if (precise)
      prep_column_term64(p, X, nullptr, F64[state], eps, X.H64);
    else
      prep_column_term(p, X, F[state], eps, X.H);
  };

  // one full iteration from state `cur`; eps_next is the eps of the f-step that follows
  auto iterate = [&](double eps, double eps_next, bool residual) {
    fstep(cur, eps, residual, true);
    if (residual) SK_HIP(hipEventRecord(p->ev, st));  // the reduction wrote host_ctl
    gstep(cur, eps, eps_next, false, true);
    o.halfsteps += 2;
    cur = 1 - cur;
  };

  // annealing stages
  double eps = s.eps_start;
  bool first = true;
  while (eps > s.eps_target) {
    const double nxt = eps * s.eps_factor;
    const double eps_after = nxt > s.eps_target ? nxt : s.eps_target;
    if (s.iters_per_stage > 0) {
      if (first) yterm(cur, eps);
      first = false;
      for (int32_t k = 0; k < s.iters_per_stage; ++k) {
        const bool last = k + 1 == s.iters_per_stage;
        iterate(eps, last ? eps_after : eps, false);
        ++o.iters;
      }
    }
    ++o.stages;
    progress("solve: stage %d at eps %.4g done (%d iterations, %.3f s)", (int)o.stages, eps,
             (int)o.iters, seconds_since(t0));
    eps = nxt;
  }
  eps = s.eps_target;
  if (first) yterm(cur, eps);

  int ret = cur;
  if (s.fixed_iters > 0) {
    for (int32_t k = 0; k < s.fixed_iters; ++k) {
      iterate(eps, eps, false);
      ++o.iters;
      ++o.final_iters;
    }
    ret = cur;
    o.converged = 1;
  } else {
    const int32_t every = s.check_every > 1 ? s.check_every : 1;
    // iteration k checks the state left by iteration k-1
    for (int64_t k = 1;; ++k) {
      const int64_t prev_done = k - 1;
      const bool check = prev_done >= 1 && prev_done % every == 0;
      if (prev_done >= s.max_iters) {
        // only the residual of the final state is still needed
        fstep(cur, eps, true, false);
        ++o.halfsteps;
        double v;
        int32_t bad;
        read_reduction(p, &v, &bad);
        if (bad) fail(SINKHORN_ERR_NONFINITE, "non-finite potential during solve");
        o.row_l1 = v;
        o.history.push_back(v);
        ret = cur;
        o.converged = v <= s.tol ? 1 : 0;
        o.seconds = seconds_since(t0);
        break;
      }
      const int state = cur;
      iterate(eps, eps, check);
      if (check) {
        SK_HIP(hipEventSynchronize(p->ev));
        if (p->host_ctl->nonfinite) fail(SINKHORN_ERR_NONFINITE, "non-finite potential during solve");
        const double v = p->host_ctl->residual;
        std::vector<double>& hist = o.history;
        hist.push_back(v);
        if (hist.size() % 100 == 0)
          progress("solve: %d iterations at eps %.4g, row residual %.4g (%.3f s)", (int)o.iters, eps,
                   v, seconds_since(t0));
        const bool stalled = stall_window > 0 && (int64_t)hist.size() > stall_window &&
                             v > (1.0 - stall_rel) * hist[hist.size() - 1 - stall_window];
        if (v <= s.tol || stalled) {
          o.row_l1 = v;
          ret = state;
          o.converged = v <= s.tol ? 1 : 0;
          o.stalled = stalled && v > s.tol;
          o.seconds = seconds_since(t0);
          break;
        }
      }
      ++o.iters;
      ++o.final_iters;
    }
    if (!o.converged && !o.stalled) o.status = SINKHORN_NOT_CONVERGED;
  }
  // residuals of the returned state (the row side is known in the tol mode)
  {
    if (std::isnan(o.row_l1)) {
      yterm(ret, eps);
      reset_nonfinite(p);
      fstep(ret, eps, true, false);
      read_reduction(p, &o.row_l1, nullptr);
      ++o.halfsteps;
    }
    xterm(ret, eps);
    reset_nonfinite(p);
    gstep(ret, eps, eps, true, false);
    read_reduction(p, &o.col_l1, nullptr);
    ++o.halfsteps;
  }
  if (o.seconds == 0.0) o.seconds = seconds_since(t0);
  progress("solve: %d iterations at eps %.4g, row residual %.4g, column residual %.4g (%.3f s)",
           (int)o.iters, eps, o.row_l1, o.col_l1, o.seconds);
  if (precise) {
    narrow_f64(F64[ret], X.count, f, st);
    narrow_f64(G64[ret], Y.count, g, st);
  } else {
    copy_f32(F[ret], X.count, f, st);
    copy_f32(G[ret], Y.count, g, st);
  }
  SK_HIP(hipStreamSynchronize(st));
  o.pairs = pairs * (double)o.halfsteps;
  return o;
}

}  // namespace sk

namespace sk {
// setup.hip: the library's device memory (current, peak, largest buffer)
void device_memory(int64_t* current, int64_t* peak, int64_t* largest, bool reset);
}  // namespace sk

using namespace sk;

extern "C" {

const char* sinkhorn_strerror(int code) {
  switch (code) {
    case SINKHORN_OK: return "ok";
    case SINKHORN_NOT_CONVERGED: return "not converged (iteration cap reached)";
    case SINKHORN_ERR_INVALID_ARG: return "invalid argument";
    case SINKHORN_ERR_OOM: return "out of memory";
    case SINKHORN_ERR_HIP: return "HIP runtime error";
    case SINKHORN_ERR_CAPACITY: return "output capacity too small";
    case SINKHORN_ERR_NONFINITE: return "non-finite value";
    case SINKHORN_ERR_MASS: return "unbalanced masses";
    case SINKHORN_ERR_UNSUPPORTED: return "unsupported";
    default: return "unknown status";
  }
}

const char* sinkhorn_last_error(void) { return g_last_error.c_str(); }

int sinkhorn_mean_sqeuclid(const float* x, const float* y, int64_t n, int64_t m, int32_t d,
                           void* stream, double* mean_out) {
  return guard([&] {
    require(x && y && mean_out, "null pointer");
    require(n >= 1 && m >= 1 && d >= 1 && d <= 1024, "bad sizes");
    *mean_out = device_mean_sqeuclid(x, y, n, m, d, (hipStream_t)stream);
    return SINKHORN_OK;
  });
}

int sinkhorn_init(sinkhorn_problem** out, const float* x, const float* y, const float* a,
                  const float* b, int64_t n, int64_t m, int32_t d, double cost_scale,
                  uint32_t flags, void* stream) {
  return guard([&] {
    require(out != nullptr, "null output handle");
    *out = nullptr;
    require(x && y, "null coordinates");
    require(n >= 1 && m >= 1, "n and m must be >= 1");
    require(d >= 1 && d <= kMaxMfmaD, "d must be in [1, 63]");
    require(std::isfinite(cost_scale) && cost_scale > 0.0, "cost_scale must be finite and > 0");
    require((flags & ~(uint32_t)SINKHORN_FLAG_FP32_PAIRS) == 0, "unknown flags");
    const int64_t bytes0 = thread_alloc_current();
    sinkhorn_problem* p = new sinkhorn_problem();
    try {
      p->n = n;
      p->m = m;
      p->d = d;
      p->scale = cost_scale;
      p->flags = flags;
      p->precise = d <= 3 && !(flags & SINKHORN_FLAG_FP32_PAIRS);
      p->stream = (hipStream_t)stream;
      p->ctl = (Ctl*)dev_alloc(sizeof(Ctl));
      p->host_ctl = (Ctl*)host_alloc_coherent(sizeof(Ctl));
      SK_HIP(hipHostGetDevicePointer((void**)&p->host_ctl_dev, p->host_ctl, 0));
      {
        int dev = 0;
        SK_HIP(hipGetDevice(&dev));
        p->device = dev;
        SK_HIP(hipDeviceGetAttribute(&p->num_cu, hipDeviceAttributeMultiprocessorCount, dev));
        if (p->num_cu < 1) p->num_cu = 1;
        static_scratch_setup(dev);
      }
      p->host_tmp = (double*)host_alloc(sizeof(double) * 8);
      side_init(p, p->X, x, a, n, p->precise);
      side_init(p, p->Y, y, b, m, p->precise);
      const double sa = p->X.wsum, sb = p->Y.wsum;
      if (std::fabs(sa - sb) > 1e-5 * std::fmax(sa, sb))
        fail(SINKHORN_ERR_MASS, "sum(a) = " + std::to_string(sa) + " differs from sum(b) = " +
                                    std::to_string(sb));
      if (d > kMaxValuD) setup_mfma(p, x, y);
      p->part_cap = std::max(partial_floats_needed(p, n, p->X.padded, m),
                             partial_floats_needed(p, m, p->Y.padded, n));
      if (p->precise)
        p->part_cap = std::max(p->part_cap, std::max(dense64_partial_floats(p, n, m),
                                                     dense64_partial_floats(p, m, n)));
      p->Mpart = (float*)dev_alloc(sizeof(float) * p->part_cap);
      p->Spart = (float*)dev_alloc(sizeof(float) * p->part_cap);
      p->red_cap = std::max(row_groups(n), row_groups(m)) + 16;
      p->red_part = (double*)dev_alloc(sizeof(double) * p->red_cap);
      p->tile_flag = (int32_t*)dev_alloc(sizeof(int32_t) * p->red_cap);
      zero_i32(p->tile_flag, (int32_t)p->red_cap, p->stream);
      reset_nonfinite(p);
      for (int k = 0; k < 2; ++k) {
        p->fbuf[k] = (float*)dev_alloc(sizeof(float) * n);
        p->gbuf[k] = (float*)dev_alloc(sizeof(float) * m);
        if (p->precise) {
          p->fbuf64[k] = (double*)dev_alloc(sizeof(double) * n);
          p->gbuf64[k] = (double*)dev_alloc(sizeof(double) * m);
        }
      }
      if (p->precise) p->shift64 = (double*)dev_alloc(sizeof(double) * std::max(n, m));
      SK_HIP(hipEventCreateWithFlags(&p->ev, hipEventDisableTiming));
      SK_HIP(hipStreamSynchronize(p->stream));
      p->workspace_bytes = thread_alloc_current() - bytes0;
    } catch (...) {
      problem_free(p);
      throw;
    }
    *out = p;
    return SINKHORN_OK;
  });
}

int sinkhorn_destroy(sinkhorn_problem* p) {
  return guard([&] {
    problem_free(p);
    return SINKHORN_OK;
  });
}

int sinkhorn_device_memory(int64_t* current_bytes, int64_t* peak_bytes, int64_t* largest_bytes,
                           int32_t reset) {
  return guard([&] {
    device_memory(current_bytes, peak_bytes, largest_bytes, reset != 0);
    return SINKHORN_OK;
  });
}

int sinkhorn_problem_info(const sinkhorn_problem* p, int64_t* n, int64_t* m, int32_t* d,
                          double* cost_scale) {
  return guard([&] {
    require(p != nullptr, "null handle");
    if (n) *n = p->n;
    if (m) *m = p->m;
    if (d) *d = p->d;
    if (cost_scale) *cost_scale = p->scale;
    return SINKHORN_OK;
  });
}

int sinkhorn_halfstep_f(sinkhorn_problem* p, double eps, const float* g, float* f_out,
                        const float* f_prev, double* row_l1) {
  return guard([&] {
    halfstep(p, true, eps, g, f_out, f_prev, row_l1);
    return SINKHORN_OK;
  });
}

int sinkhorn_halfstep_g(sinkhorn_problem* p, double eps, const float* f, float* g_out,
                        const float* g_prev, double* col_l1) {
  return guard([&] {
    halfstep(p, false, eps, f, g_out, g_prev, col_l1);
    return SINKHORN_OK;
  });
}

int sinkhorn_marginal_residual(sinkhorn_problem* p, double eps, const float* f, const float* g,
                               double* row_l1, double* col_l1) {
  return guard([&] {
    require(p && f && g, "null pointer");
    double r = NAN, c = NAN;
    const auto t0 = std::chrono::steady_clock::now();
    halfstep(p, true, eps, g, p->fbuf[0], f, &r);
    progress("marginal residual: row %.6g (%.3f s)", r, seconds_since(t0));
    halfstep(p, false, eps, f, p->gbuf[0], g, &c);
    progress("marginal residual: column %.6g (%.3f s)", c, seconds_since(t0));
    if (row_l1) *row_l1 = r;
    if (col_l1) *col_l1 = c;
    return SINKHORN_OK;
  });
}

int sinkhorn_solve(sinkhorn_problem* p, const sinkhorn_schedule* sc, float* f, float* g,
                   sinkhorn_report* rep) {
  return guard([&] {
    require(p && sc && f && g, "null pointer");
    float* F[2] = {p->fbuf[0], p->fbuf[1]};
    float* G[2] = {p->gbuf[0], p->gbuf[1]};
    if (rep) require(rep->history_cap >= 0 && (rep->history_cap == 0 || rep->history),
                     "report history buffer");
    const int64_t base = thread_alloc_current();
    thread_alloc_mark();
    const SolveOut o = dense_solve(p, p->X, p->Y, f, g, F, G, *sc, 0, 0.0);
    if (rep) {
      rep->halfsteps = o.halfsteps;
      rep->iters = o.iters;
      rep->final_iters = o.final_iters;
      rep->pairs_evaluated = o.pairs;
      rep->row_l1 = o.row_l1;
      rep->col_l1 = o.col_l1;
      rep->seconds = o.seconds;
      rep->stages = o.stages;
      rep->converged = o.converged;
      rep->seconds_per_halfstep = o.halfsteps > 0 ? o.seconds / (double)o.halfsteps : 0.0;
      rep->workspace_bytes = p->workspace_bytes;
      rep->peak_extra_bytes = thread_alloc_peak() - base;
      const int64_t len = (int64_t)o.history.size();
      rep->history_len = (int32_t)len;
      const int64_t keep = std::min<int64_t>(len, rep->history_cap);
      for (int64_t k = 0; k < keep; ++k) rep->history[k] = o.history[len - keep + k];
    }
    return o.status;
  });
}

}  // extern "C"

extern "C" {

int sinkhorn_profile_enable(sinkhorn_problem* p, int32_t kinds) {
  return guard([&] {
    require(p != nullptr, "null handle");
    p->prof = kinds;
    return SINKHORN_OK;
  });
}

int sinkhorn_profile_read(sinkhorn_problem* p, double* kernel_ms, int64_t* launches,
                          double* pairs) {
  return guard([&] {
    require(p != nullptr, "null handle");
    SK_HIP(hipStreamSynchronize(p->stream));
    double total = 0.0;
    for (size_t k = 0; k < p->prof_used; ++k) {
      float ms = 0.0f;
      SK_HIP(hipEventElapsedTime(&ms, p->prof_ev[2 * k], p->prof_ev[2 * k + 1]));
      total += (double)ms;
    }
    if (kernel_ms) *kernel_ms = total;
    if (launches) *launches = (int64_t)p->prof_used;
    if (pairs) *pairs = p->prof_pairs;
    p->prof_used = 0;
    p->prof_pairs = 0.0;
    return SINKHORN_OK;
  });
}

}  // extern "C"
