"""Python binding of the MI355X online log-domain Sinkhorn library.

Thin ctypes wrappers around the C ABI declared in ``include/sinkhorn.h``: the
functions here only marshal arguments (torch device tensors -> raw pointers,
the current HIP stream -> ``void*``) and turn status codes into exceptions.
Every step of the computation runs in the HIP kernels of ``libsinkhorn.so``.
PyTorch provides device memory and streams only.

The library must have been built (``python -m log_domain_sinkhorn_amd.build``);
every entry point raises ``ImportError`` without it: there is no CPU or
PyTorch fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch  # loads the HIP runtime the library links against

__all__ = [
    "SinkhornError",
    "Schedule",
    "MultiscaleParams",
    "Problem",
    "mean_sqeuclid",
    "morton_order",
    "lib",
    "LIB_PATH",
    "OK",
    "NOT_CONVERGED",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsinkhorn.so")

OK = 0
NOT_CONVERGED = 1
ERR_INVALID_ARG = -1
ERR_OOM = -2
ERR_HIP = -3
ERR_CAPACITY = -4
ERR_NONFINITE = -5
ERR_MASS = -6
ERR_UNSUPPORTED = -7

# kernel kinds for Problem.profile_enable (SINKHORN_PROF_* in sinkhorn.h)
PROF_DENSE = 1
PROF_SPARSE = 2
PROF_MATERIALIZE = 4
PROF_BARY = 8
PROF_DENSE_EXACT = 16

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f64 = ctypes.c_double


class _ScheduleC(ctypes.Structure):
    _fields_ = [
        ("eps_start", _f64),
        ("eps_target", _f64),
        ("eps_factor", _f64),
        ("iters_per_stage", _i32),
        ("fixed_iters", _i32),
        ("tol", _f64),
        ("max_iters", _i32),
        ("check_every", _i32),
    ]


class _ReportC(ctypes.Structure):
    _fields_ = [
        ("halfsteps", _i64),
        ("iters", _i64),
        ("final_iters", _i64),
        ("pairs_evaluated", _f64),
        ("row_l1", _f64),
        ("col_l1", _f64),
        ("seconds", _f64),
        ("stages", _i32),
        ("converged", _i32),
        ("history", ctypes.POINTER(_f64)),
        ("history_cap", _i32),
        ("history_len", _i32),
        ("seconds_per_halfstep", _f64),
        ("workspace_bytes", _i64),
        ("peak_extra_bytes", _i64),
    ]


class _MultiscaleParamsC(ctypes.Structure):
    _fields_ = [
        ("B", _i32),
        ("p_bits", _i32),
        ("eps", _f64),
        ("tol", _f64),
        ("delta_scale", _f64),
        ("coarse_eps_start", _f64),
        ("coarse_factor", _f64),
        ("coarse_iters_per_stage", _i32),
        ("coarse_tol", _f64),
        ("coarse_max", _i32),
        ("stall_window", _i32),
        ("stall_rel", _f64),
        ("max_fine", _i32),
        ("verify", _i32),
        ("adaptive", _i32),
        ("check_every", _i32),
        ("check_samples", _i32),
        ("check_samples_max", _i32),
        ("sample_seed", ctypes.c_uint64),
        ("warm_start", _i32),
    ]


class _MultiscaleReportC(ctypes.Structure):
    _fields_ = [
        ("coarse_iters", _i64),
        ("fine_updates", _i64),
        ("ncells_x", _i64),
        ("ncells_y", _i64),
        ("last_tiles", _i64),
        ("pairs_evaluated", _f64),
        ("R_A_row", _f64),
        ("R_A_col", _f64),
        ("omega", _f64),
        ("seconds_total", _f64),
        ("seconds_sort", _f64),
        ("seconds_coarse", _f64),
        ("seconds_lift", _f64),
        ("seconds_fine", _f64),
        ("certified", _i32),
        ("last_candidates", _i64),
        ("accepted_by_sample", _i32),
        ("checks", _i64),
        ("last_check_samples", _i64),
        ("last_check", _f64 * 4),
        ("peak_extra_bytes", _i64),
    ]


# name -> argtypes (every entry point declared in include/sinkhorn.h)
_SIGS = {
    "sinkhorn_strerror": ([_i32], ctypes.c_char_p),
    "sinkhorn_last_error": ([], ctypes.c_char_p),
    "sinkhorn_mean_sqeuclid": ([_p, _p, _i64, _i64, _i32, _p, _p], _i32),
    "sinkhorn_init": ([_p, _p, _p, _p, _p, _i64, _i64, _i32, _f64, ctypes.c_uint32, _p], _i32),
    "sinkhorn_destroy": ([_p], _i32),
    "sinkhorn_problem_info": ([_p, _p, _p, _p, _p], _i32),
    "sinkhorn_device_memory": ([_p, _p, _p, _i32], _i32),
    "sinkhorn_halfstep_f": ([_p, _f64, _p, _p, _p, _p], _i32),
    "sinkhorn_halfstep_g": ([_p, _f64, _p, _p, _p, _p], _i32),
    "sinkhorn_marginal_residual": ([_p, _f64, _p, _p, _p, _p], _i32),
    "sinkhorn_solve": ([_p, _p, _p, _p, _p], _i32),
    "sinkhorn_materialize_rows": ([_p, _f64, _p, _p, _p, _i64, _p, _p], _i32),
    "sinkhorn_materialize_rows_noalloc": ([_p, _f64, _p, _p, _p, _i64, _p, _p], _i32),
    "sinkhorn_min_row": ([_p, _f64, _p, _p, _p], _i32),
    "sinkhorn_morton_order": ([_p, _p, _i64, _i64, _i32, _p, _p, _p, _p, _p], _i32),
    "sinkhorn_morton_sort": ([_p, _i32, _p, _p], _i32),
    "sinkhorn_block_screen": ([_p, _f64, _p, _p, _i32, _f64, _i32, _p, _p, _i64, _p], _i32),
    "sinkhorn_verify_tiles": ([_p, _f64, _p, _p, _i32, _f64, _p, _p, _p, _p, _p, _p, _p], _i32),
    "sinkhorn_sparse_halfstep_f": ([_p, _f64, _p, _i32, _p, _p, _p, _p, _p], _i32),
    "sinkhorn_sparse_halfstep_g": ([_p, _f64, _p, _i32, _p, _p, _p, _p, _p], _i32),
    "sinkhorn_barycentric": ([_p, _f64, _p, _p, _p, _p], _i32),
    "sinkhorn_sparsify": ([_p, _f64, _p, _p, ctypes.c_float, _i64, _p, _p, _p, _i64, _p], _i32),
    "sinkhorn_sparse_barycentric": ([_p, _f64, _p, _p, _i32, _p, _p, _p, _p], _i32),
    "sinkhorn_solve_multiscale": ([_p, _p, _p, _p, _p], _i32),
    "sinkhorn_sample_indices": ([_i64, _i32, ctypes.c_uint64, ctypes.c_uint64, _p, _p], _i32),
    "sinkhorn_sampled_residual": ([_p, _f64, _p, _p, _i32, _i32, ctypes.c_uint64, _p, _p], _i32),
    "sinkhorn_profile_enable": ([_p, _i32], _i32),
    "sinkhorn_profile_read": ([_p, _p, _p, _p], _i32),
    "sinkhorn_probe_issue_rate": ([_i32, _i32, _p, _p, _p, _p], _i32),
}

EXPORTED = tuple(_SIGS)

_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises ImportError if it was not built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing; build it with `python -m log_domain_sinkhorn_amd.build`"
            )
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _LIB = handle
    return _LIB


class SinkhornError(RuntimeError):
    def __init__(self, code: int, where: str):
        L = lib()
        detail = L.sinkhorn_last_error().decode()
        name = L.sinkhorn_strerror(code).decode()
        super().__init__(f"{where}: {name} ({code}){': ' + detail if detail else ''}")
        self.code = code


def _check(code: int, where: str) -> int:
    if code < 0:
        raise SinkhornError(code, where)
    return code


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, dtype, name: str, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


@dataclass
class Schedule:
    eps_start: float
    eps_target: float
    eps_factor: float = 0.5
    iters_per_stage: int = 10
    fixed_iters: int = 0
    tol: float = 1e-3
    max_iters: int = 10000
    check_every: int = 1

    def _c(self) -> _ScheduleC:
        return _ScheduleC(self.eps_start, self.eps_target, self.eps_factor, self.iters_per_stage,
                          self.fixed_iters, self.tol, self.max_iters, self.check_every)


@dataclass
class MultiscaleParams:
    B: int = 128
    p_bits: int = 0
    eps: float = 1e-4
    tol: float = 1e-2
    delta_scale: float = 1e-3
    coarse_eps_start: float = 1.0
    coarse_factor: float = 0.5
    coarse_iters_per_stage: int = 10
    coarse_tol: float = 1e-3
    coarse_max: int = 2048
    stall_window: int = 10
    stall_rel: float = 0.01
    max_fine: int = 8192
    verify: bool = False
    adaptive: bool = False
    check_every: int = 128
    check_samples: int = 1024
    check_samples_max: int = 8192
    sample_seed: int = 0
    warm_start: bool = False

    def _c(self) -> _MultiscaleParamsC:
        return _MultiscaleParamsC(self.B, self.p_bits, self.eps, self.tol, self.delta_scale,
                                  self.coarse_eps_start, self.coarse_factor,
                                  self.coarse_iters_per_stage, self.coarse_tol, self.coarse_max,
                                  self.stall_window, self.stall_rel, self.max_fine,
                                  int(bool(self.verify)), int(bool(self.adaptive)), self.check_every,
                                  self.check_samples, self.check_samples_max, self.sample_seed,
                                  int(bool(self.warm_start)))


def _struct_dict(s) -> dict:
    out = {}
    for name, _ in s._fields_:
        v = getattr(s, name)
        out[name] = list(v) if isinstance(v, ctypes.Array) else v
    return out


def sample_indices(count: int, k: int, seed: int, stream_id: int, device="cuda:0") -> torch.Tensor:
    """The sampled checks' indices as an int32 device tensor."""
    out = torch.empty(max(1, k), dtype=torch.int32, device=device)
    _check(lib().sinkhorn_sample_indices(int(count), int(k), int(seed), int(stream_id),
                                         _stream(torch.device(device)), _ptr(out)), "sample_indices")
    return out[:k]


def mean_sqeuclid(x: torch.Tensor, y: torch.Tensor) -> float:
    """Unweighted mean of ||x_i - y_j||^2 over all pairs (device fp64)."""
    _dev(x, torch.float32, "x")
    _dev(y, torch.float32, "y")
    out = _f64()
    _check(lib().sinkhorn_mean_sqeuclid(_ptr(x), _ptr(y), x.shape[0], y.shape[0], x.shape[1],
                                        _stream(x.device), ctypes.byref(out)), "mean_sqeuclid")
    return out.value


def morton_order(x: torch.Tensor, y: torch.Tensor):
    """(codes_x, perm_x, codes_y, perm_y): sorted Morton codes (int64 tensors
    holding the uint64 bits) and the original index of each sorted point."""
    _dev(x, torch.float32, "x")
    _dev(y, torch.float32, "y")
    n, d = x.shape
    m = y.shape[0]
    cx = torch.empty(n, dtype=torch.int64, device=x.device)
    cy = torch.empty(m, dtype=torch.int64, device=x.device)
    px = torch.empty(n, dtype=torch.int32, device=x.device)
    py = torch.empty(m, dtype=torch.int32, device=x.device)
    _check(lib().sinkhorn_morton_order(_ptr(x), _ptr(y), n, m, d, _stream(x.device), _ptr(cx),
                                       _ptr(px), _ptr(cy), _ptr(py)), "morton_order")
    return cx, px, cy, py


(PROBE_FMA_F32, PROBE_EXP_F32, PROBE_FMA_F64, PROBE_PAIR_F32, PROBE_PAIR_F32_NOEXP, PROBE_PAIR_F64,
 PROBE_SUB_F32, PROBE_FMAC_F32, PROBE_ADD_F64, PROBE_CVT_F32_F64, PROBE_PAIR_TILE_F32,
 PROBE_PAIR_SPLIT_F32, PROBE_PAIR_TILE_MFMA) = range(13)
FLAG_FP32_PAIRS = 1


def probe_issue_rate(kind: int, iters: int = 20000, device="cuda:0"):
    """(lane-instructions/s, pairs/s, kernel ms) of an issue-rate probe kernel."""
    rate, pairs, ms = _f64(), _f64(), _f64()
    with torch.cuda.device(device):
        _check(lib().sinkhorn_probe_issue_rate(int(kind), int(iters), _stream(device), ctypes.byref(rate),
                                               ctypes.byref(pairs), ctypes.byref(ms)), "probe_issue_rate")
    return rate.value, pairs.value, ms.value


def device_memory(reset: bool = False):
    """(current, peak, largest) device bytes the library holds, over all
    handles (``sinkhorn_device_memory``); reset=True then starts a new peak."""
    cur, peak, big = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().sinkhorn_device_memory(ctypes.byref(cur), ctypes.byref(peak), ctypes.byref(big),
                                        int(bool(reset))), "device_memory")
    return cur.value, peak.value, big.value


class Problem:
    """A problem handle (``sinkhorn_init``) over device clouds x [n,d], y [m,d]."""

    def __init__(self, x, y, a=None, b=None, cost_scale: float = 1.0, flags: int = 0):
        _dev(x, torch.float32, "x")
        _dev(y, torch.float32, "y")
        if x.dim() != 2 or y.dim() != 2 or x.shape[1] != y.shape[1]:
            raise ValueError("x and y must be [n,d] and [m,d]")
        self.n, self.d = x.shape
        self.m = y.shape[0]
        if a is not None:
            _dev(a, torch.float32, "a", (self.n,))
        if b is not None:
            _dev(b, torch.float32, "b", (self.m,))
        self.device = x.device
        self.cost_scale = float(cost_scale)
        self.flags = int(flags)
        h = ctypes.c_void_p()
        _check(lib().sinkhorn_init(ctypes.byref(h), _ptr(x), _ptr(y), _ptr(a), _ptr(b), self.n,
                                   self.m, self.d, self.cost_scale, self.flags, _stream(self.device)),
               "init")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            lib().sinkhorn_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def info(self):
        """(n, m, d, cost_scale) as the handle holds them (``sinkhorn_problem_info``)."""
        n, m, d, sc = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32(), ctypes.c_double()
        _check(lib().sinkhorn_problem_info(self._h, ctypes.byref(n), ctypes.byref(m), ctypes.byref(d),
                                           ctypes.byref(sc)), "problem_info")
        return n.value, m.value, d.value, sc.value

    def _pot(self, t, k, name):
        return _dev(t, torch.float32, name, (k,))

    def _new(self, k):
        return torch.empty(k, dtype=torch.float32, device=self.device)

    def halfstep_f(self, eps, g, out=None, f_prev=None):
        """f = f-step(g). Returns (f, R_row of (f_prev, g) or None)."""
        self._pot(g, self.m, "g")
        out = self._new(self.n) if out is None else self._pot(out, self.n, "out")
        res = _f64() if f_prev is not None else None
        if f_prev is not None:
            self._pot(f_prev, self.n, "f_prev")
        _check(lib().sinkhorn_halfstep_f(self._h, float(eps), _ptr(g), _ptr(out), _ptr(f_prev),
                                         ctypes.byref(res) if res is not None else None), "halfstep_f")
        return out, (res.value if res is not None else None)

    def halfstep_g(self, eps, f, out=None, g_prev=None):
        """g = g-step(f). Returns (g, R_col of (f, g_prev) or None)."""
        self._pot(f, self.n, "f")
        out = self._new(self.m) if out is None else self._pot(out, self.m, "out")
        res = _f64() if g_prev is not None else None
        if g_prev is not None:
            self._pot(g_prev, self.m, "g_prev")
        _check(lib().sinkhorn_halfstep_g(self._h, float(eps), _ptr(f), _ptr(out), _ptr(g_prev),
                                         ctypes.byref(res) if res is not None else None), "halfstep_g")
        return out, (res.value if res is not None else None)

    def marginal_residual(self, eps, f, g):
        self._pot(f, self.n, "f")
        self._pot(g, self.m, "g")
        r, c = _f64(), _f64()
        _check(lib().sinkhorn_marginal_residual(self._h, float(eps), _ptr(f), _ptr(g),
                                                ctypes.byref(r), ctypes.byref(c)), "marginal_residual")
        return r.value, c.value

    def solve(self, sched: Schedule, f=None, g=None, history: int = 256):
        """Annealed dense solve. Returns (f, g, report dict); report['status']
        is OK or NOT_CONVERGED; report['history'] holds the row residuals of
        the last `history` checks at eps_target."""
        f = torch.zeros(self.n, dtype=torch.float32, device=self.device) if f is None else self._pot(f, self.n, "f")
        g = torch.zeros(self.m, dtype=torch.float32, device=self.device) if g is None else self._pot(g, self.m, "g")
        sc = sched._c()
        rep = _ReportC()
        buf = (_f64 * max(1, history))()
        rep.history = ctypes.cast(buf, ctypes.POINTER(_f64))
        rep.history_cap = int(history)
        st = _check(lib().sinkhorn_solve(self._h, ctypes.byref(sc), _ptr(f), _ptr(g), ctypes.byref(rep)),
                    "solve")
        out = _struct_dict(rep)
        out["history"] = list(buf[:min(rep.history_len, history)])
        out["status"] = st
        return f, g, out

    def materialize_rows(self, eps, f, g, rows, T=None, row_max=None):
        """T[r] = plan row rows[r] (fp32 [k, m]); row_max optional [k]."""
        self._pot(f, self.n, "f")
        self._pot(g, self.m, "g")
        _dev(rows, torch.int64, "rows")
        k = rows.shape[0]
        T = torch.empty((k, self.m), dtype=torch.float32, device=self.device) if T is None else \
            _dev(T, torch.float32, "T", (k, self.m))
        if row_max is not None:
            _dev(row_max, torch.float32, "row_max", (k,))
        _check(lib().sinkhorn_materialize_rows(self._h, float(eps), _ptr(f), _ptr(g), _ptr(rows), k,
                                               _ptr(T), _ptr(row_max)), "materialize_rows")
        return T, row_max

    def materialize_rows_noalloc(self, eps, f, g, rows, T, row_max=None):
        """materialize_rows into caller buffers with no allocation in the call
        (T [k, m] fp32 is required; k <= 4096, m <= 2^21 when d <= 8)."""
        self._pot(f, self.n, "f")
        self._pot(g, self.m, "g")
        _dev(rows, torch.int64, "rows")
        k = rows.shape[0]
        _dev(T, torch.float32, "T", (k, self.m))
        if row_max is not None:
            _dev(row_max, torch.float32, "row_max", (k,))
        _check(lib().sinkhorn_materialize_rows_noalloc(self._h, float(eps), _ptr(f), _ptr(g), _ptr(rows),
                                                       k, _ptr(T), _ptr(row_max)),
               "materialize_rows_noalloc")
        return T, row_max

    def min_row(self, eps, f, g) -> float:
        self._pot(f, self.n, "f")
        self._pot(g, self.m, "g")
        out = ctypes.c_float()
        _check(lib().sinkhorn_min_row(self._h, float(eps), _ptr(f), _ptr(g), ctypes.byref(out)),
               "min_row")
        return out.value

    def morton_sort(self, side: int):
        """(codes int64 holding the uint64 bits, perm int32) of side 0 (x) or 1 (y)."""
        count = self.n if side == 0 else self.m
        codes = torch.empty(count, dtype=torch.int64, device=self.device)
        perm = torch.empty(count, dtype=torch.int32, device=self.device)
        _check(lib().sinkhorn_morton_sort(self._h, int(side), _ptr(perm), _ptr(codes)), "morton_sort")
        return codes, perm

    def block_screen(self, eps, f, g, B, delta_rel, transpose=False, cap=None):
        """Admitted tiles as (ptr int64, idx int32) device tensors."""
        self._pot(f, self.n, "f")
        self._pot(g, self.m, "g")
        nb = (self.m + B - 1) // B if transpose else (self.n + B - 1) // B
        ptr = torch.empty(nb + 1, dtype=torch.int64, device=self.device)
        nnz = _i64()
        if cap is None:
            code = lib().sinkhorn_block_screen(self._h, float(eps), _ptr(f), _ptr(g), B,
                                               float(delta_rel), int(transpose), _ptr(ptr), None, 0,
                                               ctypes.byref(nnz))
            if code not in (OK, ERR_CAPACITY):
                _check(code, "block_screen")
            cap = nnz.value
        idx = torch.empty(max(1, cap), dtype=torch.int32, device=self.device)
        _check(lib().sinkhorn_block_screen(self._h, float(eps), _ptr(f), _ptr(g), B, float(delta_rel),
                                           int(transpose), _ptr(ptr), _ptr(idx), cap,
                                           ctypes.byref(nnz)), "block_screen")
        return ptr, idx[: nnz.value]

    def verify_tiles(self, eps, f, g, B, delta_rel, ptr, idx):
        """Verified tiles of a row-major candidate list: (vptr, vidx, tptr,
        tidx) device tensors, the kept tiles row-major and column-major."""
        self._pot(f, self.n, "f")
        self._pot(g, self.m, "g")
        nb = (self.n + B - 1) // B
        mb = (self.m + B - 1) // B
        _dev(ptr, torch.int64, "ptr", (nb + 1,))
        nnz = int(idx.shape[0])
        if nnz:
            _dev(idx, torch.int32, "idx")
        vptr = torch.empty(nb + 1, dtype=torch.int64, device=self.device)
        tptr = torch.empty(mb + 1, dtype=torch.int64, device=self.device)
        vidx = torch.empty(max(1, nnz), dtype=torch.int32, device=self.device)
        tidx = torch.empty(max(1, nnz), dtype=torch.int32, device=self.device)
        kept = _i64()
        _check(lib().sinkhorn_verify_tiles(self._h, float(eps), _ptr(f), _ptr(g), int(B),
                                           float(delta_rel), _ptr(ptr), _ptr(idx) if nnz else None,
                                           _ptr(vptr), _ptr(vidx), _ptr(tptr), _ptr(tidx),
                                           ctypes.byref(kept)), "verify_tiles")
        k = kept.value
        return vptr, vidx[:k], tptr, tidx[:k]

    def sparse_halfstep_f(self, eps, g, B, ptr, idx, out=None, f_prev=None):
        self._pot(g, self.m, "g")
        out = self._new(self.n) if out is None else self._pot(out, self.n, "out")
        res = _f64() if f_prev is not None else None
        _check(lib().sinkhorn_sparse_halfstep_f(self._h, float(eps), _ptr(g), B, _ptr(ptr), _ptr(idx),
                                                _ptr(out), _ptr(f_prev),
                                                ctypes.byref(res) if res is not None else None),
               "sparse_halfstep_f")
        return out, (res.value if res is not None else None)

    def sparse_halfstep_g(self, eps, f, B, ptr, idx, out=None, g_prev=None):
        self._pot(f, self.n, "f")
        out = self._new(self.m) if out is None else self._pot(out, self.m, "out")
        res = _f64() if g_prev is not None else None
        _check(lib().sinkhorn_sparse_halfstep_g(self._h, float(eps), _ptr(f), B, _ptr(ptr), _ptr(idx),
                                                _ptr(out), _ptr(g_prev),
                                                ctypes.byref(res) if res is not None else None),
               "sparse_halfstep_g")
        return out, (res.value if res is not None else None)

    def sparsify(self, eps, f, g, threshold: float, batch: int = 1024, cap=None):
        """(row_ptr, col, val): the plan entries >= threshold as CSR (int64,
        int32, fp32 device tensors). With cap=None the count is taken first
        (row_ptr only), then the entries are written into buffers of that size."""
        self._pot(f, self.n, "f")
        self._pot(g, self.m, "g")
        row_ptr = torch.empty(self.n + 1, dtype=torch.int64, device=self.device)
        nnz = _i64()
        if cap is None:
            _check(lib().sinkhorn_sparsify(self._h, float(eps), _ptr(f), _ptr(g), float(threshold), int(batch),
                                           _ptr(row_ptr), None, None, 0, ctypes.byref(nnz)), "sparsify")
            cap = nnz.value
        col = torch.empty(max(1, cap), dtype=torch.int32, device=self.device)
        val = torch.empty(max(1, cap), dtype=torch.float32, device=self.device)
        st = lib().sinkhorn_sparsify(self._h, float(eps), _ptr(f), _ptr(g), float(threshold), int(batch),
                                     _ptr(row_ptr), _ptr(col), _ptr(val), int(cap), ctypes.byref(nnz))
        if st != OK:
            raise SinkhornError(st, "sparsify")
        k = nnz.value
        return row_ptr, col[:k], val[:k]

    def barycentric(self, eps, g, f_hint=None, T=None, grad=None, want_T=True, want_grad=True):
        """(T, grad): barycentric projection of the plan rows and the source
        gradient 2 s a_i (x_i - T_i), [n, d] fp32 each (None when not wanted).
        f_hint, the f-step potential of g, only speeds up the loop."""
        self._pot(g, self.m, "g")
        if f_hint is not None:
            self._pot(f_hint, self.n, "f_hint")
        T, grad = self._bary_out(T, grad, want_T, want_grad)
        _check(lib().sinkhorn_barycentric(self._h, float(eps), _ptr(g), _ptr(f_hint), _ptr(T), _ptr(grad)),
               "barycentric")
        return T, grad

    def sparse_barycentric(self, eps, g, B, ptr, idx, f_hint=None, T=None, grad=None, want_T=True,
                           want_grad=True):
        """The projection and gradient restricted to the admitted tiles."""
        self._pot(g, self.m, "g")
        if f_hint is not None:
            self._pot(f_hint, self.n, "f_hint")
        T, grad = self._bary_out(T, grad, want_T, want_grad)
        _check(lib().sinkhorn_sparse_barycentric(self._h, float(eps), _ptr(g), _ptr(f_hint), int(B), _ptr(ptr),
                                                 _ptr(idx), _ptr(T), _ptr(grad)), "sparse_barycentric")
        return T, grad

    def _bary_out(self, T, grad, want_T, want_grad):
        shape = (self.n, self.d)
        if T is None and want_T:
            T = torch.empty(shape, dtype=torch.float32, device=self.device)
        elif T is not None:
            _dev(T, torch.float32, "T", shape)
        if grad is None and want_grad:
            grad = torch.empty(shape, dtype=torch.float32, device=self.device)
        elif grad is not None:
            _dev(grad, torch.float32, "grad", shape)
        return T, grad

    def profile_enable(self, kinds: int = PROF_DENSE):
        """Bracket every later launch of the selected kernel kinds (PROF_*
        bits; 0 stops) with HIP events on the library's stream."""
        _check(lib().sinkhorn_profile_enable(self._h, int(kinds)), "profile_enable")

    def profile_read(self):
        """(kernel_ms, launches, pairs) recorded since the last read (syncs)."""
        ms, n, pairs = _f64(), _i64(), _f64()
        _check(lib().sinkhorn_profile_read(self._h, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(pairs)),
               "profile_read")
        return ms.value, n.value, pairs.value

    def sampled_residual(self, eps, f, g, side=0, k=1024, seed=0):
        """(estimate, standard error) of one side's L1 marginal residual from k
        drawn rows (side 0: x, side 1: y)."""
        self._pot(f, self.n, "f")
        self._pot(g, self.m, "g")
        est, se = _f64(), _f64()
        _check(lib().sinkhorn_sampled_residual(self._h, float(eps), _ptr(f), _ptr(g), int(side), int(k),
                                               int(seed), ctypes.byref(est), ctypes.byref(se)),
               "sampled_residual")
        return est.value, se.value

    def solve_multiscale(self, prm: MultiscaleParams, f=None, g=None):
        f = self._new(self.n) if f is None else self._pot(f, self.n, "f")
        g = self._new(self.m) if g is None else self._pot(g, self.m, "g")
        c = prm._c()
        rep = _MultiscaleReportC()
        st = _check(lib().sinkhorn_solve_multiscale(self._h, ctypes.byref(c), _ptr(f), _ptr(g),
                                                    ctypes.byref(rep)), "solve_multiscale")
        out = _struct_dict(rep)
        out["status"] = st
        return f, g, out

