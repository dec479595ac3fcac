"""Host-side checks of the C ABI: the library loads without a GPU and exports
every entry point that include/sinkhorn.h declares, with the binding's table
matching the header."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sinkhorn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sinkhorn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_path():
    names = _declared()
    for required in ("sinkhorn_init", "sinkhorn_halfstep_f", "sinkhorn_halfstep_g", "sinkhorn_solve",
                     "sinkhorn_marginal_residual", "sinkhorn_materialize_rows", "sinkhorn_block_screen"):
        assert required in names


def test_library_exports_every_declared_symbol():
    import log_domain_sinkhorn_amd as sk

    if not os.path.exists(sk.LIB_PATH):
        pytest.fail("libsinkhorn.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(sk.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert sorted(sk.EXPORTED) == _declared()


def test_status_strings_without_a_device():
    import log_domain_sinkhorn_amd as sk

    L = sk.lib()
    assert L.sinkhorn_strerror(0) == b"ok"
    assert L.sinkhorn_strerror(sk.ERR_CAPACITY) == b"output capacity too small"
    assert L.sinkhorn_strerror(12345) == b"unknown status"


def test_invalid_arguments_are_rejected_before_any_device_work():
    import log_domain_sinkhorn_amd as sk

    L = sk.lib()
    h = ctypes.c_void_p()
    # null coordinates, bad sizes, bad scale: rejected on the host
    assert L.sinkhorn_init(ctypes.byref(h), None, None, None, None, 10, 10, 3, 1.0, 0, None) == sk.ERR_INVALID_ARG
    fake = ctypes.c_void_p(16)
    assert L.sinkhorn_init(ctypes.byref(h), fake, fake, None, None, 0, 10, 3, 1.0, 0, None) == sk.ERR_INVALID_ARG
    assert L.sinkhorn_init(ctypes.byref(h), fake, fake, None, None, 10, 10, 0, 1.0, 0, None) == sk.ERR_INVALID_ARG
    assert L.sinkhorn_init(ctypes.byref(h), fake, fake, None, None, 10, 10, 3, float("nan"), 0, None) == sk.ERR_INVALID_ARG
    assert L.sinkhorn_init(ctypes.byref(h), fake, fake, None, None, 10, 10, 3, -1.0, 0, None) == sk.ERR_INVALID_ARG
    assert b"cost_scale" in L.sinkhorn_last_error()
    # unknown flag bits
    assert L.sinkhorn_init(ctypes.byref(h), fake, fake, None, None, 10, 10, 3, 1.0, 2, None) == sk.ERR_INVALID_ARG
    assert b"flags" in L.sinkhorn_last_error()
    # null handle
    assert L.sinkhorn_halfstep_f(None, 0.1, fake, fake, None, None) == sk.ERR_INVALID_ARG
    assert L.sinkhorn_solve(None, None, None, None, None) == sk.ERR_INVALID_ARG
    assert L.sinkhorn_destroy(None) == sk.OK
    assert L.sinkhorn_problem_info(None, None, None, None, None) == sk.ERR_INVALID_ARG


def test_device_memory_needs_no_device():
    import log_domain_sinkhorn_amd as sk

    cur, peak, big = sk.device_memory(reset=True)
    assert cur == 0 and peak == 0 and big == 0
    assert sk.lib().sinkhorn_device_memory(None, None, None, 0) == sk.OK
