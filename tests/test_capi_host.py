"""The C ABI without a GPU: the library loads, exports every symbol the public
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "schnet_continuous_filter_amd", "libschnet_mi355x.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        sys.path.insert(0, ROOT)
        import __graft_entry__
        __graft_entry__.build()
    from schnet_continuous_filter_amd import _lib
    return _lib


def test_exports_every_declared_symbol(lib):
    names = lib.declared_functions()
    assert len(names) >= 14
    raw = ctypes.CDLL(LIB)
    missing = [n for n in names if not hasattr(raw, n)]
    assert not missing, missing
    # the header declares the three calls the path is built around
    for n in ("sn_build_neighbors", "sn_energy_forces", "sn_md_step"):
        assert n in names


def test_status_strings(lib):
    for s in range(7):
        assert lib.status_string(s) and lib.status_string(s) != "unknown status"
    assert lib.status_string(99) == "unknown status"


def test_weight_count_matches_generator(lib):
    from gen.systems import n_model_weights
    for (nt, D, Dr, T, H) in [(1, 64, 32, 2, 32), (20, 128, 50, 3, 64), (4, 128, 64, 3, 64)]:
        d = lib.make_desc(nt, D, Dr, T, H, 0.0, 10.0, 10.0)
        assert lib.sn_model_weight_count(d) == n_model_weights(nt, D, Dr, T, H)
    assert lib.sn_model_weight_count(lib.make_desc(1, 96, 32, 2, 32, 0.0, 10.0, 10.0)) == 0


def test_invalid_arguments_rejected_on_host(lib):
    L = lib.LIB
    n = ctypes.c_size_t()
    bad_sys = lib.make_system(0, 10)
    assert L.sn_workspace_size(None, ctypes.byref(bad_sys), ctypes.byref(n)) == lib.SN_ERR_INVALID_ARG
    good = lib.make_system(2, 10, False, 0.0)
    assert L.sn_workspace_size(None, ctypes.byref(good), ctypes.byref(n)) == lib.SN_OK
    assert n.value > 0 and n.value % 256 == 0
    # periodic box smaller than twice the radius, null pointers, negative capacity
    per = lib.make_system(1, 10, True, 9.0)
    dummy = ctypes.c_void_p(256)
    assert L.sn_build_neighbors(ctypes.byref(per), dummy, 5.0, dummy, dummy, 10, None, dummy,
                                10**9, None) == lib.SN_ERR_INVALID_ARG
    assert L.sn_build_neighbors(ctypes.byref(good), None, 5.0, dummy, dummy, 10, None, dummy,
                                10**9, None) == lib.SN_ERR_INVALID_ARG
    assert L.sn_build_neighbors(ctypes.byref(good), dummy, 5.0, dummy, dummy, -1, None, dummy,
                                10**9, None) == lib.SN_ERR_INVALID_ARG
    assert L.sn_build_neighbors(ctypes.byref(good), dummy, float("nan"), dummy, dummy, 10, None,
                                dummy, 10**9, None) == lib.SN_ERR_INVALID_ARG
    # workspace too small or misaligned
    assert L.sn_build_neighbors(ctypes.byref(good), dummy, 5.0, dummy, dummy, 10, None, dummy, 16,
                                None) == lib.SN_ERR_WORKSPACE
    assert L.sn_build_neighbors(ctypes.byref(good), dummy, 5.0, dummy, dummy, 10, None,
                                ctypes.c_void_p(100), 10**9, None) == lib.SN_ERR_INVALID_ARG
    # model creation: wrong weight count, unsupported width, non-finite weight
    d = lib.make_desc(1, 64, 32, 2, 32, 0.0, 10.0, 10.0)
    out = ctypes.c_void_p()
    w = np.zeros(10, np.float32)
    assert L.sn_model_create(ctypes.byref(d), w.ctypes.data_as(ctypes.c_void_p), 10,
                             ctypes.byref(out)) == lib.SN_ERR_INVALID_ARG
    d96 = lib.make_desc(1, 96, 32, 2, 32, 0.0, 10.0, 10.0)
    assert L.sn_model_create(ctypes.byref(d96), w.ctypes.data_as(ctypes.c_void_p), 10,
                             ctypes.byref(out)) == lib.SN_ERR_UNSUPPORTED
    nw = lib.sn_model_weight_count(d)
    w = np.zeros(nw, np.float32)
    w[5] = np.nan
    assert L.sn_model_create(ctypes.byref(d), w.ctypes.data_as(ctypes.c_void_p), nw,
                             ctypes.byref(out)) == lib.SN_ERR_INVALID_ARG
    # MD parameters: zero step, zero mass, bad cadence
    st = lib.SnMdState(256, 256, 256, 256, 256, 256, 10, 0)
    for prm in (lib.make_md_params(dt_fs=0.0), lib.make_md_params(mass_amu=0.0),
                lib.make_md_params(rebuild_every=0)):
        assert L.sn_md_step(dummy, ctypes.byref(good), dummy, ctypes.byref(prm), ctypes.byref(st),
                            1, None, dummy, 10**9, None) == lib.SN_ERR_INVALID_ARG
    # an active list needs both of its buffers
    half = lib.SnMdState(256, 256, 256, 256, 256, 256, 10, 0, 256, None)
    prm = lib.make_md_params()
    assert L.sn_md_step(dummy, ctypes.byref(good), dummy, ctypes.byref(prm), ctypes.byref(half), 1,
                        None, dummy, 10**9, None) == lib.SN_ERR_INVALID_ARG
    assert L.sn_philox4x64_10(None, 0, 0, None, -1, None) == lib.SN_ERR_INVALID_ARG
    assert L.sn_get_device_status(None, 0, None, None, None, None) == lib.SN_ERR_INVALID_ARG
    zero = ctypes.c_int64()
    ms = ctypes.c_double()
    assert L.sn_profile_read(0, ctypes.byref(ms), ctypes.byref(zero)) == lib.SN_OK
    assert zero.value == 0
