"""The C ABI: every declared symbol is exported; argument errors are reported
before any device work (these calls never touch a GPU)."""
import ctypes

import numpy as np
import pytest

import sid_constrained_beam_amd as zgr


def test_library_exports_every_declared_symbol():
    names = zgr.header_symbols()
    assert len(names) >= 15
    lib = ctypes.CDLL(zgr.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    for code in range(0, 10):
        s = zgr.status_str(code)
        assert s and s != "unknown status"
    assert zgr.status_str(99) == "unknown status"


def _expect(status, fn, *args):
    with pytest.raises(zgr.ZgrError) as e:
        fn(*args)
    assert e.value.status == status, (e.value.status, e.value.detail)
    return e.value


def test_index_argument_errors():
    ok = np.array([[0, 1], [1, 0]], np.int32)
    _expect(zgr.ZGR_E_ARG, zgr.zgr_index_build_host, ok, 1)            # V < 2
    _expect(zgr.ZGR_E_ARG, zgr.zgr_index_build_host, ok, 70000)        # V > 65536
    _expect(zgr.ZGR_E_ARG, zgr.zgr_index_build_host, np.zeros((0, 2), np.int32), 4)
    _expect(zgr.ZGR_E_ARG, zgr.zgr_index_build_host, np.zeros((3, 9), np.int32), 4)  # L > 8
    e = _expect(zgr.ZGR_E_TOKEN_RANGE, zgr.zgr_index_build_host, np.array([[0, 1], [1, 4]], np.int32), 4)
    assert "row 1" in e.detail
    _expect(zgr.ZGR_E_TOKEN_RANGE, zgr.zgr_index_build_host, np.array([[0, -1]], np.int32), 4)
    e = _expect(zgr.ZGR_E_DUP_SID, zgr.zgr_index_build_host,
                np.array([[0, 1], [2, 3], [0, 1]], np.int32), 4)
    assert "0" in e.detail and "2" in e.detail
    _expect(zgr.ZGR_E_SHAPE, zgr.zgr_index_build_host, np.zeros((1, 5), np.int32), 65536)  # 80 bits
    _expect(zgr.ZGR_E_ARG, zgr.zgr_index_build_host, ok, 4, [4, 0])    # bad fmt code
    L = zgr.lib()
    h = ctypes.c_void_p()
    assert L.zgr_index_build_host(None, 2, 2, 4, None, None, ctypes.byref(h)) == zgr.ZGR_E_ARG
    assert L.zgr_index_stats(None, 1, None) == zgr.ZGR_E_ARG
    assert L.zgr_index_to_device(None, None) == zgr.ZGR_E_ARG
    L.zgr_index_free(None)  # no-op


def test_rebuild_argument_errors():
    L = zgr.lib()
    ok = np.array([[0, 1], [1, 0]], np.int32)
    h = ctypes.c_void_p()
    tm = zgr.BuildTimes()
    neg = zgr.BuildOpts(-1, zgr.ZGR_UPLOAD_STAGED, 0)
    bad_mode = zgr.BuildOpts(0, 7, 0)
    neg_stage = zgr.BuildOpts(0, zgr.ZGR_UPLOAD_STAGED, -4)
    # checks run before any HIP call
    assert L.zgr_index_build_host_ex(ok.ctypes.data, 2, 2, 4, None, None, ctypes.byref(neg), None,
                                     ctypes.byref(h)) == zgr.ZGR_E_ARG
    for o in (bad_mode, neg_stage):
        assert L.zgr_index_upload_ex(ok.ctypes.data, 2, 2, 4, None, None, ctypes.byref(o), None,
                                     ctypes.byref(h), None) == zgr.ZGR_E_ARG
    assert L.zgr_index_upload_ex(ok.ctypes.data, 2, 2, 4, None, None, None, None, None, None) == zgr.ZGR_E_ARG
    assert L.zgr_index_to_device_ex(None, None, None, None) == zgr.ZGR_E_ARG
    assert L.zgr_index_times(None, ctypes.byref(tm)) == zgr.ZGR_E_ARG
    idx, _ = zgr.zgr_index_build_host(ok, 4)
    assert L.zgr_index_to_device_ex(idx.handle, None, ctypes.byref(bad_mode), None) == zgr.ZGR_E_ARG
    assert L.zgr_index_to_device_ex(idx.handle, None, ctypes.byref(neg_stage), None) == zgr.ZGR_E_ARG
    _expect(zgr.ZGR_E_STATE, zgr.zgr_index_device_table, idx, 1)  # host-only index
    _expect(zgr.ZGR_E_ARG, zgr.zgr_index_device_table, idx, 3)
    t = zgr.zgr_index_times(idx)
    assert t["threads"] == 1 and t["upload_ms"] == 0.0 and t["device_bytes"] > 0


def test_index_stats_range():
    idx, _ = zgr.zgr_index_build_host(np.array([[0, 1], [1, 0]], np.int32), 4)
    _expect(zgr.ZGR_E_ARG, zgr.zgr_index_stats, idx, 0)
    _expect(zgr.ZGR_E_ARG, zgr.zgr_index_stats, idx, 3)
    assert zgr.zgr_index_shape(idx) == (2, 4, 2)


def test_plan_and_step_argument_errors():
    L = zgr.lib()
    idx, _ = zgr.zgr_index_build_host(np.array([[0, 1], [1, 0]], np.int32), 4)
    W = (ctypes.c_void_p * 2)(1, 1)
    out = ctypes.c_void_p()
    cb = zgr.HIDDEN_FN()
    # null index / weights / out
    assert L.zgr_plan_warmup(None, W, 0, 64, 1, 1, cb, None, 0, None, None, ctypes.byref(out)) == zgr.ZGR_E_ARG
    assert L.zgr_plan_warmup(idx.handle, None, 0, 64, 1, 1, cb, None, 0, None, None, ctypes.byref(out)) == zgr.ZGR_E_ARG
    # bad dtype, sizes, hidden size, K
    assert L.zgr_plan_warmup(idx.handle, W, 7, 64, 1, 1, cb, None, 0, None, None, ctypes.byref(out)) == zgr.ZGR_E_ARG
    assert L.zgr_plan_warmup(idx.handle, W, 0, 64, 0, 1, cb, None, 0, None, None, ctypes.byref(out)) == zgr.ZGR_E_ARG
    assert L.zgr_plan_warmup(idx.handle, W, 0, 100, 1, 1, cb, None, 0, None, None, ctypes.byref(out)) == zgr.ZGR_E_SHAPE
    assert L.zgr_plan_warmup(idx.handle, W, 0, 64, 1, 2000, cb, None, 0, None, None, ctypes.byref(out)) == zgr.ZGR_E_SHAPE
    bad_force = (ctypes.c_int32 * 2)(0, 5)
    assert L.zgr_plan_warmup(idx.handle, W, 0, 64, 1, 1, cb, None, 0, bad_force, None, ctypes.byref(out)) == zgr.ZGR_E_ARG
    # every named projection (the staged comparison included) passes the force check
    ok_force = (ctypes.c_int32 * 2)(zgr.ZGR_PROJ_NAIVE, zgr.ZGR_PROJ_STAGED)
    assert L.zgr_plan_warmup(idx.handle, W, 0, 64, 1, 1, cb, None, 0, ok_force, None, ctypes.byref(out)) == zgr.ZGR_E_STATE
    # the index was built on the host only: a plan needs it on the device
    assert L.zgr_plan_warmup(idx.handle, W, 0, 64, 1, 1, cb, None, 0, None, None, ctypes.byref(out)) == zgr.ZGR_E_STATE
    assert "not on the device" in zgr.last_error()
    # step / decode / choice on a null plan
    assert L.zgr_step(None, 1, 1, 1, 1, 1, 1, 1, 1, 1, None, None) == zgr.ZGR_E_ARG
    assert L.zgr_decode(None, cb, None, 1, 1, None, None, None) == zgr.ZGR_E_ARG
    assert L.zgr_plan_choice(None, 1, None, None, None) == zgr.ZGR_E_ARG
    assert L.zgr_plan_set_choice(None, 1, 1) == zgr.ZGR_E_ARG
    assert L.zgr_plan_status(None, None) == zgr.ZGR_E_ARG
    assert L.zgr_plan_set_mode(None, 0) == zgr.ZGR_E_ARG
    assert L.zgr_plan_mode(None, None) == zgr.ZGR_E_ARG
    assert L.zgr_plan_request_path(None, 1, None, None) == zgr.ZGR_E_ARG
    L.zgr_plan_free(None)


def test_last_error_is_thread_local():
    import threading
    _expect(zgr.ZGR_E_ARG, zgr.zgr_index_build_host, np.array([[0, 1]], np.int32), 1)
    seen = {}

    def other():
        _expect(zgr.ZGR_E_DUP_SID, zgr.zgr_index_build_host, np.array([[0, 1], [0, 1]], np.int32), 4)
        seen["other"] = zgr.last_error()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert "share one SID" in seen["other"]
    assert "V must be" in zgr.last_error()


def test_step_noalloc_argument_errors():
    """zgr_step_noalloc checks its arguments before any HIP call."""
    L = zgr.lib()
    sids = np.array([[0, 1], [1, 0], [1, 1]], np.int32)
    idx, _ = zgr.zgr_index_build_host(sids, 4)   # host only: not on a device
    p = ctypes.c_void_p(8)  # never dereferenced: every call below fails its checks first
    args = lambda **kw: dict(dict(idx=idx.handle, W=p, dtype=zgr.ZGR_F32, d=64, B=2, K=4, t=1,
                                  proj=zgr.ZGR_PROJ_SELECTIVE, k_in=1), **kw)

    def call(a):
        return L.zgr_step_noalloc(a["idx"], a["W"], a["dtype"], a["d"], a["B"], a["K"], a["t"],
                                  a["proj"], p, p, p, a["k_in"], p, p, p, p, None, None, None)
    assert call(args(idx=None)) == zgr.ZGR_E_ARG
    assert call(args(W=None)) == zgr.ZGR_E_ARG
    assert call(args(dtype=5)) == zgr.ZGR_E_ARG
    assert call(args(K=2000)) == zgr.ZGR_E_SHAPE
    assert call(args(d=100)) == zgr.ZGR_E_SHAPE
    assert call(args(t=3)) == zgr.ZGR_E_ARG
    assert call(args(k_in=5)) == zgr.ZGR_E_ARG
    assert call(args(proj=zgr.ZGR_PROJ_AUTO)) == zgr.ZGR_E_ARG
    assert call(args(proj=zgr.ZGR_PROJ_NAIVE)) == zgr.ZGR_E_ARG
    assert call(args(proj=zgr.ZGR_PROJ_STAGED)) == zgr.ZGR_E_ARG
    assert call(args()) == zgr.ZGR_E_STATE  # the index is not on a device
    idx.free()
