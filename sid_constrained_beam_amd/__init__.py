"""Python binding of libzgr (filter-first constrained beam search on MI355X).

Argument marshalling only: every step of the search runs in the HIP kernels
of ``libzgr.so`` behind the C ABI declared in ``include/zgr.h``.  Device
buffers are passed as torch tensors on the current HIP device (their
``data_ptr()``), host buffers as numpy arrays, streams as torch streams (or
raw ``hipStream_t`` integers).  There is no fallback: if the library is
missing, importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Callable, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzgr.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "zgr.h")

ZGR_OK, ZGR_E_ARG, ZGR_E_DUP_SID, ZGR_E_TOKEN_RANGE, ZGR_E_SHAPE = 0, 1, 2, 3, 4
ZGR_E_NOMEM, ZGR_E_HIP, ZGR_E_STATE, ZGR_E_CALLBACK, ZGR_E_DEVICE = 5, 6, 7, 8, 9
ZGR_F32, ZGR_BF16, ZGR_F16 = 0, 1, 2
ZGR_FMT_AUTO, ZGR_FMT_DENSE, ZGR_FMT_SPARSE, ZGR_FMT_DENSE_NEXT = 0, 1, 2, 3
ZGR_PROJ_AUTO, ZGR_PROJ_FULL, ZGR_PROJ_SELECTIVE = 0, 1, 2
ZGR_UPLOAD_STAGED, ZGR_UPLOAD_DIRECT = 0, 1
UPLOAD_CODES = {"staged": ZGR_UPLOAD_STAGED, "direct": ZGR_UPLOAD_DIRECT}
ZGR_SLICES_AUTO, ZGR_SLICES_ALWAYS, ZGR_SLICES_NEVER = 0, 1, 2
SLICE_CODES = {"auto": ZGR_SLICES_AUTO, "always": ZGR_SLICES_ALWAYS, "never": ZGR_SLICES_NEVER}
KERNELS = ["units", "selective", "gemm", "request", "norm"]
ZGR_MODE_FILTER_FIRST, ZGR_MODE_SCORE_FIRST, ZGR_MODE_UNCONSTRAINED = 0, 1, 2
MODE_CODES = {"filter_first": ZGR_MODE_FILTER_FIRST, "score_first": ZGR_MODE_SCORE_FIRST,
              "unconstrained": ZGR_MODE_UNCONSTRAINED}

DTYPE_CODES = {"f32": ZGR_F32, "bf16": ZGR_BF16, "f16": ZGR_F16}
FMT_CODES = {None: ZGR_FMT_AUTO, "A": ZGR_FMT_AUTO, "D": ZGR_FMT_DENSE, "S": ZGR_FMT_SPARSE,
             "N": ZGR_FMT_DENSE_NEXT}
ZGR_PROJ_NAIVE = 3
ZGR_PROJ_STAGED = 4
ZGR_REQ_TOKEN, ZGR_REQ_SLOT, ZGR_REQ_SCORED, ZGR_REQ_PRUNED = 0, 1, 2, 5
PROJ_CODES = {None: ZGR_PROJ_AUTO, "auto": ZGR_PROJ_AUTO, "full": ZGR_PROJ_FULL,
              "selective": ZGR_PROJ_SELECTIVE, "naive": ZGR_PROJ_NAIVE, "staged": ZGR_PROJ_STAGED}

_P = ctypes.c_void_p
_I32, _I64 = ctypes.c_int32, ctypes.c_int64

HIDDEN_FN = ctypes.CFUNCTYPE(ctypes.c_int32, _P, _I32, _I32, _I32, _P, _I32, _P, _P)


class StepStats(ctypes.Structure):
    _fields_ = [("rows", _I64), ("nnz", _I64), ("fmt", _I32), ("stride", _I32), ("bytes", _I64),
                ("max_legal", _I32), ("slice_dir", _I32)]


class BuildOpts(ctypes.Structure):
    _fields_ = [("host_threads", _I32), ("upload", _I32), ("staging_bytes", _I64),
                ("slices", _I32), ("reserved", _I32)]


class BuildTimes(ctypes.Structure):
    _fields_ = [("keys_ms", ctypes.c_double), ("sort_ms", ctypes.c_double),
                ("layout_ms", ctypes.c_double), ("encode_ms", ctypes.c_double),
                ("build_ms", ctypes.c_double), ("alloc_ms", ctypes.c_double),
                ("upload_ms", ctypes.c_double), ("device_bytes", _I64), ("threads", _I32),
                ("upload", _I32)]

    def as_dict(self) -> dict:
        d = {k: getattr(self, k) for k, _ in self._fields_}
        d["upload"] = {v: k for k, v in UPLOAD_CODES.items()}.get(d["upload"], d["upload"])
        return d


class ZgrError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_str(status)} ({status}): {detail}")
        self.status = status
        self.detail = detail


_lib = None


def lib() -> ctypes.CDLL:
    """Load libzgr.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(hipcc, gfx950); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "zgr_status_str": (ctypes.c_char_p, [_I32]),
            "zgr_last_error": (_I32, [ctypes.c_char_p, ctypes.c_size_t]),
            "zgr_index_build_host": (_I32, [_P, _I64, _I32, _I32, _P, _P, ctypes.POINTER(_P)]),
            "zgr_index_to_device": (_I32, [_P, _P]),
            "zgr_index_upload": (_I32, [_P, _I64, _I32, _I32, _P, _P, ctypes.POINTER(_P), _P]),
            "zgr_index_build_host_ex": (_I32, [_P, _I64, _I32, _I32, _P, _P,
                                               ctypes.POINTER(BuildOpts),
                                               ctypes.POINTER(BuildTimes), ctypes.POINTER(_P)]),
            "zgr_index_to_device_ex": (_I32, [_P, _P, ctypes.POINTER(BuildOpts),
                                              ctypes.POINTER(BuildTimes)]),
            "zgr_index_upload_ex": (_I32, [_P, _I64, _I32, _I32, _P, _P, ctypes.POINTER(BuildOpts),
                                           ctypes.POINTER(BuildTimes), ctypes.POINTER(_P), _P]),
            "zgr_index_times": (_I32, [_P, ctypes.POINTER(BuildTimes)]),
            "zgr_index_device_table": (_I32, [_P, _I32, ctypes.POINTER(_P), ctypes.POINTER(_P),
                                              ctypes.POINTER(_P), ctypes.POINTER(_P),
                                              ctypes.POINTER(_P)]),
            "zgr_index_stats": (_I32, [_P, _I32, ctypes.POINTER(StepStats)]),
            "zgr_index_host_table": (_I32, [_P, _I32, ctypes.POINTER(_P), ctypes.POINTER(_P),
                                            ctypes.POINTER(_P)]),
            "zgr_index_host_slices": (_I32, [_P, _I32, ctypes.POINTER(_P)]),
            "zgr_index_shape": (_I32, [_P, ctypes.POINTER(_I32), ctypes.POINTER(_I32),
                                       ctypes.POINTER(_I64)]),
            "zgr_index_free": (None, [_P]),
            "zgr_plan_warmup": (_I32, [_P, _P, _I32, _I32, _I32, _I32, HIDDEN_FN, _P, _I32, _P, _P,
                                       ctypes.POINTER(_P)]),
            "zgr_plan_choice": (_I32, [_P, _I32, ctypes.POINTER(_I32), ctypes.POINTER(ctypes.c_float),
                                       ctypes.POINTER(ctypes.c_float)]),
            "zgr_plan_set_choice": (_I32, [_P, _I32, _I32]),
            "zgr_plan_set_mode": (_I32, [_P, _I32]),
            "zgr_plan_mode": (_I32, [_P, ctypes.POINTER(_I32)]),
            "zgr_plan_free": (None, [_P]),
            "zgr_step": (_I32, [_P, _I32, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _P]),
            "zgr_decode": (_I32, [_P, HIDDEN_FN, _P, _I32, _P, _P, _P, _P]),
            "zgr_plan_status": (_I32, [_P, _P]),
            "zgr_plan_request_path": (_I32, [_P, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
            "zgr_plan_profile": (_I32, [_P, _I32]),
            "zgr_plan_profile_read": (_I32, [_P, _I32, _I32, ctypes.POINTER(_I64),
                                             ctypes.POINTER(ctypes.c_double)]),
            "zgr_step_noalloc": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P,
                                        _I32, _P, _P, _P, _P, _P, _P, _P]),
            "zgr_full_projection_variant": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32,
                                                   ctypes.POINTER(_I32), ctypes.POINTER(_I32),
                                                   ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_symbols() -> List[str]:
    """Names of the functions that include/zgr.h declares."""
    import re
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(zgr_[a-z0-9_]+)\s*\(", text)) - {"zgr_hidden_fn"})


def status_str(status: int) -> str:
    return lib().zgr_status_str(status).decode()


def last_error() -> str:
    buf = ctypes.create_string_buffer(1024)
    lib().zgr_last_error(buf, len(buf))
    return buf.value.decode()


def _check(status: int):
    if status != ZGR_OK:
        raise ZgrError(status, last_error())


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


# --------------------------------------------------------------------------- index

class Index:
    """Owner of a zgr_index handle."""

    def __init__(self, handle: ctypes.c_void_p):
        self._h = handle

    @property
    def handle(self):
        return self._h

    def free(self):
        if self._h is not None and self._h.value:
            lib().zgr_index_free(self._h)
        self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass

    def shape(self):
        return zgr_index_shape(self)

    def stats(self, t: int) -> dict:
        return zgr_index_stats(self, t)

    def host_table(self, t: int):
        return zgr_index_host_table(self, t)


def _fmt_array(fmt, L):
    if fmt is None:
        return None
    a = np.asarray([FMT_CODES[f] if not isinstance(f, (int, np.integer)) else int(f) for f in fmt],
                   dtype=np.int32)
    if a.shape != (L,):
        raise ValueError("fmt must have L entries")
    return a


def _opts(threads: int, upload, staging_bytes: int, slices="auto"):
    sl = SLICE_CODES[slices] if isinstance(slices, str) else int(slices)
    if threads == 0 and upload in (None, "staged") and staging_bytes == 0 and sl == ZGR_SLICES_AUTO:
        return None
    code = UPLOAD_CODES[upload] if isinstance(upload, str) else (
        ZGR_UPLOAD_STAGED if upload is None else int(upload))
    return BuildOpts(int(threads), code, int(staging_bytes), sl, 0)


def _ref(x):
    return None if x is None else ctypes.byref(x)


def zgr_index_build_host(sids: np.ndarray, V: int, fmt=None, want_rank: bool = True,
                         threads: int = 0, times: bool = False, slices="auto"):
    """Host-only build on `threads` threads (0 = automatic); `slices` is
    "auto", "always" or "never" (the sparse tables' slice directory).
    Returns (Index, rank_of_input int64 [N] or None), plus the phase times as
    a dict when `times`."""
    sids = np.ascontiguousarray(sids, dtype=np.int32)
    N, L = sids.shape
    f = _fmt_array(fmt, L)
    rank = np.empty(N, dtype=np.int64) if want_rank else None
    h = ctypes.c_void_p()
    o = _opts(threads, None, 0, slices)
    tm = BuildTimes() if times else None
    fp = None if f is None else f.ctypes.data
    rp = None if rank is None else rank.ctypes.data
    if o is None and tm is None:
        _check(lib().zgr_index_build_host(sids.ctypes.data, N, L, V, fp, rp, ctypes.byref(h)))
    else:
        _check(lib().zgr_index_build_host_ex(sids.ctypes.data, N, L, V, fp, rp, _ref(o), _ref(tm),
                                             ctypes.byref(h)))
    return (Index(h), rank, tm.as_dict()) if times else (Index(h), rank)


def zgr_index_to_device(index: Index, stream=None, threads: int = 0, upload=None,
                        staging_bytes: int = 0):
    """Copy a host-built index to HBM; returns the build and upload phase times."""
    o = _opts(threads, upload, staging_bytes)
    tm = BuildTimes()
    if o is None:
        _check(lib().zgr_index_to_device(index.handle, _stream_ptr(stream)))
        _check(lib().zgr_index_times(index.handle, ctypes.byref(tm)))
    else:
        _check(lib().zgr_index_to_device_ex(index.handle, _stream_ptr(stream), ctypes.byref(o),
                                            ctypes.byref(tm)))
    return tm.as_dict()


def zgr_index_upload(sids: np.ndarray, V: int, fmt=None, stream=None, want_rank: bool = True,
                     threads: int = 0, upload=None, staging_bytes: int = 0, slices="auto"):
    """Build on the host and copy to HBM.  Returns (Index, rank_of_input)."""
    sids = np.ascontiguousarray(sids, dtype=np.int32)
    N, L = sids.shape
    f = _fmt_array(fmt, L)
    rank = np.empty(N, dtype=np.int64) if want_rank else None
    h = ctypes.c_void_p()
    o = _opts(threads, upload, staging_bytes, slices)
    fp = None if f is None else f.ctypes.data
    rp = None if rank is None else rank.ctypes.data
    if o is None:
        _check(lib().zgr_index_upload(sids.ctypes.data, N, L, V, fp, _stream_ptr(stream),
                                      ctypes.byref(h), rp))
    else:
        _check(lib().zgr_index_upload_ex(sids.ctypes.data, N, L, V, fp, _stream_ptr(stream),
                                         ctypes.byref(o), None, ctypes.byref(h), rp))
    return Index(h), rank


def zgr_index_times(index: Index) -> dict:
    tm = BuildTimes()
    _check(lib().zgr_index_times(index.handle, ctypes.byref(tm)))
    return tm.as_dict()


def zgr_index_device_table(index: Index, t: int):
    """Device pointers of table t: (row_ptr, tok, bits, rank, next), 0 where absent."""
    ptrs = [_P() for _ in range(5)]
    _check(lib().zgr_index_device_table(index.handle, t, *[ctypes.byref(p) for p in ptrs]))
    return tuple(p.value or 0 for p in ptrs)


def zgr_index_stats(index: Index, t: int) -> dict:
    st = StepStats()
    _check(lib().zgr_index_stats(index.handle, t, ctypes.byref(st)))
    return {k: getattr(st, k) for k, _ in StepStats._fields_}


def zgr_index_shape(index: Index):
    L, V, N = _I32(), _I32(), _I64()
    _check(lib().zgr_index_shape(index.handle, ctypes.byref(L), ctypes.byref(V), ctypes.byref(N)))
    return L.value, V.value, N.value


def zgr_index_host_table(index: Index, t: int):
    """Copies of table t: (row_ptr int32 [rows+1], tok uint16 [nnz], bits uint32 [rows, words] or None)."""
    rp, tk, bt = _P(), _P(), _P()
    _check(lib().zgr_index_host_table(index.handle, t, ctypes.byref(rp), ctypes.byref(tk),
                                      ctypes.byref(bt)))
    st = zgr_index_stats(index, t)
    _, V, _ = zgr_index_shape(index)
    rows, nnz = st["rows"], st["nnz"]
    row_ptr = np.ctypeslib.as_array(ctypes.cast(rp, ctypes.POINTER(ctypes.c_int32)), (rows + 1,)).copy()
    tok = (np.ctypeslib.as_array(ctypes.cast(tk, ctypes.POINTER(ctypes.c_uint16)), (nnz,)).copy()
           if nnz else np.zeros(0, np.uint16))
    bits = None
    if bt.value:
        words = (V + 31) // 32
        bits = np.ctypeslib.as_array(ctypes.cast(bt, ctypes.POINTER(ctypes.c_uint32)),
                                     (rows, words)).copy()
    return row_ptr, tok, bits


def zgr_index_host_slices(index: Index, t: int):
    """Copy of table t's slice directory (uint16 [rows, 8]), or None when the table has none."""
    sp = _P()
    _check(lib().zgr_index_host_slices(index.handle, t, ctypes.byref(sp)))
    if not sp.value:
        return None
    rows = zgr_index_stats(index, t)["rows"]
    return np.ctypeslib.as_array(ctypes.cast(sp, ctypes.POINTER(ctypes.c_uint16)), (rows, 8)).copy()


def zgr_index_free(index: Index):
    index.free()


# --------------------------------------------------------------------------- plan

HiddenCallable = Callable[[int, int, int, int, int, int, int], int]


def make_hidden_fn(fn: HiddenCallable):
    """Wrap fn(t, B, k_in, prefix_ptr, prefix_ld, hidden_ptr, stream_ptr) -> int
    as a C callback.  Keep the returned object alive while it may be called."""
    def tramp(user, t, B, k_in, prefix_ptr, prefix_ld, hidden_ptr, stream_ptr):
        try:
            return int(fn(t, B, k_in, prefix_ptr or 0, prefix_ld, hidden_ptr or 0, stream_ptr or 0))
        except Exception:  # noqa: BLE001 - report as a callback failure
            import traceback
            traceback.print_exc()
            return 1
    return HIDDEN_FN(tramp)


class Plan:
    """Owner of a zgr_plan handle (keeps the weights and callback alive)."""

    def __init__(self, handle, index: Index, W, L: int):
        self._h = handle
        self.index = index
        self.W = W
        self.L = L
        self._keep = []

    @property
    def handle(self):
        return self._h

    def free(self):
        if self._h is not None and self._h.value:
            lib().zgr_plan_free(self._h)
        self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:  # noqa: BLE001
            pass

    def choice(self, t: int):
        return zgr_plan_choice(self, t)


def zgr_plan_warmup(index: Index, W: Sequence, dtype: str, d: int, B: int, K: int,
                    hidden_fn: Optional[HiddenCallable] = None, n_warmup: int = 0, force=None,
                    stream=None) -> Plan:
    """W: L device tensors [V, d] of dtype (kept alive by the plan).
    force: None or L entries of 'auto' / 'full' / 'selective' (or ZGR_PROJ_* ints)."""
    L = len(W)
    ptrs = (ctypes.c_void_p * L)(*[w.data_ptr() for w in W])
    f = None
    if force is not None:
        f = np.asarray([PROJ_CODES[x] if not isinstance(x, (int, np.integer)) else int(x)
                        for x in force], dtype=np.int32)
    cb = make_hidden_fn(hidden_fn) if hidden_fn is not None else HIDDEN_FN()
    h = ctypes.c_void_p()
    _check(lib().zgr_plan_warmup(index.handle, ctypes.cast(ptrs, _P), DTYPE_CODES.get(dtype, dtype),
                                 d, B, K, cb, None, n_warmup, None if f is None else f.ctypes.data,
                                 _stream_ptr(stream), ctypes.byref(h)))
    p = Plan(h, index, list(W), L)
    p._keep.append(cb)
    return p


def zgr_plan_choice(plan: Plan, t: int):
    proj, uf, us = _I32(), ctypes.c_float(), ctypes.c_float()
    _check(lib().zgr_plan_choice(plan.handle, t, ctypes.byref(proj), ctypes.byref(uf), ctypes.byref(us)))
    return proj.value, uf.value, us.value


def zgr_plan_request_path(plan: Plan, t: int):
    """(kind, parts) of the request kernel at step t in the plan's last step or decode;
    kind is one of ZGR_REQ_TOKEN / SLOT / SCORED / PRUNED."""
    kind, parts = _I32(), _I32()
    _check(lib().zgr_plan_request_path(plan.handle, t, ctypes.byref(kind), ctypes.byref(parts)))
    return kind.value, parts.value


def zgr_plan_set_choice(plan: Plan, t: int, proj):
    code = PROJ_CODES[proj] if isinstance(proj, str) else int(proj)
    _check(lib().zgr_plan_set_choice(plan.handle, t, code))


def zgr_plan_set_mode(plan: Plan, mode):
    """Decoding mode: 'filter_first' (the method), 'score_first' or
    'unconstrained' (the comparisons), or a ZGR_MODE_* code."""
    code = MODE_CODES[mode] if isinstance(mode, str) else int(mode)
    _check(lib().zgr_plan_set_mode(plan.handle, code))


def zgr_plan_mode(plan: Plan) -> str:
    m = _I32()
    _check(lib().zgr_plan_mode(plan.handle, ctypes.byref(m)))
    return {v: k for k, v in MODE_CODES.items()}[m.value]


def zgr_plan_free(plan: Plan):
    plan.free()


def zgr_step(plan: Plan, t: int, hidden, row_in, cum_in, k_in: int, parent_out, token_out,
             row_out, cum_out, slot_dbg=None, stream=None):
    """Enqueue one step (all buffers are device tensors; see include/zgr.h)."""
    _check(lib().zgr_step(plan.handle, t, _dptr(hidden), _dptr(row_in), _dptr(cum_in), k_in,
                          _dptr(parent_out), _dptr(token_out), _dptr(row_out), _dptr(cum_out),
                          _dptr(slot_dbg), _stream_ptr(stream)))


def zgr_step_noalloc(index: Index, W_t, dtype: str, d: int, B: int, K: int, t: int, proj, hidden,
                     row_in, cum_in, k_in: int, parent_out, token_out, row_out, cum_out,
                     slot_dbg=None, err_out=None, stream=None):
    """One step without a plan: scratch from the library's static device array."""
    _check(lib().zgr_step_noalloc(index.handle, _dptr(W_t), DTYPE_CODES[dtype], int(d), int(B), int(K),
                                  int(t), PROJ_CODES[proj] if isinstance(proj, str) else int(proj),
                                  _dptr(hidden), _dptr(row_in), _dptr(cum_in),
                                  int(k_in), _dptr(parent_out), _dptr(token_out), _dptr(row_out),
                                  _dptr(cum_out), _dptr(slot_dbg), _dptr(err_out), _stream_ptr(stream)))


def zgr_decode(plan: Plan, hidden_fn: HiddenCallable, top_k: int, item_out, sid_out=None,
               score_out=None, stream=None):
    cb = make_hidden_fn(hidden_fn)
    _check(lib().zgr_decode(plan.handle, cb, None, top_k, _dptr(item_out), _dptr(sid_out),
                            _dptr(score_out), _stream_ptr(stream)))


GEMM_KERNELS = {0: "small", 1: "tiled"}
EPILOGUES = {0: "plain", 1: "dense", 2: "slot"}


def zgr_full_projection_variant(M: int, V: int, dtype: str, fmt: int, mode, n_cu: int = 256):
    """The full-projection kernel the library launches for a step shape:
    (kernel name, tile_m, tile_n, epilogue name).  Host only."""
    k, tm, tn, ep = _I32(), _I32(), _I32(), _I32()
    m = MODE_CODES[mode] if isinstance(mode, str) else int(mode)
    _check(lib().zgr_full_projection_variant(int(M), int(V), DTYPE_CODES[dtype], int(fmt), m, int(n_cu),
                                             ctypes.byref(k), ctypes.byref(tm), ctypes.byref(tn),
                                             ctypes.byref(ep)))
    return GEMM_KERNELS[k.value], tm.value, tn.value, EPILOGUES[ep.value]


def zgr_plan_status(plan: Plan, stream=None):
    _check(lib().zgr_plan_status(plan.handle, _stream_ptr(stream)))


def zgr_plan_profile(plan: Plan, repeat: int):
    """repeat > 0: time every launch, issued `repeat` times between two events; 0: off."""
    _check(lib().zgr_plan_profile(plan.handle, int(repeat)))


def zgr_plan_profile_read(plan: Plan, kernel, t: int):
    """(launches, total_ms) of a kernel class ('selective', 'gemm', ... or id) at step t."""
    k = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    n, ms = _I64(), ctypes.c_double()
    _check(lib().zgr_plan_profile_read(plan.handle, k, t, ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


# --------------------------------------------------------------------------- HIP memcpy helper

_hip = None


def hip_runtime() -> ctypes.CDLL:
    """libamdhip64 for raw-pointer copies inside hidden-vector callbacks."""
    global _hip
    if _hip is None:
        for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
            try:
                h = ctypes.CDLL(name)
                break
            except OSError:
                h = None
        if h is None:
            raise ImportError("libamdhip64.so not found")
        h.hipMemcpyAsync.restype = ctypes.c_int
        h.hipMemcpyAsync.argtypes = [_P, _P, ctypes.c_size_t, ctypes.c_int, _P]
        h.hipStreamSynchronize.restype = ctypes.c_int
        h.hipStreamSynchronize.argtypes = [_P]
        _hip = h
    return _hip


HIP_H2D, HIP_D2H, HIP_D2D = 1, 2, 3


def copy_to_device(dst_ptr: int, src: np.ndarray, stream_ptr: int):
    src = np.ascontiguousarray(src)
    h = hip_runtime()
    if h.hipMemcpyAsync(dst_ptr, src.ctypes.data, src.nbytes, HIP_H2D, stream_ptr) != 0:
        raise RuntimeError("hipMemcpyAsync H2D failed")
    if h.hipStreamSynchronize(stream_ptr) != 0:
        raise RuntimeError("hipStreamSynchronize failed")


def copy_to_host(dst: np.ndarray, src_ptr: int, stream_ptr: int):
    h = hip_runtime()
    if h.hipStreamSynchronize(stream_ptr) != 0:
        raise RuntimeError("hipStreamSynchronize failed")
    if h.hipMemcpyAsync(dst.ctypes.data, src_ptr, dst.nbytes, HIP_D2H, stream_ptr) != 0:
        raise RuntimeError("hipMemcpyAsync D2H failed")
    if h.hipStreamSynchronize(stream_ptr) != 0:
        raise RuntimeError("hipStreamSynchronize failed")


def copy_device(dst_ptr: int, src_ptr: int, nbytes: int, stream_ptr: int):
    if hip_runtime().hipMemcpyAsync(dst_ptr, src_ptr, nbytes, HIP_D2D, stream_ptr) != 0:
        raise RuntimeError("hipMemcpyAsync D2D failed")
