"""CPU oracle for filter-first constrained beam search (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use this package.  The product library never imports, links or
calls it.  See ``oracle.c`` for what is computed and which passages of the
ZeroGR description each part follows.

The decode loop below is the "overall pipeline" section of the ZeroGR page,
step by step: the model (here the seeded hidden-vector stub) gives each beam a
hidden vector, the oracle step filters, scores, normalises over the legal
tokens, adds to the cumulative log-prob and keeps the best K per request.
A request starts from one empty-prefix beam with cumulative log-prob 0.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Callable, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", _SRC, "-lm", "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None
_P = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        # ORACLE_LIB points the binding at another build of oracle.c (the
        # mutation tests load deliberately broken copies this way).
        path = os.environ.get("ORACLE_LIB", _LIB)
        if path == _LIB and not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(path)
        L.orc_build.restype = ctypes.c_int
        L.orc_build.argtypes = [_P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                ctypes.POINTER(ctypes.c_void_p)]
        L.orc_free.restype = None
        L.orc_free.argtypes = [_P]
        L.orc_count.restype = ctypes.c_int64
        L.orc_count.argtypes = [_P, ctypes.c_int32]
        L.orc_input_row.restype = ctypes.c_int64
        L.orc_input_row.argtypes = [_P, ctypes.c_int64]
        L.orc_node.restype = ctypes.c_int64
        L.orc_node.argtypes = [_P, _P, ctypes.c_int32]
        L.orc_legal.restype = ctypes.c_int64
        L.orc_legal.argtypes = [_P, _P, ctypes.c_int32, _P, ctypes.c_int64]
        L.orc_step_mode.restype = ctypes.c_int
        L.orc_step_mode.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32,
                                    ctypes.c_int32, _P, _P, _P, ctypes.c_int32, ctypes.c_int64,
                                    _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        L.orc_step.restype = ctypes.c_int
        L.orc_step.argtypes = [_P, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                               ctypes.c_int32, ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                               _P]
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


# Decoding modes (oracle.c, orc_step_mode): the method, and the two orders it
# is compared with.
MODES = {"filter_first": 0, "score_first": 1, "unconstrained": 2}


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


@dataclass
class StepResult:
    """Every legal candidate of one request at one step, and the selection."""
    cand_beam: np.ndarray   # int32 [n]
    cand_token: np.ndarray  # int32 [n]
    cand_logp: np.ndarray   # float64 [n], log-softmax over the beam's legal tokens
    cand_score: np.ndarray  # float64 [n], cumulative + logp
    sel_beam: np.ndarray    # int32 [k]  (rank order)
    sel_token: np.ndarray   # int32 [k]
    sel_score: np.ndarray   # float64 [k]
    sel_node: np.ndarray    # int64 [k]  row of the extended prefix; item id at the last step


class Catalog:
    """The catalog's trie (per-depth sorted node sets) for one list of SIDs."""

    def __init__(self, sids: np.ndarray, V: int):
        sids = np.ascontiguousarray(sids, dtype=np.int32)
        if sids.ndim != 2:
            raise ValueError("sids must be [N, L]")
        self.N, self.L = sids.shape
        self.V = V
        h = ctypes.c_void_p()
        rc = lib().orc_build(sids.ctypes.data, self.N, self.L, V, ctypes.byref(h))
        if rc != 0:
            raise OracleError({1: "bad arguments", 2: "token out of range", 3: "duplicate SID",
                               4: "out of memory"}.get(rc, str(rc)))
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            lib().orc_free(h)
            self._h = None

    def count(self, depth: int) -> int:
        """Distinct prefixes of length `depth` (rows of the step-(depth+1) table)."""
        return int(lib().orc_count(self._h, depth))

    def node(self, prefix) -> int:
        p = np.ascontiguousarray(np.asarray(prefix, dtype=np.int32).reshape(-1))
        return int(lib().orc_node(self._h, _ptr(p) if p.size else None, p.size))

    def legal(self, prefix) -> np.ndarray:
        p = np.ascontiguousarray(np.asarray(prefix, dtype=np.int32).reshape(-1))
        out = np.empty(self.V, dtype=np.int32)
        n = lib().orc_legal(self._h, _ptr(p) if p.size else None, p.size, out.ctypes.data, self.V)
        if n < 0:
            raise OracleError("bad prefix length")
        return out[:n].copy()

    def input_row(self, item: int) -> int:
        return int(lib().orc_input_row(self._h, item))

    def step(self, t: int, W: np.ndarray, prefix: np.ndarray, cum: np.ndarray, h: np.ndarray,
             K: int, mode: str = "filter_first") -> StepResult:
        """One step of one request.  W [V, d] float32 (stored values widened),
        prefix [k_in, t-1] int32, cum [k_in] (float64; -inf = dead beam),
        h [k_in, d] float32.  mode: a key of MODES."""
        m = MODES[mode]
        W = np.ascontiguousarray(W, dtype=np.float32)
        h = np.ascontiguousarray(h, dtype=np.float32)
        cum = np.ascontiguousarray(cum, dtype=np.float64)
        k_in, d = h.shape
        if W.shape[1] != d or cum.shape[0] != k_in:
            raise ValueError("shape mismatch")
        prefix = np.ascontiguousarray(np.asarray(prefix, dtype=np.int32).reshape(k_in, t - 1))
        cap = 0
        for k in range(k_in):
            if np.isfinite(cum[k]):
                cap += self.V if m == 2 else len(self.legal(prefix[k]))
        cap = max(cap, 1)
        cb = np.empty(cap, np.int32)
        ct = np.empty(cap, np.int32)
        cl = np.empty(cap, np.float64)
        cs = np.empty(cap, np.float64)
        sb = np.empty(K, np.int32)
        st = np.empty(K, np.int32)
        ss = np.empty(K, np.float64)
        sn = np.empty(K, np.int64)
        n_cand = ctypes.c_int64()
        n_sel = ctypes.c_int32()
        rc = lib().orc_step_mode(self._h, m, t, W.ctypes.data, d, k_in,
                            prefix.ctypes.data if t > 1 else None, cum.ctypes.data, h.ctypes.data,
                            K, cap, cb.ctypes.data, ct.ctypes.data, cl.ctypes.data, cs.ctypes.data,
                            ctypes.byref(n_cand), sb.ctypes.data, st.ctypes.data, ss.ctypes.data,
                            sn.ctypes.data, ctypes.byref(n_sel))
        if rc != 0:
            raise OracleError(f"orc_step failed ({rc})")
        n, k = n_cand.value, n_sel.value
        return StepResult(cb[:n], ct[:n], cl[:n], cs[:n], sb[:k], st[:k], ss[:k], sn[:k])


@dataclass
class DecodeResult:
    item: np.ndarray    # int64 [top_k]  item id (lexicographic rank); -1 = none
    sid: np.ndarray     # int32 [top_k, L]
    score: np.ndarray   # float64 [top_k]
    steps: List[dict]   # per step: the beams fed in and the StepResult


HiddenFn = Callable[[int, int, np.ndarray], np.ndarray]


def decode(cat: Catalog, W: List[np.ndarray], hidden: HiddenFn, request: int, K: int,
           top_k: Optional[int] = None, keep_steps: bool = False,
           mode: str = "filter_first") -> DecodeResult:
    """Beam search for one request (filter-first unless `mode` says otherwise).

    W[t-1] is the step-t weight matrix [V, d] (float32 values as stored);
    hidden(request, t, prefixes [k_in, t-1]) returns [k_in, d] float32.
    In the unconstrained mode a returned SID need not be a catalog item: its
    item id is then -1.
    """
    top_k = K if top_k is None else top_k
    L = cat.L
    prefixes = np.zeros((1, 0), dtype=np.int32)
    cum = np.zeros(1, dtype=np.float64)
    steps = []
    res = None
    for t in range(1, L + 1):
        h = hidden(request, t, prefixes)
        res = cat.step(t, W[t - 1], prefixes, cum, h, K, mode)
        if keep_steps:
            steps.append(dict(prefix=prefixes.copy(), cum=cum.copy(), h=h, res=res))
        k = len(res.sel_beam)
        new_prefix = np.empty((k, t), dtype=np.int32)
        new_prefix[:, : t - 1] = prefixes[res.sel_beam]
        new_prefix[:, t - 1] = res.sel_token
        prefixes = new_prefix
        cum = res.sel_score.copy()
    k = len(cum)
    item = np.full(top_k, -1, dtype=np.int64)
    sid = np.full((top_k, L), -1, dtype=np.int32)
    score = np.full(top_k, -np.inf, dtype=np.float64)
    n = min(k, top_k)
    item[:n] = res.sel_node[:n]
    sid[:n] = prefixes[:n]
    score[:n] = cum[:n]
    return DecodeResult(item, sid, score, steps)
