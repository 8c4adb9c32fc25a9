"""Seeded synthetic workloads for filter-first constrained beam search.

The catalogs, per-step weights W_t and per-beam hidden vectors that both the
CPU oracle and the HIP library consume.  Nothing here computes any part of
the search itself; it only draws inputs (see ``wl.cpp``).

Workload shapes follow the five configurations the method is evaluated on
(ZeroGR page, "is it really better" section, for the codebook sweep at batch
32; the Watch profile of 100% / ~90% legal tokens at steps 1 and 2 in the
"fewer scores is not faster" section; the 10^7 - 10^8 item production scale
in the "what problem" section).  The readings taken where the description is
open (std deviations, hash, Zipf via keyed permutation, redraw rounds, the 90%
subset) are: N(0, x) takes x as the standard deviation; per-level tokens are
ranks of the level law mapped through a keyed bijection of [0, V) seeded by
the prefix; a repeated SID is redrawn whole with the next attempt number; the
~90% level-2 profile is a uniform law over the first 90% of that bijection.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wl.cpp")
_LIB = os.path.join(_HERE, "libwl.so")

DTYPES = {"f32": 0, "bf16": 1, "f16": 2}


def build(force: bool = True) -> str:
    """Compile the generator with the host compiler (no GPU code)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        L.wl_catalog.restype = ctypes.c_int32
        L.wl_catalog.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p]
        L.wl_weights.restype = None
        L.wl_weights.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_double, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_int32]
        L.wl_hidden.restype = None
        L.wl_hidden.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double,
                                ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
        L.wl_round.restype = None
        L.wl_round.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                               ctypes.c_void_p]
        L.wl_perm.restype = ctypes.c_uint32
        L.wl_perm.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32]
        _lib = L
    return _lib


def _threads() -> int:
    try:
        n = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        n = 0
    return max(1, min(n if n > 0 else (os.cpu_count() or 1), 16))


ZIPF, UNIFORM, UNIFORM_SUBSET = 0, 1, 2


@dataclass
class Config:
    """One synthetic workload: catalog law, model shape, batch and precision."""
    name: str
    L: int
    V: int
    N: int
    kinds: List[int]
    params: List[float]
    d: int
    K: int
    B: int
    dtype: str
    fmt: Optional[List[str]] = None  # per-step table format ("D"/"S"/"N"), None = automatic
    seed_cat: int = 1000
    seed_w: int = 2000
    seed_h: int = 3000

    @property
    def w_std(self) -> float:
        return 3.0 / np.sqrt(self.d)

    @property
    def h_std(self) -> float:
        return 1.0 / np.sqrt(self.d)

    def scaled(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


def _cfg(c, name, L, V, N, kinds, params, d, K, B, dtype, fmt=None):
    return Config(name, L, V, N, kinds, params, d, K, B, dtype, fmt,
                  seed_cat=1000 + c, seed_w=2000 + c, seed_h=3000 + c)


CONFIGS = {
    # tiny CPU-scale case
    "n1e4_v256": _cfg(1, "n1e4_v256", 3, 256, 10_000, [ZIPF] * 3, [1.1] * 3, 64, 16, 1, "f32"),
    # dense step 1 -> sparse step 3, batch 32
    "n1e6_v2048": _cfg(2, "n1e6_v2048", 3, 2048, 1_000_000, [ZIPF] * 3, [1.1] * 3, 256, 64, 32, "f32"),
    # codebook sweep at a fixed 10^7-item catalog, bf16 storage
    "n1e7_v2048": _cfg(3, "n1e7_v2048", 4, 2048, 10_000_000, [ZIPF] * 4, [1.1] * 4, 512, 128, 32, "bf16"),
    "n1e7_v4096": _cfg(3, "n1e7_v4096", 4, 4096, 10_000_000, [ZIPF] * 4, [1.1] * 4, 512, 128, 32, "bf16"),
    "n1e7_v8192": _cfg(3, "n1e7_v8192", 4, 8192, 10_000_000, [ZIPF] * 4, [1.1] * 4, 512, 128, 32, "bf16"),
    "n1e7_v16384": _cfg(3, "n1e7_v16384", 4, 16384, 10_000_000, [ZIPF] * 4, [1.1] * 4, 512, 128, 32,
                     "bf16"),
    # dense-early catalog (100% / ~90% legal at steps 1 / 2), fp16 storage
    "n5e7_v1024_dense": _cfg(4, "n5e7_v1024_dense", 4, 1024, 50_000_000,
                        [UNIFORM, UNIFORM_SUBSET, ZIPF, ZIPF], [0.0, 0.9, 1.3, 1.3],
                        512, 256, 128, "f16"),
    # production scale, 1e8 items, sparse tables at the last two steps
    "n1e8_v16384": _cfg(5, "n1e8_v16384", 4, 16384, 100_000_000, [ZIPF] + [ZIPF] * 3, [1.1, 1.5, 1.5, 1.5],
                 1024, 256, 32, "f32", fmt=["D", "D", "S", "S"]),
}


def catalog(cfg: Config, n_threads: Optional[int] = None) -> np.ndarray:
    """The catalog as int32 [N, L]; row i is item i's SID (all rows distinct)."""
    out = np.empty((cfg.N, cfg.L), dtype=np.int32)
    kinds = np.asarray(cfg.kinds, dtype=np.int32)
    params = np.asarray(cfg.params, dtype=np.float64)
    r = lib().wl_catalog(cfg.N, cfg.L, cfg.V, kinds.ctypes.data, params.ctypes.data,
                         cfg.seed_cat, n_threads or _threads(), out.ctypes.data)
    if r < 0:
        raise ValueError("wl_catalog: bad arguments")
    return out


def _bits_array(dtype: str, shape):
    return np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)


def weights(cfg: Config, t: int):
    """W_t as (stored bits [V, d], widened float32 [V, d]); t is 1-based."""
    bits = _bits_array(cfg.dtype, (cfg.V, cfg.d))
    f32 = np.empty((cfg.V, cfg.d), dtype=np.float32)
    lib().wl_weights(cfg.seed_w, t, cfg.V, cfg.d, cfg.w_std, DTYPES[cfg.dtype], bits.ctypes.data,
                     f32.ctypes.data, _threads())
    return bits, f32


def hidden(cfg: Config, t: int, req: Sequence[int], prefix: np.ndarray, want_f32: bool = True,
           threads: Optional[int] = None):
    """Hidden vectors of M beams at step t (1-based).

    req: int64 [M] request ids; prefix: int32 [M, >= t-1] prefix tokens.
    threads: generator threads (default: the host's, at most 16).
    Returns (stored bits [M, d], widened float32 [M, d] or None).
    """
    req = np.ascontiguousarray(np.asarray(req, dtype=np.int64))
    M = req.shape[0]
    if prefix is None or prefix.size == 0:
        prefix = np.zeros((M, 1), dtype=np.int32)
    prefix = np.ascontiguousarray(prefix, dtype=np.int32)
    if prefix.shape[0] != M or (t > 1 and prefix.shape[1] < t - 1):
        raise ValueError("prefix shape")
    bits = _bits_array(cfg.dtype, (M, cfg.d))
    f32 = np.empty((M, cfg.d), dtype=np.float32) if want_f32 else None
    lib().wl_hidden(cfg.seed_h, t, M, req.ctypes.data, prefix.ctypes.data, prefix.shape[1], cfg.d,
                    cfg.h_std, DTYPES[cfg.dtype], bits.ctypes.data,
                    f32.ctypes.data if f32 is not None else None,
                    _threads() if threads is None else max(1, int(threads)))
    return bits, f32


def round_to(dtype: str, x: np.ndarray):
    """Round float32 values to bf16/f16: (bits uint16, widened float32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = np.empty(x.shape, dtype=np.uint16)
    f = np.empty(x.shape, dtype=np.float32)
    lib().wl_round(DTYPES[dtype], x.ctypes.data, x.size, bits.ctypes.data, f.ctypes.data)
    return bits, f


def perm(key: int, V: int, x: int) -> int:
    return int(lib().wl_perm(key, V, x))
