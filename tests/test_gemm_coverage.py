"""Every full-projection kernel that the benchmarks run at full size has a
GPU parity case (CPU only).

The library's own dispatch rule (zgr_full_projection_variant, shared with
its launcher) names the kernel, tile and epilogue of a step shape.  Required:
what bench.py can launch on the full-size workloads -- the full projection
of any step in filter-first decoding (the planner or a forced choice may pick
it anywhere), every step of the score-first and unconstrained comparisons,
and the next-row-matrix encoding of the dense steps.  Covered: the steps that
the oracle-checked GPU tests run (tests/cases.py).  A kernel variant that a
benchmark times but no parity test reaches fails this test.
"""
import functools

import pytest

import sid_constrained_beam_amd as zgr
import workload
from cases import (ENCODING_WORKLOADS, FULLSIZE, FULLSIZE_FMT, GEMM_CASES, MODE_CASES, NEXT_CASES,
                   PARITY_CASES, gemm_case_config)
from workload import CONFIGS

N_CU = 256  # MI355X
FMT = {"D": zgr.ZGR_FMT_DENSE, "S": zgr.ZGR_FMT_SPARSE, "N": zgr.ZGR_FMT_DENSE_NEXT}


def variant(cfg, t, fmt_char, mode):
    """(dtype, kernel, tile_m, tile_n, epilogue, next-row matrix) of step t."""
    M = cfg.B * (1 if t == 1 else cfg.K)
    kern, tm, tn, ep = zgr.zgr_full_projection_variant(M, cfg.V, cfg.dtype, FMT[fmt_char], mode, N_CU)
    # only the filter-first epilogues read the table (the comparison modes keep every column)
    nx = fmt_char == "N" and mode == "filter_first"
    return (cfg.dtype, kern, tm, tn, ep, nx)


@functools.lru_cache(maxsize=None)
def built_fmts(name, fmt=None):
    """Table formats of a reduced case as the host index builds them."""
    cfg = PARITY_CASES.get(name) or MODE_CASES[name]
    if fmt is not None:
        cfg = cfg.scaled(fmt=list(fmt))
    sids = workload.catalog(cfg)
    idx, _ = zgr.zgr_index_build_host(sids, cfg.V, cfg.fmt, want_rank=False)
    inv = {v: k for k, v in FMT.items()}
    out = "".join(inv[idx.stats(t)["fmt"]] for t in range(1, cfg.L + 1))
    idx.free()
    return out


def required():
    need = {}
    for name in FULLSIZE:
        cfg, fmts = CONFIGS[name], FULLSIZE_FMT[name]
        for t in range(1, cfg.L + 1):
            for mode in ("filter_first", "score_first", "unconstrained"):
                need.setdefault(variant(cfg, t, fmts[t - 1], mode), (name, t, mode))
            if name in ENCODING_WORKLOADS and fmts[t - 1] == "D":
                need.setdefault(variant(cfg, t, "N", "filter_first"), (name, t, "next-row matrix"))
    return need


def covered():
    have = set()
    for name, cfg in PARITY_CASES.items():
        fmts = built_fmts(name)
        for t in range(1, cfg.L + 1):
            have.add(variant(cfg, t, fmts[t - 1], "filter_first"))
    for name, fmt in NEXT_CASES.items():
        cfg = PARITY_CASES[name]
        fmts = built_fmts(name, "".join(fmt))
        for t in range(1, cfg.L + 1):
            have.add(variant(cfg, t, fmts[t - 1], "filter_first"))
    for name, cfg in MODE_CASES.items():
        fmts = built_fmts(name)
        for t in range(1, cfg.L + 1):
            for mode in ("score_first", "unconstrained"):
                have.add(variant(cfg, t, fmts[t - 1], mode))
    for _, name, over, t, mode in GEMM_CASES:
        cfg = gemm_case_config(name, over)
        if "fmt" in over:
            fmts = over["fmt"]
        else:
            assert "N" not in over, "a reduced GEMM case must fix its table formats"
            fmts = FULLSIZE_FMT[name]
        # the case forces the full projection at every step up to t and checks each
        for tt in range(1, t + 1):
            have.add(variant(cfg, tt, fmts[tt - 1], mode))
    return have


def test_every_benchmarked_gemm_variant_has_a_parity_case():
    need, have = required(), covered()
    missing = {v: where for v, where in need.items() if v not in have}
    assert not missing, "full-projection variants timed at full size without a parity case: " + \
        "; ".join(f"{v} (first at {w})" for v, w in sorted(missing.items()))


def test_variant_rule_rejects_bad_arguments():
    with pytest.raises(zgr.ZgrError):
        zgr.zgr_full_projection_variant(0, 1024, "f32", zgr.ZGR_FMT_DENSE, "filter_first")
    with pytest.raises(zgr.ZgrError):
        zgr.zgr_full_projection_variant(64, 1024, "f32", 7, "filter_first")
    with pytest.raises(zgr.ZgrError):
        zgr.zgr_full_projection_variant(64, 1024, "f32", zgr.ZGR_FMT_DENSE, 5)
