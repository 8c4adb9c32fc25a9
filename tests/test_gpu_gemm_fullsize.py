"""GPU parity of the full-projection kernels at the sizes the benchmarks run
them (tests/cases.py GEMM_CASES; tests/test_gemm_coverage.py checks that every
kernel variant a benchmark times at full size is among them).

Each case forces the full projection at every step of its mode's decode up
to the listed step and runs the GPU's own trajectory over the whole batch;
every step is checked against the oracle, teacher-forced, on sampled requests
{0, B/2, B-1} (legal slots bit-exact, log-probs within tolerance, selection
by the band protocol, next rows bit-exact), with the observed error and the
tight-band selection check of gpu_util.check_step reported beside it.
"""
import time

import numpy as np
import pytest

import gpu_util as gu
import sid_constrained_beam_amd as zgr
from cases import GEMM_CASES, gemm_case_config

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

N_CU = 256

# Steps whose request kernel must take the word-pruned path (dense rows after
# the tiled full projection, many candidates per kept-word bound), and one
# dense full step that must not (V = 4096: too many words per thread).
PRUNED = {("v2048_t2_dense", 2), ("v2048_t2_next", 2), ("dense_t2_next", 2), ("dense_t3_slot", 2)}
NOT_PRUNED = {("v4096_t2_dense", 2)}


def log(*a):
    print(*a, flush=True)


_setup = {}


def setup_of(name, over):
    key = (name, tuple(sorted(over.items())))
    if key not in _setup:
        _setup.clear()  # one full-size workload in memory at a time
        _setup[key] = gu.Setup(gemm_case_config(name, over))
    return _setup[key]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("label,name,over,t_last,mode", GEMM_CASES, ids=[c[0] for c in GEMM_CASES])
def test_full_projection_at_size(label, name, over, t_last, mode):
    t0 = time.time()
    s = setup_of(name, over)
    cfg = s.cfg
    B, K, L = cfg.B, cfg.K, cfg.L
    log(f"[{label}] {cfg.name} {over} ready in {time.time() - t0:.1f}s")
    plan = s.plan(force=["full"] * L)
    zgr.zgr_plan_set_mode(plan, mode)
    sample = sorted({0, B // 2, B - 1})
    tol = gu.TOL[cfg.dtype]
    prefixes = np.zeros((B, 0), np.int32)
    cum = np.zeros(B, np.float32)
    for t in range(1, t_last + 1):
        st = s.stats[t - 1]
        M = B * (1 if t == 1 else K)
        fmt = st["fmt"] if mode == "filter_first" else zgr.ZGR_FMT_DENSE
        var = zgr.zgr_full_projection_variant(M, cfg.V, cfg.dtype, fmt, mode, N_CU)
        out = gu.run_gpu_step(s, plan, t, prefixes, cum, B, K, list(range(B)), with_dbg=sample,
                              mode=mode)
        kind, parts = zgr.zgr_plan_request_path(plan, t)
        if (label, t) in PRUNED:
            assert kind == zgr.ZGR_REQ_PRUNED, (label, t, kind)
        if (label, t) in NOT_PRUNED:
            assert kind == zgr.ZGR_REQ_SLOT, (label, t, kind)
        diag = {}
        amb = gu.check_step(s, t, prefixes, cum, out, B, K, tol, requests=sample, mode=mode,
                            diag=diag)
        log(f"[{label}] step {t} M={M} kernel {var} request {kind}x{parts}: ambiguous {amb}/{len(sample)}, max |dlogp| "
            f"{diag['max_dlogp']:.3g}, max |dscore| {diag['max_dscore']:.3g} (tol {tol:g}); "
            f"tight band {diag['tight_band_max']:.3g}: {diag.get('tight_exact', 0)} exact, "
            f"{diag.get('tight_ambiguous', 0)} ambiguous ({time.time() - t0:.1f}s)")
        par = out["parent"]
        new = np.full((B * K, t), -1, np.int32)
        ok = par >= 0
        if t > 1:
            new[ok, : t - 1] = prefixes[par[ok]]
        new[ok, t - 1] = out["token"][ok]
        prefixes, cum = new, out["cum_out"]
    plan.free()
