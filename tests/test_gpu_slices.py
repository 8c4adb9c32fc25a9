"""GPU parity of the sliced selective projection: sparse tables that carry a
slice directory (per row, its legal tokens below each eighth of the codebook)
are scored by XCD-sliced work lists.  Each case runs with the directory forced
on and forced off, teacher-forced steps and whole decodes, against the oracle
(protocol in gpu_util)."""
import numpy as np
import pytest

import gpu_util as gu
import sid_constrained_beam_amd as zgr
from workload import CONFIGS

pytestmark = pytest.mark.gpu


def _long_rows(V, n1, per_row, L3, seed):
    """Three-level catalog with n1 first tokens, per_row second tokens each
    (long sparse rows at step 2) and L3 third tokens per 2-prefix."""
    rng = np.random.default_rng(seed)
    out = []
    for f in rng.choice(V, n1, replace=False):
        for s2 in rng.choice(V, per_row, replace=False):
            for s3 in rng.choice(V, L3, replace=False):
                out.append((f, s2, s3))
    return np.asarray(out, np.int32)


# (config, catalog or None, table formats): sparse steps with long rows, V
# not a multiple of 8, rows that leave slices empty, every storage type
CASES = {
    "n1e7_v16384_small": (CONFIGS["n1e7_v16384"].scaled(N=300_000, B=3, K=24), None),
    "n1e6_v2048_sparse": (CONFIGS["n1e6_v2048"].scaled(N=200_000, B=4, K=32, fmt=["D", "S", "S"]), None),
    "long_v5000_f16": (CONFIGS["n1e4_v256"].scaled(V=5000, L=3, N=0, d=128, K=40, B=3, dtype="f16",
                                                  fmt=["S", "S", "S"]),
                       lambda: _long_rows(5000, 24, 700, 2, 11)),
    "long_v4100_bf16": (CONFIGS["n1e4_v256"].scaled(V=4100, L=3, N=0, d=512, K=64, B=2, dtype="bf16",
                                                   fmt=["S", "S", "S"]),
                        lambda: _long_rows(4100, 6, 3000, 1, 12)),
}

_setups = {}


def setup_of(name, slices):
    key = (name, slices)
    if key not in _setups:
        cfg, make = CASES[name]
        sids = None if make is None else make()
        if sids is not None:
            cfg = cfg.scaled(N=len(sids))
        print(f"[setup] {name} slices={slices}", flush=True)
        _setups[key] = gu.Setup(cfg, sids=sids, slices=slices)
    return _setups[key]


def oracle_inputs(s, requests, t):
    cfg = s.cfg
    k_in = 1 if t == 1 else cfg.K
    prefixes = np.zeros((len(requests) * k_in, max(t - 1, 0)), np.int32)
    cum = np.full(len(requests) * k_in, -np.inf, np.float32)
    for qi, r in enumerate(requests):
        st = s.oracle_decode(r).steps[t - 1]
        n = len(st["cum"])
        prefixes[qi * k_in: qi * k_in + n] = st["prefix"]
        cum[qi * k_in: qi * k_in + n] = st["cum"].astype(np.float32)
    return prefixes, cum


@pytest.mark.parametrize("slices", ["always", "never"])
@pytest.mark.parametrize("name", list(CASES))
def test_sliced_step_parity(name, slices):
    s = setup_of(name, slices)
    cfg = s.cfg
    sparse = [t for t in range(1, cfg.L + 1) if s.stats[t - 1]["fmt"] == zgr.ZGR_FMT_SPARSE]
    assert sparse
    for t in sparse:
        assert s.stats[t - 1]["slice_dir"] == (1 if slices == "always" else 0)
    plan = s.plan(force=["selective"] * cfg.L)
    requests = list(range(cfg.B))
    amb = 0
    for t in range(1, cfg.L + 1):
        prefixes, cum = oracle_inputs(s, requests, t)
        out = gu.run_gpu_step(s, plan, t, prefixes, cum, cfg.B, cfg.K, requests)
        amb += gu.check_step(s, t, prefixes, cum, out, cfg.B, cfg.K, gu.TOL[cfg.dtype])
    print(f"{name} slices={slices}: ambiguous request-steps {amb}")


@pytest.mark.parametrize("name", list(CASES))
def test_sliced_decode_parity(name):
    s = setup_of(name, "always")
    cfg = s.cfg
    plan = s.plan(force=["selective"] * cfg.L)
    requests = list(range(cfg.B))
    items, sids, scores, amb = gu.gpu_trajectory(s, plan, requests)
    tol = gu.TOL[cfg.dtype]
    exact = 0
    for q in requests:
        dec = s.oracle_decode(q)
        if gu.oracle_unambiguous(dec, cfg.K, tol):
            exact += 1
            gu.assert_same_ranking(items[q], dec.item, dec.score, tol, q)
    print(f"{name}: {exact}/{cfg.B} requests compared item-for-item, {amb} ambiguous request-steps")
