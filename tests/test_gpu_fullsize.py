"""GPU parity at the workloads' full sizes, in the planner-chosen launch
configuration that bench.py times.

The whole batch is decoded on the GPU; the oracle checks sampled requests:
every step of the GPU's own trajectory is checked teacher-forced (legal
slots bit-exact, log-probs within tolerance, selection by the band protocol,
next rows bit-exact), zgr_decode must reproduce that trajectory bit for bit,
and where the oracle's own decode meets no near-tie at a K-th boundary the
returned items must be identical.
"""
import time

import numpy as np
import pytest

import gpu_util as gu
import sid_constrained_beam_amd as zgr
from cases import FULLSIZE, FULLSIZE_FMT
from workload import CONFIGS

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

NAMES = FULLSIZE
FMT_CHAR = {zgr.ZGR_FMT_DENSE: "D", zgr.ZGR_FMT_SPARSE: "S", zgr.ZGR_FMT_DENSE_NEXT: "N"}


def log(*a):
    print(*a, flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", NAMES)
def test_fullsize_decode_parity(name):
    import torch
    cfg = CONFIGS[name]
    t0 = time.time()
    s = gu.Setup(cfg)
    log(f"[{name}] catalog, index, weights, oracle trie in {time.time() - t0:.1f}s")
    # the table formats the CPU coverage test assumes for this workload
    assert "".join(FMT_CHAR[st["fmt"]] for st in s.stats) == FULLSIZE_FMT[name]
    plan = s.plan(force=None, n_warmup=2)
    choices = [plan.choice(t)[0] for t in range(1, cfg.L + 1)]
    log(f"[{name}] planner: {choices}")
    B, K, L = cfg.B, cfg.K, cfg.L
    sample = sorted({0, B // 2, B - 1})
    tol = gu.TOL[cfg.dtype]
    # the GPU's own step-by-step trajectory, sampled requests checked per step
    prefixes = np.zeros((B, 0), np.int32)
    cum = np.zeros(B, np.float32)
    amb = 0
    out = None
    for t in range(1, L + 1):
        out = gu.run_gpu_step(s, plan, t, prefixes, cum, B, K, list(range(B)), with_dbg=sample)
        diag = {}
        amb += gu.check_step(s, t, prefixes, cum, out, B, K, tol, requests=sample, diag=diag)
        log(f"[{name}] step {t} diagnostics: max |dlogp| {diag['max_dlogp']:.3g}, max |dscore| "
            f"{diag['max_dscore']:.3g} (tolerance {tol:g}); at ten times the observed error "
            f"(band <= {diag['tight_band_max']:.3g}) {diag.get('tight_exact', 0)} of {len(sample)} "
            f"sampled requests picked exactly the oracle's set, "
            f"{diag.get('tight_ambiguous', 0)} had a boundary gap inside that band")
        par = out["parent"]
        new = np.full((B * K, t), -1, np.int32)
        ok = par >= 0
        if t > 1:
            new[ok, : t - 1] = prefixes[par[ok]]
        new[ok, t - 1] = out["token"][ok]
        prefixes, cum = new, out["cum_out"]
        log(f"[{name}] step {t} checked ({time.time() - t0:.1f}s)")
    items = out["row_out"].reshape(B, K)
    item_t = torch.empty(B * K, dtype=torch.int64, device="cuda")
    sc_t = torch.empty(B * K, dtype=torch.float32, device="cuda")
    zgr.zgr_decode(plan, s.hidden_source(0), K, item_t, None, sc_t)
    d_items = item_t.cpu().numpy().reshape(B, K)
    assert np.array_equal(d_items, items)
    assert np.array_equal(sc_t.cpu().numpy().reshape(B, K), cum.reshape(B, K))
    # every returned item is real: its id maps back to the SID the beam spelled
    for q in sample:
        live = d_items[q] >= 0
        assert live.all()
        for it, sid in zip(d_items[q], prefixes.reshape(B, K, L)[q]):
            assert np.array_equal(s.sids[s.cat.input_row(int(it))], sid)
    exact = 0
    for q in sample:
        dec = s.oracle_decode(q)
        from test_gpu_parity import oracle_unambiguous
        if oracle_unambiguous(dec, K, tol):
            exact += 1
            gu.assert_same_ranking(d_items[q], dec.item, dec.score, tol, q)
    log(f"[{name}] sampled requests {sample}: {exact} compared item-for-item, "
        f"{amb} ambiguous request-steps, {time.time() - t0:.1f}s")
