"""GPU parity of the comparison modes (score-first and unconstrained) with
the oracle's modes, on the same protocol as the filter-first path: exact
legal / candidate sets and rows, log-probs within tolerance, the band rule
for the selection, and item-for-item decodes where the oracle meets no
ambiguity."""
import numpy as np
import pytest

import gpu_util as gu
import sid_constrained_beam_amd as zgr
from cases import MODE_CASES

pytestmark = pytest.mark.gpu

CASES = MODE_CASES
MODES = ["score_first", "unconstrained"]

_setups = {}


def setup_of(name):
    if name not in _setups:
        print(f"[setup] {name}", flush=True)
        _setups[name] = gu.Setup(CASES[name])
    return _setups[name]


def mode_plan(s, mode):
    # the frozen per-step choice is irrelevant in these modes (every token is scored)
    plan = s.plan(force=["selective"] * s.cfg.L)
    zgr.zgr_plan_set_mode(plan, mode)
    assert zgr.zgr_plan_mode(plan) == mode
    return plan


def oracle_inputs(s, requests, t, mode):
    cfg = s.cfg
    k_in = 1 if t == 1 else cfg.K
    prefixes = np.zeros((len(requests) * k_in, max(t - 1, 0)), np.int32)
    cum = np.full(len(requests) * k_in, -np.inf, np.float32)
    for qi, r in enumerate(requests):
        st = s.oracle_decode(r, mode=mode).steps[t - 1]
        n = len(st["cum"])
        prefixes[qi * k_in: qi * k_in + n] = st["prefix"]
        cum[qi * k_in: qi * k_in + n] = st["cum"].astype(np.float32)
    return prefixes, cum


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", list(CASES))
def test_mode_step_parity(name, mode):
    s = setup_of(name)
    cfg = s.cfg
    print(f"[mode step] {name} {mode}", flush=True)
    plan = mode_plan(s, mode)
    requests = list(range(cfg.B))
    amb = 0
    for t in range(1, cfg.L + 1):
        prefixes, cum = oracle_inputs(s, requests, t, mode)
        out = gu.run_gpu_step(s, plan, t, prefixes, cum, cfg.B, cfg.K, requests, mode=mode)
        amb += gu.check_step(s, t, prefixes, cum, out, cfg.B, cfg.K, gu.TOL[cfg.dtype], mode=mode)
    print(f"{name} {mode}: ambiguous request-steps {amb}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", list(CASES))
def test_mode_decode_parity(name, mode):
    import torch
    s = setup_of(name)
    cfg = s.cfg
    B, K, L = cfg.B, cfg.K, cfg.L
    print(f"[mode decode] {name} {mode}", flush=True)
    plan = mode_plan(s, mode)
    rows, sids, scores, amb = gu.gpu_trajectory(s, plan, list(range(B)), mode=mode)
    item_t = torch.empty(B * K, dtype=torch.int64, device="cuda")
    sid_t = torch.empty(B * K * L, dtype=torch.int32, device="cuda")
    sc_t = torch.empty(B * K, dtype=torch.float32, device="cuda")
    zgr.zgr_decode(plan, s.hidden_source(0), K, item_t, sid_t, sc_t)
    d_items = item_t.cpu().numpy().reshape(B, K)
    d_sids = sid_t.cpu().numpy().reshape(B, K, L)
    d_scores = sc_t.cpu().numpy().reshape(B, K)
    # the decode reproduces the step-by-step trajectory
    assert np.array_equal(d_sids, sids)
    assert np.array_equal(d_scores, scores)
    live = np.isfinite(scores)
    if mode == "unconstrained":
        # item ids by catalog lookup: the oracle's node numbering, -1 off-catalog
        want = np.array([[s.cat.node(sids[q, k]) if live[q, k] else -1 for k in range(K)]
                         for q in range(B)])
        assert np.array_equal(d_items, want)
    else:
        assert np.array_equal(d_items, rows)
        assert np.all(d_items[live] >= 0)
    tol = gu.TOL[cfg.dtype]
    exact = 0
    for q in range(B):
        dec = s.oracle_decode(q, mode=mode)
        if gu.oracle_unambiguous(dec, K, tol):
            exact += 1
            # codes by SID (off-catalog codes share the item id -1), each with its item id
            n = int(live[q].sum())
            gu.assert_same_ranking([(int(i),) + tuple(c) for i, c in zip(d_items[q], d_sids[q])],
                                   [(int(i),) + tuple(c) for i, c in zip(dec.item, dec.sid)],
                                   dec.score, tol, q)
            assert np.allclose(np.sort(d_scores[q][:n]), np.sort(dec.score[:n]), atol=tol * L, rtol=0)
    off = int(((d_items < 0) & live).sum())
    print(f"{name} {mode}: {exact}/{B} requests item-for-item, {amb} ambiguous request-steps, "
          f"{off} off-catalog codes")


def test_mode_switch_round_trip():
    """Switching modes on one plan and back leaves filter-first results unchanged."""
    import torch
    s = setup_of("n1e6_v2048_small")
    cfg = s.cfg
    plan = s.plan(force=["full", "full", "selective"])
    outs = []
    for mode in ("filter_first", "unconstrained", "score_first", "filter_first"):
        zgr.zgr_plan_set_mode(plan, mode)
        item = torch.empty(cfg.B * cfg.K, dtype=torch.int64, device="cuda")
        sc = torch.empty(cfg.B * cfg.K, dtype=torch.float32, device="cuda")
        zgr.zgr_decode(plan, s.hidden_source(0), cfg.K, item, None, sc)
        outs.append((item.cpu().numpy(), sc.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[3][0]) and np.array_equal(outs[0][1], outs[3][1])
    with pytest.raises(zgr.ZgrError):
        zgr.zgr_plan_set_mode(plan, 7)
