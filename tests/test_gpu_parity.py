"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Workloads are the seeded synthetic catalogs at sizes the oracle finishes in
seconds (several kernel tiles, ragged tails); the full-size catalogs are in
test_gpu_fullsize.py.  See gpu_util for the protocol.
"""
import json
import os

import numpy as np
import pytest

import gpu_util as gu
import sid_constrained_beam_amd as zgr
import workload
from cases import NEXT_CASES, PARITY_CASES
from workload import CONFIGS

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Reduced versions of every precision / table-format mix (tests/cases.py).
CASES = PARITY_CASES

_setups = {}


def setup_of(name):
    if name not in _setups:
        print(f"[setup] {name}", flush=True)
        _setups[name] = gu.Setup(CASES[name])
    return _setups[name]


def oracle_inputs(s, requests, t):
    """Teacher-forced inputs of step t: each request's oracle beams."""
    cfg = s.cfg
    k_in = 1 if t == 1 else cfg.K
    B = len(requests)
    prefixes = np.zeros((B * k_in, max(t - 1, 0)), np.int32)
    cum = np.full(B * k_in, -np.inf, np.float32)
    for qi, r in enumerate(requests):
        dec = s.oracle_decode(r)
        st = dec.steps[t - 1]
        n = len(st["cum"])
        prefixes[qi * k_in: qi * k_in + n] = st["prefix"]
        cum[qi * k_in: qi * k_in + n] = st["cum"].astype(np.float32)
    return prefixes, cum


@pytest.mark.parametrize("proj", ["selective", "full", "naive", "staged"])
@pytest.mark.parametrize("name", list(CASES))
def test_step_parity_teacher_forced(name, proj):
    s = setup_of(name)
    cfg = s.cfg
    plan = s.plan(force=[proj] * cfg.L)
    requests = list(range(cfg.B))
    tol = gu.TOL[cfg.dtype]
    amb = 0
    for t in range(1, cfg.L + 1):
        prefixes, cum = oracle_inputs(s, requests, t)
        # oracle cumulative scores enter as float32 on both sides
        out = gu.run_gpu_step(s, plan, t, prefixes, cum, cfg.B, cfg.K, requests)
        amb += gu.check_step(s, t, prefixes, cum, out, cfg.B, cfg.K, tol)
    print(f"{name} {proj}: ambiguous request-steps {amb}")


gpu_trajectory = gu.gpu_trajectory
oracle_unambiguous = gu.oracle_unambiguous


@pytest.mark.parametrize("proj", ["selective", "full", "model", "naive"])
@pytest.mark.parametrize("name", list(CASES))
def test_decode_parity(name, proj):
    import torch
    s = setup_of(name)
    cfg = s.cfg
    B, K, L = cfg.B, cfg.K, cfg.L
    plan = s.plan(force=None if proj == "model" else [proj] * L)
    requests = list(range(B))
    items, sids, scores, amb = gpu_trajectory(s, plan, requests)
    # zgr_decode reproduces the step-by-step trajectory bit for bit
    item_t = torch.empty(B * K, dtype=torch.int64, device="cuda")
    sid_t = torch.empty(B * K * L, dtype=torch.int32, device="cuda")
    sc_t = torch.empty(B * K, dtype=torch.float32, device="cuda")
    zgr.zgr_decode(plan, s.hidden_source(0), K, item_t, sid_t, sc_t)
    d_items = item_t.cpu().numpy().reshape(B, K)
    assert np.array_equal(d_items, items)
    assert np.array_equal(sid_t.cpu().numpy().reshape(B, K, L), sids)
    assert np.array_equal(sc_t.cpu().numpy().reshape(B, K), scores)
    members = set(map(tuple, s.sids.tolist()))
    tol = gu.TOL[cfg.dtype]
    exact = 0
    for q in range(B):
        live = d_items[q] >= 0
        for it, sid in zip(d_items[q][live], sids[q][live]):
            assert tuple(sid.tolist()) in members  # a real catalog item
            assert np.array_equal(s.sids[s.cat.input_row(int(it))], sid)
        dec = s.oracle_decode(q)
        if oracle_unambiguous(dec, K, tol):
            exact += 1
            gu.assert_same_ranking(d_items[q], dec.item, dec.score, tol, q)
            assert np.allclose(sc_t.cpu().numpy().reshape(B, K)[q][live], dec.score[live], atol=tol * L, rtol=0)
    print(f"{name} {proj}: {exact}/{B} requests compared item-for-item, {amb} ambiguous request-steps")


def test_decode_deterministic():
    import torch
    s = setup_of("n1e6_v2048")
    cfg = s.cfg
    outs = []
    for proj in ("selective", "selective", "full", "full"):
        plan = s.plan(force=[proj] * cfg.L)
        item_t = torch.empty(cfg.B * cfg.K, dtype=torch.int64, device="cuda")
        sc_t = torch.empty(cfg.B * cfg.K, dtype=torch.float32, device="cuda")
        zgr.zgr_decode(plan, s.hidden_source(0), cfg.K, item_t, None, sc_t)
        outs.append((item_t.cpu().numpy(), sc_t.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(outs[2][0], outs[3][0]) and np.array_equal(outs[2][1], outs[3][1])


def test_slot_layout_golden():
    """Padded-slot sidebar: A has 1 legal token, B has 3; stride 3, 6 slots,
    B's first candidate in flat slot 3, A's slots 1-2 at -inf."""
    import torch
    g = json.load(open(os.path.join(GOLDEN, "slot_example.json")))
    cfg = CONFIGS["n1e4_v256"].scaled(V=g["V"], L=2, N=len(g["catalog"]), d=64, K=4, B=1)
    sids = np.array(g["catalog"], np.int32)
    index, _ = zgr.zgr_index_upload(sids, cfg.V, ["D", "S"])
    assert index.stats(2)["stride"] == g["slot_stride"]
    W = [gu.to_device_bits(workload.weights(cfg, t)[0], "f32") for t in (1, 2)]
    for proj in ("selective", "full"):
        plan = zgr.zgr_plan_warmup(index, W, "f32", 64, 1, 4, None, 0, [proj, proj])
        hidden = torch.randn(2, 64, device="cuda") * 0.125
        row_in = torch.tensor([0, 1], dtype=torch.int32, device="cuda")  # rows of prefixes (0), (1)
        cum_in = torch.tensor([-0.5, -0.25], device="cuda")
        dbg = torch.empty(2 * 3, device="cuda")
        outs = [torch.empty(4, dtype=dt, device="cuda") for dt in (torch.int32,) * 3 + (torch.float32,)]
        zgr.zgr_step(plan, 2, hidden, row_in, cum_in, 2, *outs, dbg)
        zgr.zgr_plan_status(plan)
        d = dbg.cpu().numpy()
        assert d.size == g["total_slots"]
        assert np.isfinite(d[0]) and d[0] == 0.0  # A's single legal token: log 1
        assert all(np.isneginf(d[j]) for j in g["empty_slots_of_A"])
        assert np.all(np.isfinite(d[g["first_slot_of_B"]:]))
        assert abs(np.log(np.exp(d[3:].astype(np.float64)).sum())) < 1e-6
        par, tok, row, cum = [o.cpu().numpy() for o in outs]
        assert sorted(zip(par.tolist(), tok.tolist())) == [(0, 2), (1, 0), (1, 1), (1, 3)]
        # next rows: lexicographic ranks of (0,2),(1,0),(1,1),(1,3) = 0,1,2,3
        assert dict(zip(zip(par.tolist(), tok.tolist()), row.tolist())) == {(0, 2): 0, (1, 0): 1, (1, 1): 2, (1, 3): 3}


def test_fewer_candidates_than_beam_and_dead_beams():
    import torch
    sids = np.array([[0, 1], [0, 2], [3, 3]], np.int32)
    cfg = CONFIGS["n1e4_v256"].scaled(V=4, L=2, N=3, d=64, K=8, B=2)
    index, rank = zgr.zgr_index_upload(sids, 4)
    W = [gu.to_device_bits(workload.weights(cfg, t)[0], "f32") for t in (1, 2)]
    for proj in ("selective", "full"):
        plan = zgr.zgr_plan_warmup(index, W, "f32", 64, 2, 8, None, 0, [proj, proj])
        item = torch.empty(2 * 8, dtype=torch.int64, device="cuda")
        sid = torch.empty(2 * 8 * 2, dtype=torch.int32, device="cuda")
        sc = torch.empty(2 * 8, device="cuda")

        def hid(t, B, k_in, pp, ld, hp, sp):
            zgr.copy_to_device(hp, np.full((B * k_in, 64), 0.01, np.float32), sp)
            return 0
        zgr.zgr_decode(plan, hid, 8, item, sid, sc)
        it = item.cpu().numpy().reshape(2, 8)
        for q in range(2):
            assert sorted(it[q, :3].tolist()) == [0, 1, 2]
            assert it[q, 3:].tolist() == [-1] * 5
            assert np.all(np.isneginf(sc.cpu().numpy().reshape(2, 8)[q, 3:]))
            assert np.all(sid.cpu().numpy().reshape(2, 8, 2)[q, 3:] == -1)


def test_row_out_of_range_sets_device_flag():
    import torch
    s = setup_of("n1e4_v256")
    cfg = s.cfg
    plan = s.plan(force=["selective"] * cfg.L)
    hidden = torch.zeros(cfg.K, cfg.d, device="cuda")
    row_in = torch.full((cfg.K,), 10 ** 8, dtype=torch.int32, device="cuda")
    cum_in = torch.zeros(cfg.K, device="cuda")
    outs = [torch.empty(cfg.K, dtype=dt, device="cuda") for dt in (torch.int32,) * 3 + (torch.float32,)]
    zgr.zgr_step(plan, 2, hidden, row_in, cum_in, cfg.K, *outs)
    with pytest.raises(zgr.ZgrError) as e:
        zgr.zgr_plan_status(plan)
    assert e.value.status == zgr.ZGR_E_DEVICE
    assert np.all(outs[0].cpu().numpy() == -1)  # every beam treated as dead
    zgr.zgr_plan_status(plan)  # flag cleared


def test_planner_warmup_freezes_a_choice():
    import torch
    s = setup_of("n1e6_v2048")
    cfg = s.cfg
    plan = s.plan(force=None, n_warmup=3)
    for t in range(1, cfg.L + 1):
        proj, uf, us = plan.choice(t)
        assert proj in (zgr.ZGR_PROJ_FULL, zgr.ZGR_PROJ_SELECTIVE)
        assert uf > 0 and us > 0
        assert proj == (zgr.ZGR_PROJ_FULL if uf < us else zgr.ZGR_PROJ_SELECTIVE)
        print(f"step {t}: full {uf:.1f} us, selective {us:.1f} us -> {'full' if proj == 1 else 'selective'}")
    # a forced step is never timed
    p2 = s.plan(force=["selective", None, "full"], n_warmup=1)
    assert p2.choice(1)[0] == zgr.ZGR_PROJ_SELECTIVE and p2.choice(1)[1] < 0
    assert p2.choice(3)[0] == zgr.ZGR_PROJ_FULL
    # a frozen plan can be re-frozen from exported choices
    zgr.zgr_plan_set_choice(p2, 2, "full")
    assert p2.choice(2)[0] == zgr.ZGR_PROJ_FULL
    item = torch.empty(cfg.B * cfg.K, dtype=torch.int64, device="cuda")
    zgr.zgr_decode(plan, s.hidden_source(0), cfg.K, item)
    assert int((item >= 0).sum()) == cfg.B * cfg.K


def test_stale_plan_rejected():
    import torch
    s = setup_of("n1e4_v256")
    cfg = s.cfg
    index, _ = zgr.zgr_index_upload(s.sids, cfg.V)
    plan = zgr.zgr_plan_warmup(index, s.W_dev, cfg.dtype, cfg.d, cfg.B, cfg.K, None, 0, None)
    index.free()
    item = torch.empty(cfg.B * cfg.K, dtype=torch.int64, device="cuda")
    with pytest.raises(zgr.ZgrError) as e:
        zgr.zgr_decode(plan, s.hidden_source(0), cfg.K, item)
    assert e.value.status == zgr.ZGR_E_STATE


def test_callback_failure_reported():
    import torch
    s = setup_of("n1e4_v256")
    cfg = s.cfg
    plan = s.plan(force=["selective"] * cfg.L)
    item = torch.empty(cfg.B * cfg.K, dtype=torch.int64, device="cuda")
    with pytest.raises(zgr.ZgrError) as e:
        zgr.zgr_decode(plan, lambda *a: 3, cfg.K, item)
    assert e.value.status == zgr.ZGR_E_CALLBACK


def test_profiled_launches_keep_results():
    """Timing mode repeats each (idempotent) launch between events: the decode's
    results are unchanged and every step records its kernels."""
    import torch
    s = setup_of("n1e6_v2048")
    cfg = s.cfg
    plan = s.plan(force=["full", "full", "selective"])
    outs = []
    for repeat in (0, 3):
        zgr.zgr_plan_profile(plan, repeat)
        item = torch.empty(cfg.B * cfg.K, dtype=torch.int64, device="cuda")
        sc = torch.empty(cfg.B * cfg.K, dtype=torch.float32, device="cuda")
        zgr.zgr_decode(plan, s.hidden_source(0), cfg.K, item, None, sc)
        outs.append((item.cpu().numpy(), sc.cpu().numpy()))
        if repeat:
            for t in range(1, cfg.L + 1):
                n, ms = zgr.zgr_plan_profile_read(plan, "request", t)
                assert n >= 1 and ms > 0
            assert zgr.zgr_plan_profile_read(plan, "gemm", 1)[0] == 1
            assert zgr.zgr_plan_profile_read(plan, "gemm", 3)[0] == 0
    zgr.zgr_plan_profile(plan, 0)
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    with pytest.raises(zgr.ZgrError):
        zgr.zgr_plan_profile(plan, -1)


def test_naive_baseline_matches_padded_slots():
    """The compaction baseline scores the same candidates as the padded-slot
    selective path: identical legal sets and selections, scores equal up to
    the summation order (both reduce the same products over one weight row)."""
    import torch
    s = setup_of("n1e6_v2048")
    cfg = s.cfg
    outs = {}
    for proj in ("selective", "naive"):
        plan = s.plan(force=[proj] * cfg.L)
        item = torch.empty(cfg.B * cfg.K, dtype=torch.int64, device="cuda")
        sc = torch.empty(cfg.B * cfg.K, dtype=torch.float32, device="cuda")
        zgr.zgr_decode(plan, s.hidden_source(0), cfg.K, item, None, sc)
        outs[proj] = (item.cpu().numpy(), sc.cpu().numpy())
        assert plan.choice(2)[0] == zgr.PROJ_CODES[proj]
    same = np.mean(outs["selective"][0] == outs["naive"][0])
    assert same > 0.99, same
    ok = np.isfinite(outs["selective"][1])
    assert np.allclose(outs["selective"][1][ok], outs["naive"][1][ok], atol=1e-4, rtol=0)


@pytest.mark.parametrize("proj", ["selective", "full", "staged"])
@pytest.mark.parametrize("name", list(NEXT_CASES))
def test_next_row_matrix_encoding(name, proj):
    """Dense steps stored as an int32 next-row matrix instead of the bitmap:
    every step passes the oracle check, and the outputs equal the bitmap
    encoding's bit for bit (only the table decode differs)."""
    import torch
    base = setup_of(name)
    cfg = base.cfg.scaled(fmt=NEXT_CASES[name])
    s = gu.Setup(cfg)
    for t in range(1, cfg.L + 1):
        want = zgr.ZGR_FMT_DENSE_NEXT if cfg.fmt[t - 1] == "N" else zgr.ZGR_FMT_SPARSE
        assert s.stats[t - 1]["fmt"] == want
    plan = s.plan(force=[proj] * cfg.L)
    gu.gpu_trajectory(s, plan, list(range(cfg.B)))
    bitmap = gu.Setup(cfg.scaled(fmt=["D" if f == "N" else f for f in cfg.fmt]), with_oracle=False)
    outs = []
    for setup in (s, bitmap):
        p = setup.plan(force=[proj] * cfg.L)
        item = torch.empty(cfg.B * cfg.K, dtype=torch.int64, device="cuda")
        sc = torch.empty(cfg.B * cfg.K, dtype=torch.float32, device="cuda")
        zgr.zgr_decode(p, setup.hidden_source(0), cfg.K, item, None, sc)
        outs.append((item.cpu().numpy(), sc.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
