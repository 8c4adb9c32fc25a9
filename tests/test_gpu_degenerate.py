"""GPU behaviour in degenerate cases the method has.

A catalog of one item: every step has exactly one legal token, whose
legal-only log-probability is exactly 0 (the log-sum-exp of one score is the
score itself), so the one surviving beam scores exactly 0 and the other K-1
outputs are empty.  A step whose beams are all dead (row -1, cumulative
score -inf) emits nothing: every output is empty and no device error is
raised (a dead beam is a valid input, unlike a row outside the table).
"""
import numpy as np
import pytest

import gpu_util as gu
import sid_constrained_beam_amd as zgr
import workload
from workload import CONFIGS

pytestmark = pytest.mark.gpu

SID = [5, 2, 7]
V, L, K, B, D = 8, 3, 4, 2, 64


def single_item_plan(proj, fmt):
    cfg = CONFIGS["n1e4_v256"].scaled(V=V, L=L, N=1, d=D, K=K, B=B)
    index, _ = zgr.zgr_index_upload(np.array([SID], np.int32), V, [fmt] * L)
    W = [gu.to_device_bits(workload.weights(cfg, t)[0], "f32") for t in range(1, L + 1)]
    plan = zgr.zgr_plan_warmup(index, W, "f32", D, B, K, None, 0, [proj] * L)
    return index, W, plan


def hidden_fn(t, Bq, k_in, pp, ld, hp, sp):
    rng = np.random.default_rng(t)
    zgr.copy_to_device(hp, rng.standard_normal((Bq * k_in, D)).astype(np.float32), sp)
    return 0


@pytest.mark.parametrize("fmt", ["D", "S"])
@pytest.mark.parametrize("proj", ["selective", "full"])
def test_single_item_catalog(proj, fmt):
    import torch
    index, W, plan = single_item_plan(proj, fmt)
    item = torch.empty(B * K, dtype=torch.int64, device="cuda")
    sid = torch.empty(B * K * L, dtype=torch.int32, device="cuda")
    sc = torch.empty(B * K, device="cuda")
    zgr.zgr_decode(plan, hidden_fn, K, item, sid, sc)
    it = item.cpu().numpy().reshape(B, K)
    sd = sid.cpu().numpy().reshape(B, K, L)
    s = sc.cpu().numpy().reshape(B, K)
    for q in range(B):
        assert it[q].tolist() == [0] + [-1] * (K - 1)
        assert sd[q, 0].tolist() == SID and np.all(sd[q, 1:] == -1)
        assert s[q, 0] == 0.0  # exactly: one legal token per step
        assert np.all(np.isneginf(s[q, 1:]))


@pytest.mark.parametrize("proj", ["selective", "full"])
def test_all_dead_step(proj):
    import torch
    index, W, plan = single_item_plan(proj, "D")
    M = B * K
    hidden = torch.zeros(M, D, device="cuda")
    row_in = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    cum_in = torch.full((M,), float("-inf"), device="cuda")
    par, tok, row = (torch.zeros(M, dtype=torch.int32, device="cuda") for _ in range(3))
    cum = torch.zeros(M, device="cuda")
    zgr.zgr_step(plan, 2, hidden, row_in, cum_in, K, par, tok, row, cum)
    zgr.zgr_plan_status(plan)  # dead beams are valid input: no device error
    for x in (par, tok, row):
        assert np.all(x.cpu().numpy() == -1)
    assert np.all(np.isneginf(cum.cpu().numpy()))
