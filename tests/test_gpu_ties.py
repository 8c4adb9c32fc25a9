"""GPU parity under exact ties.

With every weight zero, every legal candidate of a beam scores the same; on a
catalog holding every SID of the product space, every row has all V tokens
legal, so every beam of a step carries the same cumulative score too, and the
selection is decided by the tie-break alone: beam rank, then slot.  The
returned items must then be the first K SIDs in lexicographic order (item ids
0..K-1), exactly as the oracle's decode returns them; no tolerance band
applies.  The 64-token case floods the request merge with 2048 tied keys,
more than the boundary-bin capacity, so the radix select over tied keys runs.
"""
import itertools

import numpy as np
import pytest

import gpu_util as gu
import sid_constrained_beam_amd as zgr
from workload import CONFIGS

pytestmark = pytest.mark.gpu


def product_sids(V, L):
    return np.array(list(itertools.product(range(V), repeat=L)), np.int32)


CASES = {
    # name: (V, L, K, B, d, dtype)
    "v16_l3_f32": (16, 3, 40, 3, 64, "f32"),
    "v16_l3_bf16": (16, 3, 40, 3, 64, "bf16"),
    "v64_l3_f32": (64, 3, 64, 2, 64, "f32"),
    # 64 requests of 64 beams over 256 tokens: the dense second step takes the
    # tiled full projection and its word-pruned selection, where all 512 word
    # keys of a request tie on the score and the radix select runs to the codes
    "v256_l2_f32_b64": (256, 2, 64, 64, 64, "f32"),
}


@pytest.mark.parametrize("fmt", ["D", "S"])
@pytest.mark.parametrize("proj", ["selective", "full"])
@pytest.mark.parametrize("name", list(CASES))
def test_exact_ties_follow_beam_then_slot(name, proj, fmt):
    import torch
    V, L, K, B, d, dtype = CASES[name]
    cfg = CONFIGS["n1e4_v256"].scaled(name=f"ties_{name}", L=L, V=V, N=V ** L, d=d, K=K, B=B,
                                      dtype=dtype, fmt=[fmt] * L)
    s = gu.Setup(cfg, sids=product_sids(V, L))
    want_fmt = zgr.ZGR_FMT_DENSE if fmt == "D" else zgr.ZGR_FMT_SPARSE
    assert all(st["fmt"] == want_fmt for st in s.stats)
    # every weight zero: the oracle and the GPU read the same (zero) values
    s.W_bits = [np.zeros_like(b) for b in s.W_bits]
    s.W_f32 = [np.zeros_like(w) for w in s.W_f32]
    s.W_dev = [torch.zeros_like(w) for w in s.W_dev]
    torch.cuda.synchronize()
    plan = s.plan(force=[proj] * L)
    item_t = torch.empty(B * K, dtype=torch.int64, device="cuda")
    sc_t = torch.empty(B * K, dtype=torch.float32, device="cuda")
    sid_t = torch.empty(B * K * L, dtype=torch.int32, device="cuda")
    zgr.zgr_decode(plan, s.hidden_source(0), K, item_t, sid_t, sc_t)
    if name == "v256_l2_f32_b64" and proj == "full" and fmt == "D":
        assert zgr.zgr_plan_request_path(plan, 2)[0] == zgr.ZGR_REQ_PRUNED
    items = item_t.cpu().numpy().reshape(B, K)
    sids = sid_t.cpu().numpy().reshape(B, K, L)
    scores = sc_t.cpu().numpy().reshape(B, K)
    expect = np.arange(K, dtype=np.int64)
    closed = -L * np.log(V)  # every step's legal-only log-prob is -ln V
    for q in range(B):
        assert np.array_equal(items[q], expect), (q, items[q][:12])
        # the product catalog was handed over in lexicographic order: item i is row i
        assert np.array_equal(sids[q], s.sids[:K])
        dec = s.oracle_decode(q)
        assert np.array_equal(dec.item, expect), (q, dec.item[:12])
        assert np.all(np.abs(scores[q] - closed) <= gu.TOL["f32"]), (q, scores[q][:4], closed)
        # all K final scores are bitwise equal: each beam ran the same fp32 operations
        assert np.all(scores[q] == scores[q][0])
