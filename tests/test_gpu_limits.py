"""GPU parity at the limits of the interface and in degenerate shapes: beam
width 1 and 1024, the largest codebook (65536 tokens: a first step with more
candidates per request than the request kernel's key array), the deepest SID
(L = 8; a relabelled copy fills all 64 bits of the packed prefix keys), the smallest and largest hidden sizes in every
storage type, more requests than compute units, and top_k < K.  Every step is
checked against the oracle on the GPU's own trajectory, and zgr_decode must
reproduce that trajectory."""
import numpy as np
import pytest

import gpu_util as gu
import sid_constrained_beam_amd as zgr
import workload
from workload import CONFIGS, UNIFORM, ZIPF

pytestmark = pytest.mark.gpu


def cfg_of(name, L, V, N, d, K, B, dtype, kinds=None, params=None, fmt=None):
    kinds = kinds or [ZIPF] * L
    params = params or [1.1] * L
    return CONFIGS["n1e4_v256"].scaled(name=name, L=L, V=V, N=N, d=d, K=K, B=B, dtype=dtype,
                                       kinds=kinds, params=params, fmt=fmt, seed_cat=4100 + L + V,
                                       seed_w=4200 + d, seed_h=4300 + K)


LIMITS = {
    "greedy_k1": cfg_of("greedy_k1", 3, 256, 10_000, 64, 1, 4, "f32"),
    "beam_1024": cfg_of("beam_1024", 3, 256, 120_000, 64, 1024, 2, "f32"),
    "codebook_65536": cfg_of("codebook_65536", 2, 65536, 150_000, 64, 16, 2, "f32",
                             kinds=[UNIFORM, ZIPF], params=[0.0, 1.1]),
    "depth_8": cfg_of("depth_8", 8, 128, 40_000, 64, 32, 3, "f32", kinds=[ZIPF] * 8,
                      params=[1.5] * 8),
    "hidden_4096_f32": cfg_of("hidden_4096_f32", 3, 512, 20_000, 4096, 16, 2, "f32"),
    "hidden_4096_bf16": cfg_of("hidden_4096_bf16", 3, 512, 20_000, 4096, 16, 2, "bf16"),
    "hidden_768_f16": cfg_of("hidden_768_f16", 3, 1024, 50_000, 768, 24, 3, "f16"),
    "batch_300": cfg_of("batch_300", 3, 128, 5_000, 64, 8, 300, "f32"),
    # 16-bit full projections on 128x128 tiles (8-wave blocks) with ragged edges: M = 32 * 125
    # beams and V not a multiple of the tile (nor of 32) at steps 2 and 3
    # (step 2 dense: legal-rank epilogue; step 3 sparse: slot epilogue)
    "ragged_tiles_bf16": cfg_of("ragged_tiles_bf16", 3, 2000, 300_000, 512, 125, 32, "bf16",
                                fmt=["D", "D", "S"]),
    "ragged_tiles_f16": cfg_of("ragged_tiles_f16", 3, 2100, 200_000, 256, 125, 32, "f16",
                               fmt=["D", "D", "S"]),
}

_setups = {}


def setup_of(name):
    if name not in _setups:
        print(f"[setup] {name}", flush=True)
        _setups[name] = gu.Setup(LIMITS[name])
    return _setups[name]


@pytest.mark.parametrize("proj", ["selective", "full", "staged"])
@pytest.mark.parametrize("name", list(LIMITS))
def test_limit_decode(name, proj):
    import torch
    s = setup_of(name)
    cfg = s.cfg
    B, K, L = cfg.B, cfg.K, cfg.L
    print(f"[limit] {name} {proj}", flush=True)
    plan = s.plan(force=[proj] * L)
    # the oracle checks every request at every step (a sample at batch 300)
    requests = list(range(B)) if B <= 8 else [0, 1, B // 2, B - 1]
    rows, sids, scores, amb = trajectory(s, plan, requests)
    top_k = max(1, K // 3)
    item_t = torch.empty(B * top_k, dtype=torch.int64, device="cuda")
    sid_t = torch.empty(B * top_k * L, dtype=torch.int32, device="cuda")
    sc_t = torch.empty(B * top_k, dtype=torch.float32, device="cuda")
    zgr.zgr_decode(plan, s.hidden_source(0), top_k, item_t, sid_t, sc_t)
    assert np.array_equal(item_t.cpu().numpy().reshape(B, top_k), rows[:, :top_k])
    assert np.array_equal(sid_t.cpu().numpy().reshape(B, top_k, L), sids[:, :top_k])
    assert np.array_equal(sc_t.cpu().numpy().reshape(B, top_k), scores[:, :top_k])
    members = set(map(tuple, s.sids.tolist()))
    for q in requests:
        live = rows[q] >= 0
        assert live.any()
        for it, sid in zip(rows[q][live], sids[q][live]):
            assert tuple(sid.tolist()) in members
            assert np.array_equal(s.sids[s.cat.input_row(int(it))], sid)
        dec = s.oracle_decode(q)
        if gu.oracle_unambiguous(dec, K, gu.TOL[cfg.dtype]):
            gu.assert_same_ranking(rows[q], dec.item, dec.score, gu.TOL[cfg.dtype], q)
    print(f"{name} {proj}: {amb} ambiguous request-steps")


def trajectory(s, plan, requests):
    """Step-by-step decode of all B requests, oracle-checked on `requests`."""
    cfg = s.cfg
    B, K, L = cfg.B, cfg.K, cfg.L
    tol = gu.TOL[cfg.dtype]
    prefixes = np.zeros((B, 0), np.int32)
    cum = np.zeros(B, np.float32)
    amb = 0
    out = None
    for t in range(1, L + 1):
        dbg = True if B * (1 if t == 1 else K) * max(cfg.V, 1) <= (1 << 26) else requests
        out = gu.run_gpu_step(s, plan, t, prefixes, cum, B, K, list(range(B)), with_dbg=dbg)
        amb += gu.check_step(s, t, prefixes, cum, out, B, K, tol, requests=requests)
        par = out["parent"]
        new = np.full((B * K, t), -1, np.int32)
        ok = par >= 0
        if t > 1:
            new[ok, : t - 1] = prefixes[par[ok]]
        new[ok, t - 1] = out["token"][ok]
        prefixes, cum = new, out["cum_out"]
    return out["row_out"].reshape(B, K), prefixes.reshape(B, K, L), cum.reshape(B, K), amb


@pytest.mark.parametrize("proj", ["selective", "full"])
def test_full_64_bit_prefix_keys(proj):
    """L = 8 at V = 256 fills all 64 bits of a packed prefix key (the oracle
    stops at 63).  Relabel the depth-8 catalog's tokens t -> 2t + 1 at V = 256,
    with weight rows W'[2t + 1] = W[t] and the same hidden vectors: the search
    is order-isomorphic, so the decode must equal the V = 128 decode exactly
    (item ids too: the map preserves lexicographic order)."""
    import torch
    s = setup_of("depth_8")
    cfg = s.cfg
    B, K, L = cfg.B, cfg.K, cfg.L
    sids2 = 2 * s.sids + 1
    assert sids2.max() >= 128
    idx2, _ = zgr.zgr_index_upload(sids2, 256, None)
    W2 = []
    for w in s.W_dev:
        big = torch.zeros((256, cfg.d), dtype=w.dtype, device="cuda")
        big[1::2] = w
        W2.append(big)
    plan2 = zgr.zgr_plan_warmup(idx2, W2, cfg.dtype, cfg.d, B, K, None, 0, [proj] * L)
    base = s.hidden_source(0)

    def hidden2(t, B_, k_in, prefix_ptr, prefix_ld, hidden_ptr, stream_ptr):
        # the same hidden vectors: hand the original tokens to the source
        M = B_ * k_in
        pre = np.empty((M, prefix_ld), np.int32)
        zgr.copy_to_host(pre, prefix_ptr, stream_ptr)
        orig = np.where(pre >= 0, (pre - 1) // 2, pre).astype(np.int32)
        zgr.copy_to_device(prefix_ptr, orig, stream_ptr)
        rc = base(t, B_, k_in, prefix_ptr, prefix_ld, hidden_ptr, stream_ptr)
        zgr.copy_to_device(prefix_ptr, pre, stream_ptr)
        return rc

    outs = []
    for plan, hid in ((s.plan(force=[proj] * L), s.hidden_source(0)), (plan2, hidden2)):
        item = torch.empty(B * K, dtype=torch.int64, device="cuda")
        sid = torch.empty(B * K * L, dtype=torch.int32, device="cuda")
        sc = torch.empty(B * K, dtype=torch.float32, device="cuda")
        zgr.zgr_decode(plan, hid, K, item, sid, sc)
        outs.append((item.cpu().numpy(), sid.cpu().numpy(), sc.cpu().numpy()))
    (i1, s1, c1), (i2, s2, c2) = outs
    assert np.array_equal(i1, i2) and np.array_equal(c1, c2)
    assert np.array_equal(np.where(s1 >= 0, 2 * s1 + 1, s1), s2)
    assert (i1 >= 0).any()


def test_limit_configs_are_extreme():
    """The cases really sit at the limits (guards against silent shrinking)."""
    s = setup_of("codebook_65536")
    assert s.stats[0]["stride"] == 65536 and s.stats[0]["fmt"] == zgr.ZGR_FMT_DENSE
    assert setup_of("beam_1024").cfg.K == 1024
    d8 = setup_of("depth_8")
    assert d8.cfg.L == 8
    # the ragged cases reach the 16-bit 128x128 tiles at steps 2 and 3, with partial edge tiles
    for name in ("ragged_tiles_bf16", "ragged_tiles_f16"):
        s = setup_of(name)
        M = s.cfg.B * s.cfg.K
        assert M % 128 and s.cfg.V % 128 and s.cfg.V % 32
        for t in (2, 3):
            var = zgr.zgr_full_projection_variant(M, s.cfg.V, s.cfg.dtype, s.stats[t - 1]["fmt"],
                                                  "filter_first")
            assert var[1:3] == (128, 128), (name, t, var)
