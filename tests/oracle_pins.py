"""Checks that pin the CPU oracle to facts fixed outside itself.

Each pin compares the oracle against something that does not reuse its code:
the worked example and the padded-slot illustration of the ZeroGR page,
brute force with numpy/scipy, closed forms, and a textbook beam search on a
catalog that holds every SID (where constrained and unconstrained search
coincide).  ``test_oracle.py`` runs them; ``test_oracle_mutations.py`` runs
them against deliberately broken builds of the oracle and expects each build
to fail at least one.

Run as a script (``python tests/oracle_pins.py``) it executes every pin and
exits with the number that failed, printing their names.
"""
import json
import math
import os
import sys
import traceback

import numpy as np
from scipy.special import log_softmax, logsumexp

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workload  # noqa: E402

GOLDEN = os.path.join(HERE, "golden")


def small_cfg(V, d, L=3, N=60, K=4, seed=7):
    base = workload.CONFIGS["n1e4_v256"]
    return base.scaled(V=V, d=d, L=L, N=N, K=K, kinds=[workload.UNIFORM] * L, params=[0.0] * L,
                       seed_cat=100 + seed, seed_w=200 + seed, seed_h=300 + seed)


def random_catalog(V, L, N, seed):
    rng = np.random.default_rng(seed)
    seen = set()
    rows = []
    while len(rows) < N:
        s = tuple(int(x) for x in rng.integers(0, V, size=L))
        if s not in seen:
            seen.add(s)
            rows.append(s)
    return np.array(rows, dtype=np.int32)


def hidden_fn(cfg):
    def fn(request, t, prefixes):
        k = prefixes.shape[0]
        return workload.hidden(cfg, t, np.full(k, request, np.int64), prefixes)[1]
    return fn


def weights_of(cfg):
    return [workload.weights(cfg, t)[1] for t in range(1, cfg.L + 1)]


# --------------------------------------------------------------------------- pins

def pin_worked_example():
    """ZeroGR page, 'what problem': only 3-5-1 and 3-5-4 start with 3-5 -> legal {1, 4}."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    cat = oracle.Catalog(np.array(g["catalog"], dtype=np.int32), g["V"])
    for q in g["queries"]:
        got = cat.legal(q["prefix"]).tolist()
        assert got == q["legal"], (q, got)


def pin_slot_example_counts():
    """Padded-slot sidebar: beams A and B have 1 and 3 legal candidates."""
    g = json.load(open(os.path.join(GOLDEN, "slot_example.json")))
    cat = oracle.Catalog(np.array(g["catalog"], dtype=np.int32), g["V"])
    counts = [len(cat.legal(b)) for b in g["beams"]]
    assert counts == g["legal_counts"], counts
    assert max(counts) == g["slot_stride"]
    assert len(counts) * max(counts) == g["total_slots"]


def pin_index_brute_force():
    """Rows = lexicographic ranks of distinct prefixes; legal sets = next tokens (np.unique)."""
    for (V, L, N, seed) in [(6, 3, 120, 1), (16, 4, 700, 2), (256, 3, 3000, 3)]:
        sids = random_catalog(V, L, N, seed)
        cat = oracle.Catalog(sids, V)
        rng = np.random.default_rng(seed)
        for t in range(0, L + 1):
            uniq = np.unique(sids[:, :t], axis=0) if t > 0 else np.zeros((1, 0), np.int32)
            assert cat.count(t) == len(uniq), (t, cat.count(t), len(uniq))
            for i in rng.choice(len(uniq), size=min(40, len(uniq)), replace=False):
                assert cat.node(uniq[i]) == i
                if t < L:
                    mask = np.all(sids[:, :t] == uniq[i], axis=1)
                    want = sorted(set(sids[mask, t].tolist()))
                    assert cat.legal(uniq[i]).tolist() == want
        full = np.unique(sids, axis=0)
        for i in range(N):
            assert np.array_equal(sids[cat.input_row(i)], full[i])
        # a prefix not in the catalog has no legal tokens and no row
        absent = [p for p in ([a, b] for a in range(V) for b in range(V))
                  if not np.any(np.all(sids[:, :2] == p, axis=1))]
        if absent:
            assert cat.legal(absent[0]).size == 0 and cat.node(absent[0]) == -1


def pin_normalisation():
    """Legal-only log-softmax: sum exp = 1; one legal token -> 0 exactly; W = 0 -> -ln n."""
    cfg = small_cfg(V=16, d=12, L=3, N=200)
    sids = random_catalog(16, 3, 200, 11)
    cat = oracle.Catalog(sids, 16)
    W = weights_of(cfg)
    hid = hidden_fn(cfg)
    pre = np.unique(sids[:, :2], axis=0)[:10]
    cum = np.zeros(len(pre))
    r = cat.step(3, W[2], pre, cum, hid(0, 3, pre), K=1000)
    for k in range(len(pre)):
        lp = r.cand_logp[r.cand_beam == k]
        assert abs(math.fsum(np.exp(lp)) - 1.0) < 1e-12
        assert len(lp) == len(cat.legal(pre[k]))
    # a prefix with exactly one legal continuation
    single = np.array([[1, 2, 3], [1, 2, 5], [4, 0, 0]], np.int32)
    cs = oracle.Catalog(single, 8)
    Wr = np.random.default_rng(1).standard_normal((8, 4)).astype(np.float32)
    hr = np.random.default_rng(2).standard_normal((1, 4)).astype(np.float32)
    r1 = cs.step(3, Wr, np.array([[4, 0]], np.int32), np.array([-1.25]), hr, K=4)
    assert r1.cand_logp.tolist() == [0.0] and r1.cand_score.tolist() == [-1.25]
    # W = 0: every legal token gets log(1/n_b)
    Z = np.zeros((16, 12), np.float32)
    r0 = cat.step(3, Z, pre, cum, hid(0, 3, pre), K=1000)
    for k in range(len(pre)):
        n = len(cat.legal(pre[k]))
        lp = r0.cand_logp[r0.cand_beam == k]
        assert np.all(np.abs(lp + math.log(n)) <= 1e-15 * max(1.0, math.log(n)))


def _exhaustive(sids, V, W, hid, request):
    """Score every catalog item independently: sum over steps of its token's
    legal-only log-softmax (legal sets from Python sets, logsumexp from scipy)."""
    L = sids.shape[1]
    children = {}
    for s in sids.tolist():
        for t in range(L):
            children.setdefault(tuple(s[:t]), set()).add(s[t])
    scores = []
    for s in sids.tolist():
        tot = 0.0
        for t in range(L):
            pre = tuple(s[:t])
            legal = sorted(children[pre])
            h = hid(request, t + 1, np.array([s[:t]], np.int32).reshape(1, t))[0].astype(np.float64)
            z = W[t][legal].astype(np.float64) @ h
            tot += z[legal.index(s[t])] - logsumexp(z)
        scores.append(tot)
    return np.array(scores)


def pin_exhaustive_when_beam_covers_catalog():
    """K >= N: beam search keeps every prefix, so it equals exhaustive scoring."""
    for (V, L, N, d, seed) in [(5, 3, 40, 8, 21), (9, 4, 90, 6, 22)]:
        cfg = small_cfg(V=V, d=d, L=L, N=N, seed=seed)
        sids = random_catalog(V, L, N, seed)
        cat = oracle.Catalog(sids, V)
        W = weights_of(cfg)
        hid = hidden_fn(cfg)
        for request in (0, 3):
            res = oracle.decode(cat, W, hid, request, K=N)
            ex = _exhaustive(sids, V, W, hid, request)
            order = np.argsort(-ex, kind="stable")
            assert np.all(res.item >= 0)
            got_rows = [cat.input_row(int(i)) for i in res.item]
            assert got_rows == order.tolist()
            assert np.allclose(res.score, ex[order], rtol=0, atol=1e-12)
            assert np.array_equal(res.sid, sids[order])


def _numpy_beam_search(V, L, K, W, hid, request):
    """Textbook unconstrained beam search (every token legal everywhere)."""
    prefixes = np.zeros((1, 0), np.int32)
    cum = np.zeros(1)
    for t in range(1, L + 1):
        H = hid(request, t, prefixes).astype(np.float64)
        logits = H @ W[t - 1].astype(np.float64).T
        cand = cum[:, None] + log_softmax(logits, axis=1)
        flat = cand.reshape(-1)
        top = np.argsort(-flat, kind="stable")[:K]
        beam, tok = top // V, top % V
        prefixes = np.concatenate([prefixes[beam], tok[:, None].astype(np.int32)], axis=1)
        cum = flat[top]
    return prefixes, cum


def pin_full_product_equals_unconstrained():
    """A catalog of all V^L SIDs: filter-first = score-first = unconstrained search."""
    for (V, L, K, d, seed) in [(4, 3, 5, 8, 31), (3, 4, 7, 5, 32), (6, 2, 40, 4, 33)]:
        cfg = small_cfg(V=V, d=d, L=L, seed=seed)
        grid = np.stack(np.meshgrid(*[np.arange(V)] * L, indexing="ij"), -1).reshape(-1, L)
        cat = oracle.Catalog(grid.astype(np.int32), V)
        W = weights_of(cfg)
        hid = hidden_fn(cfg)
        for request, mode in [(0, "filter_first"), (1, "filter_first"), (0, "score_first"),
                              (1, "unconstrained")]:
            res = oracle.decode(cat, W, hid, request, K=K, mode=mode)
            want_sid, want_score = _numpy_beam_search(V, L, K, W, hid, request)
            n = len(want_score)
            assert np.array_equal(res.sid[:n], want_sid)
            assert np.allclose(res.score[:n], want_score, rtol=0, atol=1e-12)
            # item id of a full-product SID is its base-V value (lexicographic rank)
            vals = (want_sid * (V ** np.arange(L - 1, -1, -1))).sum(1)
            assert res.item[:n].tolist() == vals.tolist()


def pin_modes_against_scipy_log_softmax():
    """Score-first and unconstrained log-probs are scipy's log_softmax over the
    whole codebook (legal tokens only, resp. every token); filter-first is the
    same scores renormalised over the legal set."""
    V, d = 16, 12
    cfg = small_cfg(V=V, d=d, L=3, N=200)
    sids = random_catalog(V, 3, 200, 11)
    cat = oracle.Catalog(sids, V)
    W = weights_of(cfg)
    hid = hidden_fn(cfg)
    pre = np.unique(sids[:, :2], axis=0)[:10]
    cum = np.linspace(-3.0, 0.0, len(pre))
    cum[3] = -np.inf  # a dead beam contributes nothing in any mode
    H = hid(0, 3, pre)
    r = {m: cat.step(3, W[2], pre, cum, H, K=1000, mode=m) for m in oracle.MODES}
    for k in range(len(pre)):
        for m in oracle.MODES:
            if k == 3:
                assert not np.any(r[m].cand_beam == 3)
        if k == 3:
            continue
        legal = cat.legal(pre[k])
        full = log_softmax(W[2].astype(np.float64) @ H[k].astype(np.float64))
        sf, un, ff = (r[m] for m in ("score_first", "unconstrained", "filter_first"))
        sel = sf.cand_beam == k
        assert np.array_equal(sf.cand_token[sel], legal)
        assert np.allclose(sf.cand_logp[sel], full[legal], rtol=0, atol=1e-12)
        assert np.allclose(sf.cand_score[sel], cum[k] + full[legal], rtol=0, atol=1e-12)
        sel_u = un.cand_beam == k
        assert np.array_equal(un.cand_token[sel_u], np.arange(V))
        assert np.allclose(un.cand_logp[sel_u], full, rtol=0, atol=1e-12)
        assert abs(math.fsum(np.exp(un.cand_logp[sel_u])) - 1.0) < 1e-12
        # renormalising the score-first log-probs over the legal set gives filter-first
        lp_ff = ff.cand_logp[ff.cand_beam == k]
        assert np.allclose(lp_ff, full[legal] - logsumexp(full[legal]), rtol=0, atol=1e-12)
    # W = 0: every codebook token has probability 1/V before filtering
    Z = np.zeros((V, d), np.float32)
    for m in ("score_first", "unconstrained"):
        r0 = cat.step(3, Z, pre, np.zeros(len(pre)), H, K=1000, mode=m)
        assert np.all(np.abs(r0.cand_logp + math.log(V)) <= 1e-15 * math.log(V))
    # the selection is the best K of the candidates, in the fixed order
    for m in oracle.MODES:
        rr = cat.step(3, W[2], pre, cum, H, K=7, mode=m)
        order = sorted(range(len(rr.cand_score)),
                       key=lambda i: (-rr.cand_score[i], rr.cand_beam[i], rr.cand_token[i]))[:7]
        assert rr.sel_beam.tolist() == [int(rr.cand_beam[i]) for i in order]
        assert rr.sel_token.tolist() == [int(rr.cand_token[i]) for i in order]


def _exhaustive_all_v(codes, V, W, hid, request):
    """Score every code independently: sum over steps of its token's
    log-softmax over the whole codebook (scipy)."""
    L = codes.shape[1]
    out = []
    for s in codes.tolist():
        tot = 0.0
        for t in range(L):
            h = hid(request, t + 1, np.array([s[:t]], np.int32).reshape(1, t))[0].astype(np.float64)
            tot += log_softmax(W[t].astype(np.float64) @ h)[s[t]]
        out.append(tot)
    return np.array(out)


def pin_modes_exhaustive():
    """Beam covering everything: score-first ranks every catalog item by its
    summed all-codebook log-probs; unconstrained ranks every one of the V^L
    codes that way, real items keeping their id and other codes getting -1."""
    V, L, N, d, seed = 4, 3, 25, 6, 41
    cfg = small_cfg(V=V, d=d, L=L, N=N, seed=seed)
    sids = random_catalog(V, L, N, seed)
    cat = oracle.Catalog(sids, V)
    W = weights_of(cfg)
    hid = hidden_fn(cfg)
    members = {tuple(x): i for i, x in enumerate(sids.tolist())}
    for request in (0, 2):
        res = oracle.decode(cat, W, hid, request, K=N, mode="score_first")
        ex = _exhaustive_all_v(sids, V, W, hid, request)
        order = np.argsort(-ex, kind="stable")
        assert [cat.input_row(int(i)) for i in res.item] == order.tolist()
        assert np.allclose(res.score, ex[order], rtol=0, atol=1e-12)
        grid = np.stack(np.meshgrid(*[np.arange(V)] * L, indexing="ij"), -1).reshape(-1, L)
        res = oracle.decode(cat, W, hid, request, K=V ** L, mode="unconstrained")
        ex = _exhaustive_all_v(grid, V, W, hid, request)
        order = np.argsort(-ex, kind="stable")
        assert np.array_equal(res.sid, grid[order])
        assert np.allclose(res.score, ex[order], rtol=0, atol=1e-12)
        for it, sid in zip(res.item.tolist(), res.sid.tolist()):
            if tuple(sid) in members:
                assert it >= 0 and cat.input_row(it) == members[tuple(sid)]
            else:
                assert it == -1


def pin_unconstrained_leaves_the_catalog():
    """On a sparse catalog unconstrained search returns codes that are not
    items (id -1), while filter-first and score-first return only items."""
    cfg = small_cfg(V=32, d=16, L=3, N=300, K=16, seed=51)
    sids = random_catalog(32, 3, 300, 51)
    cat = oracle.Catalog(sids, 32)
    W = weights_of(cfg)
    hid = hidden_fn(cfg)
    members = set(map(tuple, sids.tolist()))
    un = oracle.decode(cat, W, hid, 0, K=16, mode="unconstrained")
    inval = [tuple(x) not in members for x in un.sid.tolist()]
    assert any(inval)
    assert all((it == -1) == bad for it, bad in zip(un.item.tolist(), inval))
    for m in ("filter_first", "score_first"):
        res = oracle.decode(cat, W, hid, 0, K=16, mode=m)
        assert np.all(res.item >= 0)
        assert all(tuple(x) in members for x in res.sid.tolist())


def pin_tie_break():
    """W = 0 on a full-product catalog: all candidates tie exactly, so the
    fixed order (beam ascending, then token ascending) decides everything."""
    V, L, K = 4, 3, 6
    grid = np.stack(np.meshgrid(*[np.arange(V)] * L, indexing="ij"), -1).reshape(-1, L)
    cat = oracle.Catalog(grid.astype(np.int32), V)
    W = [np.zeros((V, 3), np.float32)] * L
    hid = lambda r, t, p: np.ones((p.shape[0], 3), np.float32)  # noqa: E731
    res = oracle.decode(cat, W, hid, 0, K=K)
    want = [[0, 0, 0], [0, 0, 1], [0, 0, 2], [0, 0, 3], [0, 1, 0], [0, 1, 1]]
    assert res.sid.tolist() == want
    assert res.item.tolist() == [0, 1, 2, 3, 4, 5]
    s = 0.0
    for _ in range(L):
        s = s + (0.0 - (0.0 + math.log(V)))
    assert np.all(res.score == s)


def pin_results_are_catalog_items():
    """Every returned SID is a real item (set membership), its id maps back to it."""
    cfg = workload.CONFIGS["n1e4_v256"]
    sids = workload.catalog(cfg)
    cat = oracle.Catalog(sids, cfg.V)
    W = weights_of(cfg)
    hid = hidden_fn(cfg)
    members = set(map(tuple, sids.tolist()))
    for request in range(3):
        res = oracle.decode(cat, W, hid, request, K=cfg.K)
        assert np.all(res.item >= 0)
        assert len(set(res.item.tolist())) == cfg.K
        for i, s in zip(res.item, res.sid):
            assert tuple(s.tolist()) in members
            assert np.array_equal(sids[cat.input_row(int(i))], s)
        assert np.all(np.diff(res.score) <= 0)


def pin_fewer_candidates_than_beam():
    """Fewer than K candidates: all are kept; the rest of the output is empty."""
    sids = np.array([[0, 1], [0, 2], [3, 3]], np.int32)
    cat = oracle.Catalog(sids, 4)
    W = [np.eye(4, 2, dtype=np.float32)] * 2
    hid = lambda r, t, p: np.ones((p.shape[0], 2), np.float32)  # noqa: E731
    res = oracle.decode(cat, W, hid, 0, K=8)
    assert sorted(res.item[:3].tolist()) == [0, 1, 2]
    assert res.item[3:].tolist() == [-1] * 5
    assert np.all(np.isinf(res.score[3:]))


def pin_duplicate_and_range_rejected():
    for bad, msg in [(np.array([[1, 2], [1, 2]], np.int32), "duplicate"),
                     (np.array([[1, 9]], np.int32), "range")]:
        try:
            oracle.Catalog(bad, 4)
        except oracle.OracleError as e:
            assert msg in str(e)
        else:
            raise AssertionError("accepted " + msg)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


def main():
    failed = []
    for p in PINS:
        try:
            p()
        except Exception:  # noqa: BLE001 - report every failing pin
            failed.append(p.__name__)
            traceback.print_exc(limit=2)
    print("FAILED:", " ".join(failed) if failed else "none")
    return len(failed)


if __name__ == "__main__":
    sys.exit(main())
