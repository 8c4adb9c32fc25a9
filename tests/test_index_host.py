"""Host-built filter index against the oracle's trie (bit-exact), no GPU."""
import json
import os

import numpy as np
import pytest

import oracle
import sid_constrained_beam_amd as zgr
import workload

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def row_prefixes(idx, L):
    """Prefix of every row of every table, rebuilt from the tables alone:
    entry e of row r in table t is row e of table t+1, with prefix(r) + tok[e]."""
    pre = [np.zeros((1, 0), np.int32)]
    for t in range(1, L + 1):
        row_ptr, tok, bits = idx.host_table(t)
        counts = np.diff(row_ptr)
        parent = np.repeat(np.arange(len(counts)), counts)
        nxt = np.concatenate([pre[-1][parent], tok.astype(np.int32)[:, None]], axis=1)
        pre.append(nxt)
    return pre


def check_against_oracle(sids, V, fmt=None, sample=None, seed=0, threads=0):
    N, L = sids.shape
    idx, rank = zgr.zgr_index_build_host(sids, V, fmt, threads=threads)
    cat = oracle.Catalog(sids, V)
    pre = row_prefixes(idx, L)
    rng = np.random.default_rng(seed)
    for t in range(1, L + 1):
        st = idx.stats(t)
        assert st["rows"] == cat.count(t - 1)
        assert st["nnz"] == cat.count(t)
        row_ptr, tok, bits = idx.host_table(t)
        assert row_ptr[0] == 0 and row_ptr[-1] == st["nnz"]
        counts = np.diff(row_ptr)
        assert counts.min() >= 1  # every row leads to at least one item
        assert st["max_legal"] == counts.max()
        if st["fmt"] in (zgr.ZGR_FMT_DENSE, zgr.ZGR_FMT_DENSE_NEXT):
            assert st["stride"] == V
            assert bits is not None and bits.shape == (st["rows"], (V + 31) // 32)
            # bitmap rows hold exactly the sorted legal tokens
            pc = np.unpackbits(bits.view(np.uint8), axis=1, bitorder="little")[:, :V].sum(1)
            assert np.array_equal(pc, counts)
        else:
            assert st["stride"] == counts.max() and bits is None
        rows = np.arange(st["rows"]) if sample is None else rng.choice(st["rows"], min(sample, st["rows"]), replace=False)
        for r in rows:
            p = pre[t - 1][r]
            assert cat.node(p) == r  # rows are lexicographic prefix ranks
            legal = tok[row_ptr[r]:row_ptr[r + 1]]
            assert np.array_equal(legal, cat.legal(p))
            if bits is not None:
                setb = np.nonzero(np.unpackbits(bits[r].view(np.uint8), bitorder="little"))[0]
                assert np.array_equal(setb, legal)
        # the next row of entry e is the rank of the extended prefix
        ents = np.arange(st["nnz"]) if sample is None else rng.choice(st["nnz"], min(sample, st["nnz"]), replace=False)
        for e in ents:
            assert cat.node(pre[t][e]) == e
    # item ids: position in the last table = oracle item id = lexicographic rank
    for i in (range(N) if sample is None else rng.choice(N, min(sample, N), replace=False)):
        assert cat.input_row(int(rank[i])) == i
        assert np.array_equal(pre[L][rank[i]], sids[i])
    return idx


def test_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    sids = np.array(g["catalog"], np.int32)
    for fmt in (None, ["D"] * 3, ["S"] * 3):
        idx = check_against_oracle(sids, g["V"], fmt)
        pre = row_prefixes(idx, 3)
        for q in g["queries"]:
            p = np.array(q["prefix"], np.int32)
            t = len(p) + 1
            match = [r for r in range(len(pre[t - 1])) if np.array_equal(pre[t - 1][r], p)]
            if not q["legal"]:
                assert not match
                continue
            row_ptr, tok, _ = idx.host_table(t)
            r = match[0]
            assert tok[row_ptr[r]:row_ptr[r + 1]].tolist() == q["legal"]


def test_slot_example_layout():
    g = json.load(open(os.path.join(GOLDEN, "slot_example.json")))
    idx, _ = zgr.zgr_index_build_host(np.array(g["catalog"], np.int32), g["V"], ["D", "S"])
    st = idx.stats(2)
    assert st["fmt"] == zgr.ZGR_FMT_SPARSE
    assert st["stride"] == g["slot_stride"]
    row_ptr, tok, _ = idx.host_table(2)
    assert np.diff(row_ptr).tolist() == g["legal_counts"]


@pytest.mark.parametrize("fmt", [None, "D", "S", "N"])
@pytest.mark.parametrize("V,L,N,seed", [(4, 3, 40, 1), (16, 4, 900, 2), (300, 2, 5000, 3), (2, 6, 50, 4)])
def test_random_catalogs(V, L, N, seed, fmt):
    rng = np.random.default_rng(seed)
    space = V ** L
    codes = rng.choice(space, size=min(N, space), replace=False)
    sids = np.stack([(codes // V ** (L - 1 - l)) % V for l in range(L)], 1).astype(np.int32)
    check_against_oracle(sids, V, None if fmt is None else [fmt] * L)


def test_format_policy_and_forced():
    cfg = workload.CONFIGS["n1e4_v256"]
    sids = workload.catalog(cfg)
    idx, _ = zgr.zgr_index_build_host(sids, cfg.V)
    for t in range(1, cfg.L + 1):
        st = idx.stats(t)
        dense_bytes = st["rows"] * ((cfg.V + 31) // 32) * 4
        sparse_bytes = st["nnz"] * 2
        want = zgr.ZGR_FMT_DENSE if dense_bytes < sparse_bytes else zgr.ZGR_FMT_SPARSE
        assert st["fmt"] == want
    d_idx, _ = zgr.zgr_index_build_host(sids, cfg.V, ["D"] * cfg.L)
    s_idx, _ = zgr.zgr_index_build_host(sids, cfg.V, ["S"] * cfg.L)
    for t in range(1, cfg.L + 1):
        a, b = d_idx.host_table(t), s_idx.host_table(t)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("name", ["n1e4_v256", "n1e6_v2048"])
def test_config_catalogs_sampled(name):
    cfg = workload.CONFIGS[name]
    sids = workload.catalog(cfg)
    check_against_oracle(sids, cfg.V, cfg.fmt, sample=None if cfg.N <= 10_000 else 300)


def _random_sids(V, L, N, seed):
    rng = np.random.default_rng(seed)
    codes = rng.choice(V ** L, size=min(N, V ** L), replace=False)
    return np.stack([(codes // V ** (L - 1 - l)) % V for l in range(L)], 1).astype(np.int32)


@pytest.mark.parametrize("V,L,N,seed", [(4, 3, 40, 1), (16, 4, 900, 2), (300, 2, 5000, 3), (2, 6, 50, 4)])
@pytest.mark.parametrize("threads", [2, 3, 7, 64])
def test_chunked_layout_matches_oracle(V, L, N, seed, threads):
    """Chunk boundaries fall inside rows at every table; the chunked count /
    offset / fill passes must still give the oracle's trie."""
    check_against_oracle(_random_sids(V, L, N, seed), V, threads=threads)


@pytest.mark.parametrize("fmt", [None, "D", "S", "N"])
def test_layout_independent_of_threads(fmt):
    cfg = workload.CONFIGS["n1e4_v256"]
    sids = workload.catalog(cfg)
    f = None if fmt is None else [fmt] * cfg.L
    ref, ref_rank = zgr.zgr_index_build_host(sids, cfg.V, f, threads=1)
    for T in (2, 5, 16, 64):
        idx, rank, tm = zgr.zgr_index_build_host(sids, cfg.V, f, threads=T, times=True)
        assert tm["threads"] == T
        assert all(tm[k] >= 0 for k in ("keys_ms", "sort_ms", "layout_ms", "encode_ms", "build_ms"))
        assert np.array_equal(rank, ref_rank)
        for t in range(1, cfg.L + 1):
            assert idx.stats(t) == ref.stats(t)
            for a, b in zip(idx.host_table(t), ref.host_table(t)):
                assert (a is None and b is None) or np.array_equal(a, b)


@pytest.mark.parametrize("threads", [1, 4, 9])
def test_chunked_errors(threads):
    # duplicates sit at every possible chunk boundary: report the first pair
    sids = _random_sids(16, 3, 400, 7)
    order = np.lexsort(sids.T[::-1])
    sids = sids[order]
    dup = np.concatenate([sids[:200], sids[199:]])  # sorted row 199 appears twice
    with pytest.raises(zgr.ZgrError) as e:
        zgr.zgr_index_build_host(dup, 16, threads=threads)
    assert e.value.status == zgr.ZGR_E_DUP_SID
    assert "rows 199 and 200" in e.value.detail
    bad = sids.copy()
    bad[321, 2] = 16
    with pytest.raises(zgr.ZgrError) as e:
        zgr.zgr_index_build_host(bad, 16, threads=threads)
    assert e.value.status == zgr.ZGR_E_TOKEN_RANGE and "row 321" in e.value.detail


@pytest.mark.parametrize("threads", [1, 3])
def test_presorted_catalog(threads):
    """A catalog given in SID order skips the sort; item ids are then the
    input rows.  Equal neighbours are still duplicates."""
    cfg = workload.CONFIGS["n1e4_v256"]
    sids = workload.catalog(cfg)
    srt = sids[np.lexsort(sids.T[::-1])]
    ref, _ = zgr.zgr_index_build_host(sids, cfg.V, threads=threads)
    idx, rank = zgr.zgr_index_build_host(srt, cfg.V, threads=threads)
    assert np.array_equal(rank, np.arange(len(srt)))
    for t in range(1, cfg.L + 1):
        for a, b in zip(idx.host_table(t), ref.host_table(t)):
            assert (a is None and b is None) or np.array_equal(a, b)
    dup = np.concatenate([srt[:50], srt[49:]])
    with pytest.raises(zgr.ZgrError) as e:
        zgr.zgr_index_build_host(dup, cfg.V, threads=threads)
    assert e.value.status == zgr.ZGR_E_DUP_SID and "rows 49 and 50" in e.value.detail


def test_encoding_bytes():
    """Device bytes per table: sparse 2 B per entry, bitmap 6 B per 32 tokens
    of a row (bits + rank directory), next-row matrix 4 B per (row, token);
    all plus the row offsets."""
    cfg = workload.CONFIGS["n1e4_v256"]
    sids = workload.catalog(cfg)
    words = (cfg.V + 31) // 32
    for f in ("D", "S", "N"):
        idx, _ = zgr.zgr_index_build_host(sids, cfg.V, [f] * cfg.L)
        for t in range(1, cfg.L + 1):
            st = idx.stats(t)
            rp = (st["rows"] + 1) * 4
            want = {"S": rp + st["nnz"] * 2, "D": rp + st["rows"] * words * 6,
                    "N": rp + st["rows"] * cfg.V * 4}[f]
            assert st["bytes"] == want
            assert st["stride"] == (st["max_legal"] if f == "S" else cfg.V)


def _long_row_sids(V, n1, per_row, seed):
    """Two-level catalog: n1 first tokens, each with per_row distinct second tokens."""
    rng = np.random.default_rng(seed)
    first = rng.choice(V, n1, replace=False)
    rows = [np.stack([np.full(per_row, f), rng.choice(V, per_row, replace=False)], 1) for f in first]
    return np.concatenate(rows).astype(np.int32)


@pytest.mark.parametrize("V,n1,per_row", [(4, 3, 3), (300, 20, 40), (1024, 16, 100), (5000, 8, 700),
                                          (65536, 2, 9000)])
def test_slice_directory(V, n1, per_row):
    """Slice directory of sparse rows: entry x < 7 counts the row's legal
    tokens (the oracle's trie children) below (x + 1) * ceil(V / 8); entry 7 is
    0; the tables themselves do not depend on it."""
    sids = _long_row_sids(V, n1, per_row, seed=V)
    cat = oracle.Catalog(sids, V)
    span = -(-V // 8)
    never, _ = zgr.zgr_index_build_host(sids, V, ["S", "S"], slices="never")
    idx, _ = zgr.zgr_index_build_host(sids, V, ["S", "S"], slices="always")
    pre = row_prefixes(idx, 2)
    for t in (1, 2):
        assert zgr.zgr_index_host_slices(never, t) is None and never.stats(t)["slice_dir"] == 0
        st = idx.stats(t)
        assert st["slice_dir"] == 1
        assert st["bytes"] == never.stats(t)["bytes"] + st["rows"] * 16
        a, b = idx.host_table(t), never.host_table(t)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        sd = zgr.zgr_index_host_slices(idx, t)
        assert sd.shape == (st["rows"], 8) and sd.dtype == np.uint16
        for r in range(st["rows"]):
            legal = np.asarray(cat.legal(pre[t - 1][r]), np.int64)
            want = [int((legal < (x + 1) * span).sum()) for x in range(7)] + [0]
            assert sd[r].tolist() == want


def test_slice_directory_auto_rule_and_errors():
    """AUTO: sparse tables with V >= 1024 and at least 32 legal tokens per row
    on average; dense tables never; an unknown value is an argument error."""
    seen = set()
    for V, n1, per_row in [(2048, 40, 40), (2048, 40, 20), (512, 10, 60), (4096, 64, 200)]:
        sids = _long_row_sids(V, n1, per_row, seed=n1 + per_row)
        idx, _ = zgr.zgr_index_build_host(sids, V)
        for t in (1, 2):
            st = idx.stats(t)
            want = st["fmt"] == zgr.ZGR_FMT_SPARSE and V >= 1024 and st["nnz"] >= 32 * st["rows"]
            assert st["slice_dir"] == int(want), (V, n1, per_row, t, st)
            assert (zgr.zgr_index_host_slices(idx, t) is not None) == want
            seen.add(want)
    assert seen == {True, False}
    sids = _long_row_sids(2048, 40, 40, seed=1)
    assert zgr.zgr_index_build_host(sids, 2048, ["D", "D"], slices="always")[0].stats(2)["slice_dir"] == 0
    with pytest.raises(zgr.ZgrError) as e:
        zgr.zgr_index_build_host(sids, 2048, slices=7)
    assert e.value.status == zgr.ZGR_E_ARG
