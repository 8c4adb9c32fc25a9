"""The seeded input generator: determinism, catalog laws and dtype rounding."""
import numpy as np
import pytest
import torch

import workload
from workload import CONFIGS


def _rows_unique(c):
    v = np.ascontiguousarray(c).view(np.dtype((np.void, c.dtype.itemsize * c.shape[1])))
    return len(np.unique(v)) == len(c)


def test_catalog_deterministic_and_thread_independent():
    cfg = CONFIGS["n1e6_v2048"].scaled(N=200_000)
    a = workload.catalog(cfg, n_threads=1)
    b = workload.catalog(cfg, n_threads=8)
    assert np.array_equal(a, b)
    c = workload.catalog(cfg.scaled(seed_cat=cfg.seed_cat + 1), n_threads=4)
    assert not np.array_equal(a, c)


@pytest.mark.parametrize("name", ["n1e4_v256", "n1e6_v2048"])
def test_catalog_unique_and_in_range(name):
    cfg = CONFIGS[name]
    c = workload.catalog(cfg)
    assert c.shape == (cfg.N, cfg.L)
    assert c.min() >= 0 and c.max() < cfg.V
    assert _rows_unique(c)


@pytest.mark.parametrize("level", [0, 1])
@pytest.mark.parametrize("s", [1.1, 1.3, 1.5])
def test_zipf_law(level, s):
    # A Zipf(s) level, placed under a single-token level and above uniform
    # levels so that no SID repeats and no redraw reshapes it: its sorted token
    # frequencies fall as rank^-s.
    kinds = [workload.UNIFORM_SUBSET] * level + [workload.ZIPF] + [workload.UNIFORM] * 2
    params = [1e-9] * level + [s] + [0.0] * 2
    cfg = CONFIGS["n1e6_v2048"].scaled(L=level + 3, V=16384, N=300_000, kinds=kinds,
                                       params=params)
    c = workload.catalog(cfg)
    assert _rows_unique(c)
    if level == 1:
        assert len(np.unique(c[:, 0])) == 1
    counts = np.sort(np.bincount(c[:, level], minlength=cfg.V))[::-1].astype(np.float64)
    r = np.arange(1, 101)
    slope = np.polyfit(np.log(r), np.log(counts[:100]), 1)[0]
    assert abs(slope + s) < 0.06, slope


def test_dense_early_profile():
    # Level 1 uniform over all V tokens; level 2 uniform over 90% of the codebook
    # under each level-1 prefix: every level-1 token is legal and no prefix has
    # more than round(0.9 V) level-2 children.
    cfg = CONFIGS["n5e7_v1024_dense"].scaled(N=5_000_000)
    c = workload.catalog(cfg)
    assert len(np.unique(c[:, 0])) == cfg.V
    pairs = np.unique(c[:, 0].astype(np.int64) * cfg.V + c[:, 1])
    per = np.bincount(pairs // cfg.V, minlength=cfg.V)
    m = round(0.9 * cfg.V)
    assert per.max() <= m
    assert per.mean() > 0.98 * m


@pytest.mark.parametrize("V", [2, 3, 256, 1000, 1024, 2048, 16384])
def test_keyed_permutation_is_bijection(V):
    for key in (1, 0xDEADBEEF):
        img = [workload.perm(key, V, x) for x in range(V)]
        assert sorted(img) == list(range(V))


def test_weights_and_hidden_laws():
    cfg = CONFIGS["n1e6_v2048"]
    bits, w = workload.weights(cfg, 2)
    assert bits.dtype == np.float32 and np.array_equal(bits, w)
    assert abs(w.mean()) < 3e-3
    assert abs(w.std() / cfg.w_std - 1) < 0.01
    bits2, w2 = workload.weights(cfg, 2)
    assert np.array_equal(w, w2)
    _, w3 = workload.weights(cfg, 3)
    assert not np.array_equal(w, w3)
    M = 4096
    req = np.arange(M) % 7
    prefix = np.stack([np.arange(M), np.arange(M) // 3], 1).astype(np.int32)
    _, h = workload.hidden(cfg, 3, req, prefix)
    assert abs(h.std() / cfg.h_std - 1) < 0.01
    # same (request, step, prefix) -> same vector; any field changed -> different
    _, h_again = workload.hidden(cfg, 3, req[:5], prefix[:5])
    assert np.array_equal(h[:5], h_again)
    _, h_t = workload.hidden(cfg, 2, req[:5], prefix[:5])
    assert not np.array_equal(h[:5], h_t)
    _, h_r = workload.hidden(cfg, 3, req[:5] + 1, prefix[:5])
    assert not np.array_equal(h[:5], h_r)
    # only the first t-1 prefix tokens matter
    p2 = prefix[:5].copy()
    p2 = np.concatenate([p2, np.full((5, 1), 9, np.int32)], 1)
    _, h_p = workload.hidden(cfg, 3, req[:5], p2)
    assert np.array_equal(h[:5], h_p)


def test_rounding_matches_torch_and_numpy():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 0.1,
        rng.standard_normal(2000).astype(np.float32) * 1e-6,   # f16 subnormal range
        np.array([0.0, -0.0, 1.0, -2.5, 65504.0, 6.1e-5, 5.96e-8, 2.98e-8, 1e-9], np.float32),
    ])
    # values exactly halfway between two bf16 / f16 neighbours
    base = rng.standard_normal(500).astype(np.float32)
    bb = base.view(np.uint32) & np.uint32(0xFFFF0000)
    ties_bf16 = (bb | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties_bf16])
    bits, f = workload.round_to("bf16", x)
    ref = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(bits, ref.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(f, ref.float().numpy())
    bits, f = workload.round_to("f16", x)
    ref16 = x.astype(np.float16)
    assert np.array_equal(bits, ref16.view(np.uint16))
    assert np.array_equal(f, ref16.astype(np.float32))
