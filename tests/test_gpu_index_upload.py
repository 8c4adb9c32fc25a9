"""Index rebuild pipeline on the GPU: every build / upload option leaves the
same bytes in HBM as the host tables (bit-exact), and the dense rank
directory equals the running popcount of the bitmap."""
import numpy as np
import pytest

import sid_constrained_beam_amd as zgr
import workload
from workload import CONFIGS

pytestmark = pytest.mark.gpu

CATALOGS = {
    "n1e4_v256": (CONFIGS["n1e4_v256"], None),
    "n1e8_v16384_small": (CONFIGS["n1e8_v16384"].scaled(N=400_000), None),
    "n1e6_v2048_all_dense": (CONFIGS["n1e6_v2048"].scaled(N=50_000), ["D", "D", "D"]),
    "n1e6_v2048_next_matrix": (CONFIGS["n1e6_v2048"].scaled(N=50_000), ["N", "N", "S"]),
}
OPTIONS = [
    dict(),                                          # defaults: automatic threads, staged
    dict(threads=3, upload="staged", staging_bytes=4096),  # many chunks, both buffers reused
    dict(threads=1, upload="direct"),
]

_sids = {}


def sids_of(name):
    if name not in _sids:
        cfg, _ = CATALOGS[name]
        _sids[name] = workload.catalog(cfg)
    return _sids[name]


def device_array(ptr, shape, dtype, stream):
    out = np.empty(shape, dtype)
    if out.size:
        zgr.copy_to_host(out, ptr, stream)
    return out


@pytest.mark.parametrize("opt", range(len(OPTIONS)))
@pytest.mark.parametrize("name", list(CATALOGS))
def test_device_tables_match_host(name, opt):
    import torch
    cfg, fmt = CATALOGS[name]
    o = OPTIONS[opt]
    print(f"[upload] {name} {o}", flush=True)
    sids = sids_of(name)
    stream = torch.cuda.current_stream().cuda_stream
    idx, rank = zgr.zgr_index_upload(sids, cfg.V, fmt if fmt else cfg.fmt, **o)
    ref, ref_rank = zgr.zgr_index_build_host(sids, cfg.V, fmt if fmt else cfg.fmt, threads=1)
    assert np.array_equal(rank, ref_rank)
    tm = zgr.zgr_index_times(idx)
    assert tm["upload"] == o.get("upload", "staged")
    total = 0
    words = (cfg.V + 31) // 32
    for t in range(1, cfg.L + 1):
        st = idx.stats(t)
        assert st == ref.stats(t)
        row_ptr, tok, bits = ref.host_table(t)
        d_rp, d_tok, d_bits, d_rank, d_next = zgr.zgr_index_device_table(idx, t)
        assert np.array_equal(device_array(d_rp, row_ptr.shape, np.int32, stream), row_ptr)
        total += row_ptr.nbytes
        if st["fmt"] == zgr.ZGR_FMT_SPARSE:
            assert d_bits == 0 and d_rank == 0 and d_next == 0
            assert np.array_equal(device_array(d_tok, tok.shape, np.uint16, stream), tok)
            total += tok.nbytes
        elif st["fmt"] == zgr.ZGR_FMT_DENSE_NEXT:
            assert d_tok == 0 and d_bits == 0 and d_rank == 0
            # cell (row, token) = the entry's next row, -1 where not legal
            want = np.full((st["rows"], cfg.V), -1, np.int32)
            rows_of = np.repeat(np.arange(st["rows"]), np.diff(row_ptr))
            want[rows_of, tok.astype(np.int64)] = np.arange(st["nnz"], dtype=np.int32)
            assert np.array_equal(device_array(d_next, want.shape, np.int32, stream), want)
            total += want.nbytes
        else:
            assert d_next == 0
            assert d_tok == 0
            assert np.array_equal(device_array(d_bits, bits.shape, np.uint32, stream), bits)
            pc = np.unpackbits(bits.view(np.uint8), axis=1, bitorder="little").reshape(
                bits.shape[0], words, 32).sum(2)
            want_rank = (np.cumsum(pc, axis=1) - pc).astype(np.uint16)
            assert np.array_equal(device_array(d_rank, bits.shape, np.uint16, stream), want_rank)
            total += bits.nbytes * 3 // 2
    assert tm["device_bytes"] == total


def test_rebuild_swaps_plans():
    """A rebuilt index (new catalog, non-default build options) serves new
    plans exactly like an index built with the defaults, and the old plan is
    rejected once its index is freed."""
    import torch
    import gpu_util as gu
    cfg = CONFIGS["n1e4_v256"]
    s = gu.Setup(cfg, with_oracle=False)
    old_plan = s.plan(force=["selective"] * cfg.L)
    sids2 = s.sids[::2].copy()  # half the catalog
    outs = []
    for o in (dict(threads=2, staging_bytes=8192), dict()):
        idx2, rank2 = zgr.zgr_index_upload(sids2, cfg.V, cfg.fmt, **o)
        plan2 = zgr.zgr_plan_warmup(idx2, s.W_dev, cfg.dtype, cfg.d, cfg.B, cfg.K, None, 0,
                                    ["selective"] * cfg.L)
        item = torch.empty(cfg.B * cfg.K, dtype=torch.int64, device="cuda")
        score = torch.empty(cfg.B * cfg.K, dtype=torch.float32, device="cuda")
        zgr.zgr_decode(plan2, s.hidden_source(), cfg.K, item, None, score)
        torch.cuda.synchronize()
        outs.append((item.cpu().numpy(), score.cpu().numpy()))
        got = outs[-1][0]
        assert (got >= 0).any() and got.max() < len(sids2)
        plan2.free()
        idx2.free()
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    item = torch.empty(cfg.B * cfg.K, dtype=torch.int64, device="cuda")
    s.index.free()
    with pytest.raises(zgr.ZgrError) as e:
        zgr.zgr_decode(old_plan, s.hidden_source(), cfg.K, item)
    assert e.value.status == zgr.ZGR_E_STATE
