"""zgr_step_noalloc (scratch in the library's static device array, no
allocation) against zgr_step with a plan forced to the same projection:
identical outputs, bit for bit (the same kernels run on the same inputs), on
two calls in a row, the second with a smaller input; the device flag stays
clear; a step whose scratch exceeds the array is rejected."""
import numpy as np
import pytest

import gpu_util as gu
import sid_constrained_beam_amd as zgr
import workload
from workload import CONFIGS

pytestmark = pytest.mark.gpu

CFG = CONFIGS["n1e6_v2048"].scaled(N=100_000, B=4, K=32)
# the same catalog with sparse steps 2-3 carrying a slice directory (the
# sliced projection's work lists live in the static array too)
CFG_SLICED = CFG.scaled(fmt=["D", "S", "S"])
_setup = {}


def setup(sliced=False):
    key = "sliced" if sliced else "s"
    if key not in _setup:
        _setup[key] = gu.Setup(CFG_SLICED, slices="always") if sliced else gu.Setup(CFG)
    return _setup[key]


def step_inputs(s, t, requests, k_in):
    """Teacher-forced inputs of step t: each request's oracle beams (at most k_in)."""
    import torch
    cfg = s.cfg
    M = len(requests) * k_in
    prefixes = np.zeros((M, max(t - 1, 1)), np.int32)
    cum = np.full(M, -np.inf, np.float32)
    rows = np.full(M, -1, np.int32)
    for qi, r in enumerate(requests):
        st = s.oracle_decode(r).steps[t - 1]
        n = min(k_in, len(st["cum"]))
        if t > 1:
            prefixes[qi * k_in: qi * k_in + n, : t - 1] = st["prefix"][:n]
        cum[qi * k_in: qi * k_in + n] = st["cum"][:n].astype(np.float32)
        for i in range(n):
            rows[qi * k_in + i] = s.cat.node(st["prefix"][i]) if t > 1 else 0
    req = np.repeat(np.asarray(requests, np.int64), k_in)
    bits, _ = workload.hidden(cfg, t, req, prefixes)
    return dict(hidden=gu.to_device_bits(bits, cfg.dtype), row=torch.from_numpy(rows).cuda(),
                cum=torch.from_numpy(cum).cuda(), M=M)


def outputs(B, K, M, S):
    import torch
    return dict(parent=torch.empty(B * K, dtype=torch.int32, device="cuda"),
                token=torch.empty(B * K, dtype=torch.int32, device="cuda"),
                row=torch.empty(B * K, dtype=torch.int32, device="cuda"),
                cum=torch.empty(B * K, dtype=torch.float32, device="cuda"),
                dbg=torch.empty(M * S, dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("sliced", [False, True])
@pytest.mark.parametrize("proj", ["selective", "full"])
def test_noalloc_step_matches_plan_step(proj, sliced):
    import torch
    s = setup(sliced)
    if sliced:
        assert s.stats[1]["slice_dir"] == 1 and s.stats[2]["slice_dir"] == 1
    cfg = s.cfg
    K = cfg.K
    # call 1: step 2, four requests of K beams; call 2: step 3, two requests of K / 2 beams
    for t, requests, k_in in ((2, [0, 1, 2, 3], K), (3, [1, 3], K // 2)):
        B = len(requests)
        print(f"[noalloc] {proj} sliced={sliced} step {t} B={B} k_in={k_in}", flush=True)
        inp = step_inputs(s, t, requests, k_in)
        S = s.stats[t - 1]["stride"]
        plan = zgr.zgr_plan_warmup(s.index, s.W_dev, cfg.dtype, cfg.d, B, K, None, 0, [proj] * cfg.L)
        ref = outputs(B, K, inp["M"], S)
        zgr.zgr_step(plan, t, inp["hidden"], inp["row"], inp["cum"], k_in, ref["parent"], ref["token"],
                     ref["row"], ref["cum"], ref["dbg"])
        zgr.zgr_plan_status(plan)
        got = outputs(B, K, inp["M"], S)
        err = torch.full((1,), 7, dtype=torch.int32, device="cuda")
        zgr.zgr_step_noalloc(s.index, s.W_dev[t - 1], cfg.dtype, cfg.d, B, K, t, proj, inp["hidden"],
                             inp["row"], inp["cum"], k_in, got["parent"], got["token"], got["row"],
                             got["cum"], got["dbg"], err)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(ref[k], got[k]), (proj, sliced, t, k)
        assert int(err.item()) == 0
        assert int((got["parent"] >= 0).sum().item()) > 0
        plan.free()


def test_noalloc_rejects_oversized_step():
    s = setup()
    cfg = s.cfg
    import torch
    # 4096 requests of K beams need about 4096 * 32 * 2048 * 4 bytes of scores: beyond 64 MiB
    B, t = 4096, 2
    x = torch.empty(1, dtype=torch.float32, device="cuda")
    xi = torch.empty(1, dtype=torch.int32, device="cuda")
    with pytest.raises(zgr.ZgrError) as e:
        zgr.zgr_step_noalloc(s.index, s.W_dev[t - 1], cfg.dtype, cfg.d, B, cfg.K, t, "selective", x, xi,
                             x, cfg.K, xi, xi, xi, x)
    assert e.value.status == zgr.ZGR_E_SHAPE
