"""GPU parity of big request parts: a dense-early step whose requests are
split into parts holding the merge-sized key array (one block per CU) because
small parts would take more than four rounds of blocks.  80 requests of 160
beams with about 800 legal tokens each (about 128K candidates per request)
reach that rule on a 256-CU MI355X.  Step 1 runs on the GPU, step 2 takes the
GPU's own beams; sampled requests of step 2 are checked against the oracle on
those inputs (protocol in gpu_util)."""
import numpy as np
import pytest

import gpu_util as gu
import sid_constrained_beam_amd as zgr
from workload import CONFIGS

pytestmark = pytest.mark.gpu

CFG = CONFIGS["n5e7_v1024_dense"].scaled(N=2_000_000, B=80, K=160)
SAMPLE = [0, 27, 53, 79]


def test_big_parts_step_parity():
    s = gu.Setup(CFG)
    cfg = s.cfg
    assert s.stats[1]["fmt"] == zgr.ZGR_FMT_DENSE
    tol = gu.TOL[cfg.dtype]
    B, K = cfg.B, cfg.K
    plan = s.plan(force=["full", "full", "selective", "selective"])
    requests = list(range(B))
    out1 = gu.run_gpu_step(s, plan, 1, np.zeros((B, 0), np.int32), np.zeros(B, np.float32), B, K,
                           requests, with_dbg=False)
    ok = out1["parent"] >= 0
    prefixes = np.full((B * K, 1), -1, np.int32)
    prefixes[ok, 0] = out1["token"][ok]
    cum = out1["cum_out"]
    legal = np.diff(s.index.host_table(2)[0])
    per_request = [int(legal[out1["row_out"][q * K:(q + 1) * K][ok[q * K:(q + 1) * K]]].sum())
                   for q in range(B)]
    print(f"[big parts] step-2 candidates per request: min {min(per_request)} max {max(per_request)}",
          flush=True)
    assert min(per_request) > 100_000
    out2 = gu.run_gpu_step(s, plan, 2, prefixes, cum, B, K, requests, with_dbg=SAMPLE)
    amb = gu.check_step(s, 2, prefixes, cum, out2, B, K, tol, requests=SAMPLE)
    print(f"[big parts] sampled requests {SAMPLE}: {amb} ambiguous request-steps", flush=True)
