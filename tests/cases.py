"""Workload cases shared by the GPU parity tests and the CPU test that checks
which full-projection kernels they reach (not collected by pytest).

PARITY_CASES / NEXT_CASES / MODE_CASES are reduced copies of the workloads
(same L, V, d, dtype and catalog law; fewer items, requests and beams) that
the oracle checks request by request.  FULLSIZE_FMT records the table format
of each step of the full-size workloads as the index builds them (AUTO picks
the smaller encoding; the 1e8-item catalog forces its formats); the full-size
GPU tests assert it, so the CPU coverage test can use it without building a
10^8-item index.  FULLSIZE_GEMM_CASES are the teacher-forced full-size steps
that run the full-projection kernels the benchmarks time at full size.
"""
from workload import CONFIGS

PARITY_CASES = {
    "n1e4_v256": CONFIGS["n1e4_v256"],
    "n1e6_v2048": CONFIGS["n1e6_v2048"],
    "n1e7_v2048_small": CONFIGS["n1e7_v2048"].scaled(N=300_000, B=4, K=32),
    "n1e7_v16384_small": CONFIGS["n1e7_v16384"].scaled(N=300_000, B=3, K=24),
    "n5e7_v1024_dense_small": CONFIGS["n5e7_v1024_dense"].scaled(N=2_000_000, B=3, K=40),
    "n1e8_v16384_small": CONFIGS["n1e8_v16384"].scaled(N=1_000_000, B=2, K=48),
}

NEXT_CASES = {
    "n1e6_v2048": ["N", "N", "S"],
    "n1e7_v2048_small": ["N", "N", "S", "S"],
    "n5e7_v1024_dense_small": ["N", "N", "S", "S"],
}

MODE_CASES = {
    "n1e4_v256": CONFIGS["n1e4_v256"],
    "n1e6_v2048_small": CONFIGS["n1e6_v2048"].scaled(N=100_000, B=4, K=32),
    "n1e7_v2048_small": CONFIGS["n1e7_v2048"].scaled(N=300_000, B=3, K=24),
    "n5e7_v1024_dense_small": CONFIGS["n5e7_v1024_dense"].scaled(N=500_000, B=2, K=40),
    # 16 beams x 16384 tokens per request: a part holds one beam, more
    # candidates than its key array, so keys are recomputed from the scores
    "n1e8_v16384_small": CONFIGS["n1e8_v16384"].scaled(N=200_000, B=2, K=16),
}

FULLSIZE = ["n1e6_v2048", "n1e7_v2048", "n1e7_v4096", "n1e7_v8192", "n1e7_v16384",
            "n5e7_v1024_dense", "n1e8_v16384"]

FULLSIZE_FMT = {
    "n1e6_v2048": "DDS",
    "n1e7_v2048": "DDSS",
    "n1e7_v4096": "DDSS",
    "n1e7_v8192": "DSSS",
    "n1e7_v16384": "DSSS",
    "n5e7_v1024_dense": "DDSS",
    "n1e8_v16384": "DDSS",
}

# Workloads whose dense steps the encoding comparison also times as a next-row matrix.
ENCODING_WORKLOADS = ["n1e6_v2048", "n1e7_v2048", "n1e7_v4096", "n5e7_v1024_dense", "n1e8_v16384"]

# Full-projection steps at full (or tile-reaching) size: (label, workload,
# config overrides, step, mode).  Each runs the GPU's own decode with the full
# projection forced at every step up to the listed one, every step checked
# against the oracle on sampled requests.
GEMM_CASES = [
    # 1e7 items, V = 2048: dense step 2 (legal rank), sparse step 3 (slot), modes at step 2
    ("v2048_t2_dense", "n1e7_v2048", {}, 2, "filter_first"),
    ("v2048_t3_slot", "n1e7_v2048", {}, 3, "filter_first"),
    ("v2048_t2_sf", "n1e7_v2048", {}, 2, "score_first"),
    ("v2048_t2_unc", "n1e7_v2048", {}, 2, "unconstrained"),
    # the same with the dense steps stored as the int32 next-row matrix
    ("v2048_t2_next", "n1e7_v2048", {"fmt": "NNSS"}, 2, "filter_first"),
    # 1e7 items, V = 4096: dense step 2 without word pruning (64 words per beam thread group)
    ("v4096_t2_dense", "n1e7_v4096", {}, 2, "filter_first"),
    # 1e7 items, V = 16384: sparse steps 2-3 by slot; score-first first step
    ("v16384_t3_slot", "n1e7_v16384", {}, 3, "filter_first"),
    ("v16384_t1_sf", "n1e7_v16384", {}, 1, "score_first"),
    # dense-early catalog (f16, batch 128)
    ("dense_t3_slot", "n5e7_v1024_dense", {}, 3, "filter_first"),
    ("dense_t2_sf", "n5e7_v1024_dense", {}, 2, "score_first"),
    ("dense_t2_unc", "n5e7_v1024_dense", {}, 2, "unconstrained"),
    ("dense_t2_next", "n5e7_v1024_dense", {"fmt": "NNSS"}, 2, "filter_first"),
    # 1e8 items (f32, d = 1024)
    ("n1e8_t3_slot", "n1e8_v16384", {}, 3, "filter_first"),
    ("n1e8_t2_sf", "n1e8_v16384", {}, 2, "score_first"),
    ("n1e8_t2_unc", "n1e8_v16384", {}, 2, "unconstrained"),
    ("n1e8_t2_next", "n1e8_v16384", {"N": 2_000_000, "B": 4, "K": 128, "fmt": "NNSS"}, 2,
     "filter_first"),
]


def gemm_case_config(name, over):
    """The workload config of a GEMM case (overrides applied; fmt as a list)."""
    kw = dict(over)
    if "fmt" in kw:
        kw["fmt"] = list(kw["fmt"])
    return CONFIGS[name].scaled(**kw) if kw else CONFIGS[name]
