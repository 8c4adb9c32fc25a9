"""bench.py's accounting, on the host: a step's algorithmic work counts once
per step and decode however many launches the step took (a request split
over blocks launches its parts, then their merge), and the measured-traffic
field is filled only from counter summaries taken on the current kernel
source."""
import bench


def test_split_step_work_counts_once():
    steps = [{"t": 1}, {"t": 2}]

    def work(kernel, st):
        return "hbm", 100.0 * st["t"]

    n_dec = 5
    # step 1: one launch per decode (10 us each); step 2: two launches per
    # decode (parts, then merge: 30 us together)
    records = {"request": [(steps[0], 5, 5 * 0.010), (steps[1], 10, 5 * 0.030)],
               "gemm": [(steps[0], 0, 0.0), (steps[1], 0, 0.0)]}
    per = bench.kernel_classes(records, work, n_dec)
    assert set(per) == {"request"}  # a class with no launches is left out
    d = per["request"]
    assert d["launches"] == 15
    assert abs(d["ms"] - 0.2) < 1e-12
    assert d["units"] == n_dec * (100.0 + 200.0)  # not 5*100 + 10*200
    # the class's rate is its work over its time: 300 B per decode in 40 us
    rate = d["units"] / (d["ms"] * 1e-3)
    assert abs(rate - 300.0 / 40e-6) < 1e-6 * rate
    assert d["bound"] == "hbm"


def test_traffic_needs_matching_source(tmp_path, monkeypatch):
    sha = bench.source_sha()
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_sha", lambda: sha)
    path = prof / "k_request_step__wl__pmc.txt"
    assert bench.read_traffic("k_request_step", "wl") is None  # no summary
    path.write_text(f"# counters\nsource_sha: {sha}\nhbm_bytes_per_launch: 1234\n")
    assert bench.read_traffic("k_request_step", "wl") == 1234.0
    path.write_text("source_sha: 0000000000000000\nhbm_bytes_per_launch: 1234\n")
    assert bench.read_traffic("k_request_step", "wl") is None  # taken on other code
