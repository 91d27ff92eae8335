"""bench.py's host logic: the suite's record keys and the regression rule
against a baseline (a case regresses when its time exceeds the baseline's by
more than the threshold, 15% by default, as in TileKernels' benchmark plugin,
"TileKernels从入门到精通" ch.5 "铁血防线").  No GPU."""
import json

import bench


def rec(key, t):
    return {"key": key, "time_us": t}


def test_case_key_is_sorted_and_stable():
    k = bench.case_key("fused", {"hidden": 2048, "workload": "w", "group_size": 128})
    assert k == "swiglu_cast/fwd[group_size=128,hidden=2048,workload=w]"
    assert bench.case_key("topk", {"workload": "t", "seed": 0}) == "topk_gate/fwd[seed=0,workload=t]"


def test_regression_rule_at_the_threshold():
    base = [rec("a", 100.0), rec("b", 100.0), rec("c", 100.0), rec("gone", 5.0)]
    now = [rec("a", 114.9), rec("b", 115.0), rec("c", 115.1), rec("fresh", 1.0)]
    rows = {r[0]: r for r in bench.compare_records(now, base)}
    assert rows["a"][4] == "ok"
    assert rows["b"][4] == "ok"  # exactly +15% is not above the threshold
    assert rows["c"][4] == "REGRESSION"
    assert rows["fresh"][4] == "new" and rows["fresh"][2] is None
    assert rows["gone"][4] == "missing" and rows["gone"][1] is None
    assert abs(rows["c"][3] - 1.151) < 1e-12


def test_faster_is_never_a_regression_and_threshold_is_a_parameter():
    base = [rec("a", 100.0)]
    assert bench.compare_records([rec("a", 10.0)], base)[0][4] == "ok"
    assert bench.compare_records([rec("a", 106.0)], base, threshold=0.05)[0][4] == "REGRESSION"


def test_committed_baseline_reads_and_covers_every_suite_case():
    import os
    from moe_activation_bit_amd import workloads as wl
    if not os.path.exists(bench.BASELINES):
        return
    base = bench.read_records(bench.BASELINES)
    keys = {b["key"] for b in base}
    assert len(keys) == len(base), "duplicate keys"
    for b in base:
        assert b["time_us"] > 0 and b["operation"] == "fwd"
        json.dumps(b)
    names = {b["params"]["workload"] for b in base}
    assert set(wl.WORKLOADS) <= names
    assert len(base) == len(wl.WORKLOADS) + len(bench.SUITE_AUX)
