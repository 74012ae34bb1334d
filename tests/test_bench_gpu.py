"""The bench harness on the GPU: its JSON line carries the contract's keys, its timing is bracketed
around resident inputs that do not fit the last-level cache (achieved bandwidth stays below a plain
copy's), and the measured unit rates it reports are physically plausible."""
import json
import sys

import pytest

import bench

pytestmark = pytest.mark.gpu


def run_bench(capsys, monkeypatch, *args):
    """bench.main() in this process (no second process on the GPU), returning its last JSON line."""
    monkeypatch.setattr(sys, "argv", ["bench.py", *args])
    capsys.readouterr()
    bench.main()
    return json.loads(capsys.readouterr().out.strip().splitlines()[-1])


def test_bench_line_contract_and_cache_flush(capsys, monkeypatch):
    d = run_bench(capsys, monkeypatch, "--no-others", "--no-cpu-baseline", "--steps", "10", "--warmup", "3")
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 10 and d["warmup"] == 3 and d["config"]["workload"]
    rl = d["roofline"]
    assert rl["bound"] == "alu" and 0 < rl["frac"] <= 1 and abs(rl["achieved"] / rl["peak"] - rl["frac"]) < 1e-3
    mb = run_bench(capsys, monkeypatch, "--only", "ubench")
    # the headline's 1.1 GB of inputs per step: the achieved algorithmic bandwidth cannot exceed a plain HBM copy's
    assert d["hbm"]["achieved_GBs"] < mb["copy_GBs_read_plus_write"]
    # measured rates below the published unit peaks, exp at about half the FMA rate
    assert 0 < mb["fma_T_lane_ops_s"] <= mb["published"]["valu_T_lane_slots_s"] * 1.02
    assert 0.3 < mb["exp_T_lane_ops_s"] / mb["fma_T_lane_ops_s"] < 0.7
    assert 0 < mb["mfma_bf16_TFLOPs"] <= mb["published"]["mfma_bf16_TFLOPs"]
    assert 0 < mb["copy_GBs_read_plus_write"] <= mb["published"]["hbm_GBs"]
