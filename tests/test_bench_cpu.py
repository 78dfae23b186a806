"""CPU tests of bench.py's host logic: the measured-traffic figure is reported
only for the kernel source it was measured on, the benchmark refuses more
than one GPU, and each workload's ring form and dominant-launch roofline are
derived as documented.  No GPU is needed."""

import json
import os
import shutil

import pytest

import bench


def test_traffic_only_for_the_profiled_source(tmp_path, monkeypatch):
    got = bench.measured_traffic("gpt3_ffn_n8", "fused", "bidir")
    assert got is not None and got > 1e9
    # another permute form or ring direction has no counter run
    assert bench.measured_traffic("gpt3_ffn_n8", "stream", "bidir") is None
    assert bench.measured_traffic("gpt3_ffn_n8", "fused", "one-way") is None
    assert bench.measured_traffic("rs_n8", "fused", "one-way") is None
    # a changed GEMM source: the committed counters no longer describe it
    root = tmp_path / "repo"
    (root / "profiles").mkdir(parents=True)
    shutil.copy(os.path.join(bench.ROOT, "profiles", "traffic_gpt3_ffn_n8.json"), root / "profiles")
    t = json.load(open(root / "profiles" / "traffic_gpt3_ffn_n8.json"))
    src = root / t["kernel_source"]
    src.parent.mkdir(parents=True)
    data = open(os.path.join(bench.ROOT, t["kernel_source"]), "rb").read()
    src.write_bytes(data)
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.measured_traffic("gpt3_ffn_n8", "fused", "bidir") == got
    src.write_bytes(data + b"\n// changed\n")
    assert bench.measured_traffic("gpt3_ffn_n8", "fused", "bidir") is None


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    line = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_each_workload_runs_in_its_ring_form():
    from collective_overlap_amd import CCE_FLAG_BIDIRECTIONAL as B
    assert bench.preferred_bid("gpt3_ffn_n8") == B
    assert bench.preferred_bid("mlp2_n4") == B
    assert bench.preferred_bid("ag_fp32_n2") == B
    assert bench.preferred_bid("rs_n8") == 0            # faster one-way
    assert bench.preferred_bid("attn_outproj_n8") == 0  # no ring


def test_roofline_takes_the_dominant_launch_shape():
    """The dominant launch shape is the one with the most total time; its
    achieved rate is FLOP per launch over that shape's mean duration."""
    recs = ([{"kind": "gemm", "ms": 2.0, "flops": 2.0e12, "bytes": 0.0}] * 4 +
            [{"kind": "gemm", "ms": 1.0, "flops": 1.0e12, "bytes": 0.0}] * 3 +
            [{"kind": "epilogue", "ms": 0.2, "flops": 0.0, "bytes": 1e9}])
    roof, per_shape = bench.gemm_roofline(recs, "bf16", steps=1)
    assert roof["flops_per_launch"] == 2.0e12 and roof["launches"] == 4
    assert roof["avg_launch_ms"] == pytest.approx(2.0)
    assert roof["achieved"] == pytest.approx(1000.0, rel=1e-3)      # TFLOP/s
    assert roof["frac"] == pytest.approx(1000.0 / bench.PEAK_TFLOPS["bf16"], rel=1e-3)
    assert roof["bound"] == "mfma" and len(per_shape) == 2
