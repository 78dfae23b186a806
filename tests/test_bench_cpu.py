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


def test_hbm_ceiling_keeps_the_fastest_variant_of_each_mix(monkeypatch):
    """The streaming-ceiling summary: per read:write mix, the variant with
    the highest rate, as a fraction of the 8 TB/s peak; the program's own
    lines are kept as the sweep."""
    import subprocess
    lines = [
        {"mix": "read", "reads": 1, "writes": 0, "unroll": 1, "nontemporal": False,
         "workgroups": 512, "loop": True, "ms_per_launch": 0.2, "GB/s": 5000.0},
        {"mix": "read", "reads": 1, "writes": 0, "unroll": 4, "nontemporal": True,
         "workgroups": 512, "loop": True, "ms_per_launch": 0.15, "GB/s": 7000.0},
        {"mix": "5:1", "reads": 5, "writes": 1, "unroll": 1, "nontemporal": True,
         "workgroups": 262144, "loop": False, "ms_per_launch": 1.0, "GB/s": 6000.0},
    ]

    class Done:
        returncode = 0
        stdout = "".join(json.dumps(l) + "\n" for l in lines)
        stderr = ""

    monkeypatch.setattr(os.path, "exists", lambda p: True)
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: Done())
    got = bench.hbm_ceiling()
    best = {b["mix"]: b for b in got["best"]}
    assert best["read"]["GB/s"] == 7000.0 and best["read"]["unroll"] == 4
    assert best["read"]["frac_of_hbm_peak"] == 0.875
    assert best["5:1"]["frac_of_hbm_peak"] == 0.75
    assert got["sweep"] == lines
